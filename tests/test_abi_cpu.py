"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects every invalid argument before launching anything, and
its host RoPE table matches the oracle's fp64 cos/sin."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import decode_attention_loopvq_amd as lv
    if not os.path.exists(lv.LIB_PATH):
        from decode_attention_loopvq_amd import build
        build.build(verbose=False)
    return lv


def _dims(lv, **kw):
    base = dict(D=128, c=4, Tc=4, T=4, bits=8, H_kv=16, H_q=16, page_size=64, x_dtype="bf16", io_dtype="bf16")
    base.update(kw)
    return lv.loopvq_dims.make(**base)


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first


def test_header_symbols_exported(L):
    hdr = open(os.path.join(ROOT, "include", "loopvq.h")).read()
    declared = set(re.findall(r"\b(loopvq_[a-z_]+)\s*\(", hdr))
    assert declared == set(L.EXPORTED)
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(L.loopvq_status_string(s), str) and L.loopvq_status_string(s)


def test_row_bytes(L):
    assert L.loopvq_row_bytes(_dims(L)) == 32
    assert L.loopvq_row_bytes(_dims(L, c=8)) == 16
    assert L.loopvq_row_bytes(_dims(L, D=64, c=2, bits=4, x_dtype="f32")) == 16


@pytest.mark.parametrize("kw,status", [
    (dict(c=3), -1),                       # D % c
    (dict(Tc=3), -1),                      # Tc does not divide T
    (dict(H_q=20), -1),                    # H_q % H_kv
    (dict(page_size=48), -1),              # not a power of two
    (dict(page_size=4), -1),
    (dict(bits=5), -2),                    # K = 32: valid pair, not compiled
    (dict(D=96), -2),
    (dict(c=16, Tc=2), -2),
    (dict(c=2, Tc=4), -2),                 # G = 8 needs fp32 encoder input
    (dict(x_dtype=7), -1),
    # one index-cache page (H_kv*2*P*R bytes) must stay below 4 GiB
    (dict(H_kv=32768, H_q=32768, page_size=1024, c=2, x_dtype="f32"), -2),
])
def test_invalid_dims(L, kw, status):
    assert L.lib().loopvq_row_bytes(ctypes.byref(_dims(L, **kw))) == status


def test_large_page_accepted(L):
    # 1024 heads x 2 x 1024 positions x 64-byte rows: 128 MiB pages are fine
    d = _dims(L, H_kv=1024, H_q=1024, page_size=1024, c=2, x_dtype="f32")
    assert L.lib().loopvq_row_bytes(ctypes.byref(d)) == 64
    # the same shape with 32768 heads only fails on the page size
    d = _dims(L, H_kv=32768, H_q=32768, page_size=512, c=2, x_dtype="f32")
    assert L.lib().loopvq_row_bytes(ctypes.byref(d)) == 64


def test_per_group_dims(L):
    lib = L.lib()
    assert lib.loopvq_row_bytes(ctypes.byref(_dims(L, per_group=1))) == 32
    assert lib.loopvq_row_bytes(ctypes.byref(_dims(L, per_group=2))) == -1
    assert lib.loopvq_row_bytes(ctypes.byref(_dims(L, per_group=1, bits=4))) == -2   # 8-bit codes only
    assert L.loopvq_dims.make(D=128, c=4, Tc=4, T=4, bits=8, H_kv=1, H_q=1, page_size=64,
                              per_group=1).n_codebooks == 32


def test_bad_K_and_null_dims(L):
    d = _dims(L)
    d.K = 128
    assert L.lib().loopvq_row_bytes(ctypes.byref(d)) == -1
    assert L.lib().loopvq_row_bytes(None) == -1


def test_decode_validation_before_launch(L):
    lib = L.lib()
    d = _dims(L)
    ws = L.loopvq_decode_workspace_bytes(d, 4, 1000)
    assert ws > 0
    def call(t=1, B=4, max_pos=1000, max_pages=16, max_seq_len=1000, ws_bytes=ws, ptrs=FAKE, work=FAKE):
        return lib.loopvq_decode_attn(ctypes.byref(d), t, B, ptrs, ptrs, ptrs, ptrs, max_pos, ptrs, max_pages,
                                      ptrs, max_seq_len, 0.0, ptrs, None, work, ws_bytes, None)
    assert call(t=0) == -1
    assert call(t=5) == -1
    assert call(B=-1) == -1
    assert call(max_pos=999) == -1            # positions beyond the RoPE table
    assert call(max_pages=15) == -1           # block table too short for max_seq_len
    assert call(ptrs=None) == -1
    assert call(ws_bytes=ws - 1) == -3
    assert call(work=ctypes.c_void_p((1 << 20) + 8)) == -1   # workspace not 256-byte aligned
    assert call(B=0) == 0                     # nothing to do
    d4 = _dims(L, D=64, c=8, bits=4, Tc=2, T=4)
    assert lib.loopvq_decode_attn(ctypes.byref(d4), 1, 1, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 1, FAKE, 10, 0.0,
                                  FAKE, None, FAKE, 1 << 20, None) == -2


def test_window_decode_validation_before_launch(L):
    lib = L.lib()
    d = _dims(L)
    ws = L.loopvq_decode_workspace_bytes(d, 4, 1000)
    good = L.loopvq_bf16_window(1 << 20, 1 << 20, 4, 1 << 20, 1 << 20)
    def call(t=1, B=4, max_pos=1000, max_pages=16, max_seq_len=1000, ws_bytes=ws, win=good, ptrs=FAKE):
        w = None if win is None else ctypes.byref(win)
        return lib.loopvq_decode_attn_window(ctypes.byref(d), t, B, ptrs, ptrs, ptrs, ptrs, max_pos, ptrs,
                                             max_pages, ptrs, max_seq_len, w, 0.0, ptrs, None, FAKE, ws_bytes,
                                             None)
    assert call(win=None) == -1
    assert call(t=0) == -1
    assert call(max_pos=999) == -1
    assert call(max_pages=15) == -1
    assert call(ptrs=None) == -1
    assert call(ws_bytes=ws - 1) == -3
    for bad in (L.loopvq_bf16_window(None, 1 << 20, 4, 1 << 20, 1 << 20),
                L.loopvq_bf16_window(1 << 20, None, 4, 1 << 20, 1 << 20),
                L.loopvq_bf16_window(1 << 20, 1 << 20, 0, 1 << 20, 1 << 20),
                L.loopvq_bf16_window(1 << 20, 1 << 20, 4, None, 1 << 20),
                L.loopvq_bf16_window(1 << 20, 1 << 20, 4, 1 << 20, None),
                L.loopvq_bf16_window((1 << 20) + 2, 1 << 20, 4, 1 << 20, 1 << 20)):   # pages not 16-byte aligned
        assert call(win=bad) == -1
    assert call(B=0) == 0
    # the window's partials need a larger workspace than the coded pass alone
    assert ws > 0


def test_encode_validation_before_launch(L):
    lib = L.lib()
    d = _dims(L)
    def call(n_tok=10, first=0, nb=1, stride=0, ptr=FAKE, ties=None):
        return lib.loopvq_encode(ctypes.byref(d), n_tok, first, nb, ptr, ptr, ptr, ptr, ptr, ptr, stride, ties,
                                 None)
    assert call(n_tok=-1) == -1
    assert call(first=1) == -1
    assert call(nb=0) == -1
    assert call(nb=2) == -1
    assert call(ptr=None) == -1
    assert call(n_tok=0, ptr=None) == 0
    assert call(n_tok=0, ptr=None, ties=FAKE) == 0                    # the counter is optional and untouched
    assert call(ties=ctypes.c_void_p((1 << 20) + 2)) == -1            # near-tie counter not 4-byte aligned
    assert call(n_tok=-1, ties=FAKE) == -1
    d8 = _dims(L, T=8)
    assert lib.loopvq_encode(ctypes.byref(d8), 4, 0, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, None) == -1
    d_small = _dims(L, D=64, c=8, bits=4)  # 8 groups per token: 4-bit rows need a multiple of 16
    assert lib.loopvq_encode(ctypes.byref(d_small), 4, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None,
                             None) == -2


def test_encode_pages_validation_before_launch(L):
    lib = L.lib()
    d = _dims(L)
    def call(n_tok=10, first=0, nb=1, pages=FAKE, stride=1 << 20, src=FAKE, ptr=FAKE, dims=d):
        return lib.loopvq_encode_pages(ctypes.byref(dims), n_tok, first, nb, pages, stride, src, ptr, ptr, ptr, ptr,
                                       0, None)
    assert call(pages=None) == -1
    assert call(src=None) == -1
    assert call(pages=ctypes.c_void_p((1 << 20) + 8)) == -1      # pool not 16-byte aligned
    assert call(stride=0) == -1                                  # Tc = 4 steps need a step stride
    assert call(stride=12) == -1                                 # stride not a multiple of 8
    assert call(n_tok=-1) == -1
    assert call(nb=2) == -1
    assert call(ptr=None) == -1
    assert call(dims=_dims(L, x_dtype="f32")) == -2              # the window pages are bf16
    assert call(n_tok=0, pages=None, src=None) == 0


def test_tasq_validation_before_launch(L):
    lib = L.lib()
    d = _dims(L)
    F = 1 << 20
    good = L.loopvq_tasq(F, F, F, 4096)
    ws_enc = L.loopvq_encode_tasq_workspace_bytes(d, 10, 1)
    assert ws_enc == ((4 * 10 * 16 * 128 * 4 + 255) // 256) * 256
    def enc(n_tok=10, first=0, nb=1, tq=good, ptr=FAKE, ws=ws_enc, work=FAKE, dims=d):
        t = None if tq is None else ctypes.byref(tq)
        return lib.loopvq_encode_tasq(ctypes.byref(dims), n_tok, first, nb, ptr, ptr, t, ptr, ptr, ptr, ptr, 0,
                                      work, ws, None)
    assert enc(tq=None) == -1
    for bad in (L.loopvq_tasq(None, F, F, 4096), L.loopvq_tasq(F, None, F, 4096), L.loopvq_tasq(F, F, None, 4096),
                L.loopvq_tasq(F, F, F, 0), L.loopvq_tasq(F, F, F, -1),
                L.loopvq_tasq(F, F, F + 2, 4096), L.loopvq_tasq(F, F, F, 4097)):   # sigma alignment / odd stride
        assert enc(tq=bad) == -1
    assert enc(ws=ws_enc - 1) == -3
    assert enc(work=ctypes.c_void_p(F + 16)) == -1            # workspace not 256-byte aligned
    assert enc(ptr=ctypes.c_void_p(F + 8)) == -1              # keys not 16-byte aligned
    assert enc(tq=L.loopvq_tasq(F + 4, F, F, 4096)) == -1     # weights not 16-byte aligned
    assert enc(ptr=None) == -1
    assert enc(n_tok=-1) == -1
    assert enc(nb=2) == -1
    assert enc(dims=_dims(L, bits=4)) == -2                   # TaSQ keys: 8-bit codes only
    assert enc(dims=_dims(L, per_group=1)) == -2
    assert enc(dims=_dims(L, H_kv=128, H_q=128)) == -2       # the transform's LDS row: H_kv*D <= 10922
    assert enc(n_tok=0, ptr=None) == 0
    ws = L.loopvq_decode_workspace_bytes(d, 4, 1000)
    def dec(t=1, B=4, tq=good, ptr=FAKE, ws_bytes=ws, dims=d, win=None):
        q = None if tq is None else ctypes.byref(tq)
        w = None if win is None else ctypes.byref(win)
        return lib.loopvq_decode_attn_tasq(ctypes.byref(dims), t, B, ptr, ptr, ptr, ptr, 1000, ptr, 16, ptr, 1000,
                                           q, w, 0.0, ptr, None, FAKE, ws_bytes, None)
    assert dec(tq=None) == -1
    assert dec(t=0) == -1
    assert dec(ptr=None) == -1
    assert dec(ws_bytes=ws - 1) == -3
    assert dec(dims=_dims(L, bits=4)) == -2
    assert dec(win=L.loopvq_bf16_window(None, F, 4, F, F)) == -1
    assert dec(B=0) == 0


def test_kmeans_validation_before_launch(L):
    lib = L.lib()
    d = _dims(L)
    ws = L.loopvq_kmeans_workspace_bytes(d, 1)
    assert ws == ((2 * 16 * (256 * 16 + 256 + 2) * 8 + 255) // 256) * 256
    def call(n_tok=10, first=0, nb=1, ptr=FAKE, cb=FAKE, out=FAKE, work=FAKE, ws_bytes=ws, dims=d, stride=0):
        return lib.loopvq_kmeans_update(ctypes.byref(dims), n_tok, first, nb, ptr, ptr, ptr, ptr, stride, cb, out,
                                        None, work, ws_bytes, None)
    assert call(n_tok=-1) == -1
    assert call(nb=0) == -1 and call(first=1) == -1
    assert call(ptr=None) == -1
    assert call(cb=None) == -1 and call(out=None) == -1 and call(work=None) == -1
    assert call(work=ctypes.c_void_p((1 << 20) + 64)) == -1
    assert call(ws_bytes=ws - 1) == -3
    assert call(dims=_dims(L, per_group=1)) == -2
    d8 = _dims(L, T=8)
    assert call(dims=d8, nb=2) == -1                    # two blocks need a block stride
    # c = 16 at Tc = 1 (G channels of one step): encoder and k-means only
    d16 = _dims(L, c=16, Tc=1)
    assert L.loopvq_row_bytes(d16) == 8
    assert lib.loopvq_decode_attn(ctypes.byref(d16), 1, 1, FAKE, FAKE, FAKE, FAKE, 10, FAKE, 1, FAKE, 10, 0.0,
                                  FAKE, None, FAKE, 1 << 20, None) == -2
    assert lib.loopvq_row_bytes(ctypes.byref(_dims(L, c=16, Tc=2))) == -2


def test_slices_validation(L):
    lib = L.lib()
    assert lib.loopvq_build_codebook_slices(ctypes.byref(_dims(L)), None, FAKE, None, None) == -1
    assert lib.loopvq_build_codebook_slices(None, FAKE, FAKE, None, None) == -1


def test_workspace_bytes_monotone(L):
    d = _dims(L)
    a = L.loopvq_decode_workspace_bytes(d, 16, 4096)
    b = L.loopvq_decode_workspace_bytes(d, 16, 32768)
    assert 0 < a <= b and a % 256 == 0
    assert L.loopvq_decode_workspace_bytes(d, -1, 10) == 0


def test_split_plan_chunks_with_16_token_pages(L):
    # 16 requests x 32768 tokens, 16 heads: 2048-position chunks (16 per request)
    # whether pages hold 64 or 16 positions; with 16-position pages each chunk's
    # page list (128 entries per stream) is then exactly full.  The workspace
    # holds one (o, lse) partial per chunk, D + 1 floats per (head, pair, chunk)
    for P in (64, 16):
        d = _dims(L, page_size=P)
        assert L.loopvq_decode_workspace_bytes(d, 16, 32768) == \
            L.loopvq_decode_workspace_bytes(_dims(L), 16, 32768)
    n_part = 16 * 16 * 16
    parts = ((n_part * 128 * 4 + 255) // 256 * 256) + ((n_part * 4 + 255) // 256 * 256)
    window = ((16 * 16 * 128 * 4 + 255) // 256 * 256) + ((16 * 16 * 4 + 255) // 256 * 256)
    assert L.loopvq_decode_workspace_bytes(_dims(L, page_size=16), 16, 32768) == parts + window


@pytest.mark.parametrize("D,max_pos", [(64, 40001), (128, 40000)])
def test_rope_table_matches_oracle(L, D, max_pos):
    t = L.loopvq_rope_table(max_pos, D).numpy()
    padded = (max_pos + 15) // 16 * 16
    assert t.size == padded * D == L.lib().loopvq_rope_table_floats(max_pos, D)
    # [position group][chunk j][quarter i][position in group][cos f, sin f, cos f+1, sin f+1]
    t = t.reshape(padded // 4, D // 16, 4, 4, 4).transpose(0, 3, 1, 2, 4).reshape(padded, D // 16, 4, 4)
    cs, sn = oracle.rope_cos_sin(np.arange(padded), D, 10000.0)
    j = np.arange(D // 16)[None, :, None]
    i = np.arange(4)[None, None, :]
    for e in range(2):
        f = (i * (D // 8) + 2 * j + e)[0]
        for got, want in ((t[:, :, :, 2 * e], cs[:, f]), (t[:, :, :, 2 * e + 1], sn[:, f])):
            # fp64 values rounded once to fp32: within half an fp32 ulp, plus
            # 1e-10 for the last-bit difference of theta between libm and NumPy
            bound = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) / 2 + 1e-10
            assert np.all(np.abs(got.astype(np.float64) - want) <= bound)


def test_rope_table_validation(L):
    lib = L.lib()
    assert lib.loopvq_rope_table(-1, 128, 1e4, FAKE) == -1
    assert lib.loopvq_rope_table(4, 96, 1e4, FAKE) == -1
    assert lib.loopvq_rope_table(4, 128, 1e4, None) == -1
    assert lib.loopvq_rope_table(0, 128, 1e4, None) == 0


def test_noalloc_decode_rejects_batches_beyond_its_scratch(L):
    # checked on the host before the scratch address is looked up or anything
    # is launched, so it needs no GPU
    lib = L.lib()
    d = _dims(L)
    def call(B, n, ptr=FAKE):
        return lib.loopvq_decode_attn_noalloc(ctypes.byref(d), 1, B, ptr, ptr, ptr, ptr, n, ptr, 1 << 12, ptr, n,
                                              0.0, ptr, ptr, None)
    cap = 8 << 20
    assert L.loopvq_decode_workspace_bytes(d, 16, 32768) <= cap          # the 32K batch fits
    assert L.loopvq_decode_workspace_bytes(d, 256, 65536) > cap
    assert call(256, 65536) == -5
    assert "scratch" in L.loopvq_status_string(-5)
    assert call(0, 64, ptr=None) == 0                                     # empty batch: nothing to do
    assert call(-1, 64) == -1


def test_binding_takes_device_tensors_only(L):
    # the binding has no host path: host tensors are refused before any call
    import torch
    d = _dims(L)
    B, N = 1, 64
    q = torch.zeros((B, 16, 128), dtype=torch.bfloat16)
    cache = torch.zeros((1, 16, 2, 64, 32), dtype=torch.uint8)
    slices = torch.zeros((4, 16, 2, 256, 4), dtype=torch.float16)
    rope = torch.zeros(64 * 128, dtype=torch.float32)
    bt = torch.zeros((B, 1), dtype=torch.int32)
    sl = torch.full((B,), N, dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        L.loopvq_decode_attn(d, 1, q, cache, slices, rope, bt, sl, N, max_pos=64)
    ws = torch.zeros(L.loopvq_decode_workspace_bytes(d, B, N), dtype=torch.uint8)
    out = torch.zeros((B, 16, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        L.loopvq_decode_split(d, 1, q, cache, slices, rope, bt, sl, N, ws, max_pos=64)
    with pytest.raises(ValueError, match="device tensor"):
        L.loopvq_decode_combine(d, B, sl, N, ws, out)


def test_binding_checks_shapes_before_the_call(L, monkeypatch):
    # shape checks of the decode wrappers, with the device-placement check
    # relaxed so that host tensors reach them; each raises before the library
    # is asked to launch anything
    import torch
    from decode_attention_loopvq_amd import _lib

    def need_anywhere(t, dtype, name, device=True):
        if t.dtype != dtype:
            raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    monkeypatch.setattr(_lib, "_need", need_anywhere)
    d = _dims(L)
    B, N = 2, 64
    q = torch.zeros((B, 16, 128), dtype=torch.bfloat16)
    cache = torch.zeros((1, 16, 2, 64, 32), dtype=torch.uint8)
    slices = torch.zeros((4, 16, 2, 256, 4), dtype=torch.float16)
    rope = torch.zeros(int(L.lib().loopvq_rope_table_floats(64, 128)), dtype=torch.float32)
    bt = torch.zeros((B, 1), dtype=torch.int32)
    sl = torch.full((B,), N, dtype=torch.int32)
    ws = torch.zeros(L.loopvq_decode_workspace_bytes(d, B, N), dtype=torch.uint8)
    out = torch.zeros((B, 16, 128), dtype=torch.bfloat16)
    split = lambda **kw: L.loopvq_decode_split(d, 1, kw.get("q", q), cache, slices, kw.get("rope", rope),
                                               kw.get("bt", bt), kw.get("sl", sl), N, ws,
                                               max_pos=kw.get("max_pos", 64))
    with pytest.raises(ValueError, match="q must be"):
        split(q=torch.zeros((B, 8, 128), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="q: expected"):
        split(q=torch.zeros((B, 16, 128), dtype=torch.float32))
    with pytest.raises(ValueError, match="seq_lens"):
        split(sl=torch.full((1,), N, dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table"):
        split(bt=torch.zeros((1, 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="rope_table holds"):
        split(max_pos=65)
    with pytest.raises(ValueError, match="rope_table holds"):
        split(rope=rope[:-1])
    with pytest.raises(ValueError, match="out must be"):
        L.loopvq_decode_combine(d, B, sl, N, ws, torch.zeros((B, 16, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse must be"):
        L.loopvq_decode_combine(d, B, sl, N, ws, out, torch.zeros((B,), dtype=torch.float32))
    with pytest.raises(ValueError, match="seq_lens"):
        L.loopvq_decode_combine(d, B + 1, sl, N, ws, torch.zeros((B + 1, 16, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        L.loopvq_decode_attn(d, 1, q, cache, slices, rope, bt, sl, N, out=out[:1], max_pos=64)


def test_missing_library_fails_loudly(L, monkeypatch, tmp_path):
    from decode_attention_loopvq_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libloopvq.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="is missing"):
        _lib.lib()
