"""GPU parity of the HIP encoder and decode attention against the fp64 oracle.

Decode is fed index caches built by the oracle (or drawn by the synthetic
generator), never by the GPU encoder, so the two kernels are tested apart;
the end-to-end tests then chain GPU encode -> GPU decode.
Bars: indices bit-exact except inside the oracle's near-tie band (counted and
printed); outputs within 2e-3 max-abs (+ half a bf16 ulp for bf16 output);
lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (GpuLayer, bound, check_codes, compare, dims_for, io_tensor, make_cache_from_data,
                      ref_decode, to_dev, x_tensor)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401


def _note(msg):
    print(msg, flush=True)


def _encode_gpu(cfg, layer, xk, xv, slots, num_pages, n_blocks=None, first_block=0):
    nb = cfg.n_blocks if n_blocks is None else n_blocks
    cache = torch.zeros((nb, num_pages, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8,
                        device="cuda")
    lv.loopvq_encode(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), layer.cb, layer.hsq,
                     to_dev(np.asarray(slots, np.int32)), cache, first_block=first_block, n_blocks=nb,
                     block_stride_bytes=cache[0].numel())
    torch.cuda.synchronize()
    return cache.cpu().numpy()


# ---------------------------------------------------------------- slices
def test_codebook_slices_and_hsq():
    cfg = synth.config_by_name("deeploop")
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    layer = GpuLayer(cfg, cb, 16)
    s = layer.slices.cpu().numpy()
    hsq = layer.hsq.cpu().numpy()
    for t in (0, 5, 31):
        beta, m = divmod(t, cfg.Tc)
        for h in (0, 15):
            for kv in range(2):
                want = oracle.loop_slice(cb[beta, h, kv].astype(np.float64), cfg.Tc, cfg.c, m)
                np.testing.assert_array_equal(s[t, h, kv].astype(np.float64), want)
    want = 0.5 * (cb.astype(np.float64) ** 2).sum(-1)
    np.testing.assert_allclose(hsq, want, rtol=2 ** -24, atol=0)


# ---------------------------------------------------------------- tiny config
def test_tiny_encode_and_decode():
    cfg = synth.config_by_name("tiny")
    N = cfg.seq_len
    xk, xv = synth.make_kv(cfg, N)
    cb = synth.make_codebooks(cfg)
    lens = np.array([N])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, N, cfg.page_size)
    layer = GpuLayer(cfg, cb, N)
    got = _encode_gpu(cfg, layer, xk, xv, slots, npg)
    ties, bad = check_codes(cfg, got, xk, xv, cb, slots, method="direct")
    _note(f"tiny encode: near-ties {ties}, mismatches outside the band {bad}")
    assert bad == 0
    ref_cache, _, _ = oracle.build_index_cache(xk, xv, cb, cfg.Tc, cfg.c, cfg.bits, slots, npg, cfg.page_size)
    if ties == 0:
        np.testing.assert_array_equal(got, ref_cache)
    for t in range(1, cfg.T + 1):
        q = synth.make_queries(cfg, 1, t=t)
        beta = (t - 1) // cfg.Tc
        o, lse = layer.decode(t, q, ref_cache[beta], bt, lens)
        ref = ref_decode(cfg, t, q, ref_cache[beta], bt, lens, cb)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"tiny decode t={t}: max err {err:.2e}")
        assert ratio <= 1.0
        # end to end: the GPU encoder's cache into the GPU decoder
        o2, _ = layer.decode(t, q, got[beta], bt, lens)
        ref2 = ref_decode(cfg, t, q, got[beta], bt, lens, cb) if ties else ref
        assert compare(cfg, o2, None, ref2, lens)[1] <= 1.0


# ---------------------------------------------------------------- 1.4B layer shape, ragged and small
def test_layer_ragged_encode_decode():
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([1000, 1, 257, 64])
    ntot = int(lens.sum())
    xk, xv = synth.make_kv(cfg, ntot)
    cb = synth.make_codebooks(cfg)
    bt, npg = synth.make_block_table(cfg, lens)
    slots = np.concatenate([synth.slot_mapping_for(bt, b, int(n), cfg.page_size) for b, n in enumerate(lens)])
    layer = GpuLayer(cfg, cb, int(lens.max()))
    got = _encode_gpu(cfg, layer, xk, xv, slots, npg)
    ties, bad = check_codes(cfg, got, xk, xv, cb, slots, heads=[0, 7, 15])
    _note(f"layer encode: near-ties {ties}, mismatches outside the band {bad}")
    assert bad == 0
    ref_cache, _ = make_cache_from_data(cfg, xk, xv, cb, lens, bt, npg)
    for t in range(1, cfg.T + 1):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, ref_cache[0], bt, lens)
        ref = ref_decode(cfg, t, q, ref_cache[0], bt, lens, cb)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"layer decode t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def _random_cache_case(cfg, lens, seed, n_blocks=1):
    bt, npg = synth.make_block_table(cfg, lens)
    caches = [synth.random_index_cache(cfg, npg, seed + i) for i in range(n_blocks)]
    return bt, npg, caches


# ---------------------------------------------------------------- full sizes, sampled
@pytest.mark.parametrize("name,t_list,requests,heads", [
    ("layer1p4b", (1, 4), (0, 3, 7), None),
    ("longctx32k", (1, 2, 3, 4), (0, 9, 15), (0, 6, 15)),
])
def test_full_size_decode_sampled(name, t_list, requests, heads):
    cfg = synth.config_by_name(name)
    lens = synth.make_seq_lens(cfg)
    bt, npg, caches = _random_cache_case(cfg, lens, 77)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    cache_d = to_dev(caches[0])
    for t in t_list:
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, cache_d, bt, lens)
        ref = ref_decode(cfg, t, q, caches[0], bt, lens, cb, requests=requests, heads=heads)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"{name} decode t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_gpu_encoded_32k_cache_sampled():
    # the 32K batch as bench.py builds and times it: keys and values drawn on
    # the GPU (torch's generator), coded by the GPU encoder, decoded by the GPU.
    # For sampled (request, head) streams the oracle encodes the same values
    # itself (the GPU's codes must be its codes outside the near-tie band) and
    # decodes its own cache; the GPU's output on the GPU-coded cache must match
    # that within the output bound.
    cfg = synth.config_by_name("longctx32k")
    lens = synth.make_seq_lens(cfg)
    bt, npg = synth.make_block_table(cfg, lens)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    cache = torch.zeros((npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    sample = {0: (3, 12), 9: (0,)}
    host_kv = {}
    for b, n in enumerate(lens):
        xk, xv = synth.make_kv_torch(cfg, int(n), cfg.index * 1000 + b)
        slots = to_dev(synth.slot_mapping_for(bt, b, int(n), cfg.page_size))
        lv.loopvq_encode(layer.dims, xk, xv, layer.cb, layer.hsq, slots, cache)
        for h in sample.get(b, ()):
            host_kv[(b, h)] = (xk[:, :, h:h + 1].float().cpu().numpy(), xv[:, :, h:h + 1].float().cpu().numpy())
        del xk, xv
    torch.cuda.synchronize()
    got_cache = cache.cpu().numpy()
    t = 3
    q = synth.make_queries(cfg, len(lens), t=t)
    o, lse = layer.decode(t, q, cache, bt, lens)
    grp = cfg.H_q // cfg.H_kv
    for (b, h), (xk, xv) in host_kv.items():
        n = int(lens[b])
        slots = synth.slot_mapping_for(bt, b, n, cfg.page_size)
        ref_cache, ties, results = oracle.build_index_cache(xk, xv, cb[:, h:h + 1], cfg.Tc, cfg.c, cfg.bits, slots,
                                                            npg, cfg.page_size, method="gemm")
        P = cfg.page_size
        for kv, x in enumerate((xk, xv)):
            rows = got_cache[slots // P, h, kv, slots % P, :]
            codes = oracle.slots_to_groups(oracle.unpack_rows(rows, cfg.bits, cfg.n_groups)).reshape(-1)
            z = oracle.coupled_vectors(x[:, :, 0, :], cfg.Tc, cfg.c, 0).reshape(-1, cfg.G)
            assert oracle.accepts(z, cb[0, h, kv].astype(np.float64), results[(0, 0, kv)], codes).all()
        o_ref, lse_ref = oracle.decode_attention(np.asarray(q[b], np.float64)[h * grp:(h + 1) * grp], ref_cache[0],
                                                 bt[b], n, cb[0, h:h + 1], t, cfg.Tc, cfg.c, cfg.bits, cfg.base)
        err = np.abs(o[b, h * grp:(h + 1) * grp] - o_ref)
        ratio = float((err / bound(o_ref, cfg.io_dtype)).max())
        _note(f"GPU-coded 32K cache, request {b} head {h}: near-ties {ties}, max err {err.max():.2e} "
              f"(bound ratio {ratio:.2f})")
        assert ratio <= 1.0
        assert np.allclose(lse[b, h * grp:(h + 1) * grp], lse_ref, rtol=0, atol=1e-4)


def test_full_size_decode_16_token_pages():
    # 16-token pages at the 32K batch: the shared-rows split plan fills each
    # chunk's page list exactly (2048-position chunks of 128 pages)
    cfg = synth.config_by_name("longctx32k").replace(page_size=16)
    lens = synth.make_seq_lens(cfg)
    bt, npg, caches = _random_cache_case(cfg, lens, 78)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=2)
    o, lse = layer.decode(2, q, to_dev(caches[0]), bt, lens)
    ref = ref_decode(cfg, 2, q, caches[0], bt, lens, cb, requests=(0, 15), heads=(0, 15))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"longctx32k, 16-token pages: max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


def test_gqa_ragged_decode():
    cfg = synth.config_by_name("gqa_ragged")
    # small ragged batch, every pair checked
    lens = np.array([1500, 1, 0, 700, 64, 2049])
    bt, npg, caches = _random_cache_case(cfg, lens, 5)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, 16384)
    for t in (1, 3):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, caches[0], bt, lens)
        ref = ref_decode(cfg, t, q, caches[0], bt, lens, cb)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"gqa small decode t={t}: max err {err:.2e}")
        assert ratio <= 1.0
    # full batch of 64 ragged requests, sampled
    lens = synth.make_seq_lens(cfg)
    bt, npg, caches = _random_cache_case(cfg, lens, 6)
    q = synth.make_queries(cfg, len(lens), t=2)
    o, lse = layer.decode(2, q, caches[0], bt, lens)
    ref = ref_decode(cfg, 2, q, caches[0], bt, lens, cb, requests=(0, 31, 63), heads=(0, 7))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"gqa full decode: max err {err:.2e}")
    assert ratio <= 1.0


def test_deep_loop_blocks():
    cfg = synth.config_by_name("deeploop")
    cb = synth.make_codebooks(cfg)
    # encode one 4096-token chunk of all 8 blocks; check two heads fully
    n = cfg.encode_tokens
    xk, xv = synth.make_kv(cfg, n)
    lens = np.array([n])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n, cfg.page_size)
    layer = GpuLayer(cfg, cb, cfg.seq_len)
    got = _encode_gpu(cfg, layer, xk, xv, slots, npg)
    ties, bad = check_codes(cfg, got, xk, xv, cb, slots, heads=[0, 9])
    _note(f"deeploop encode: near-ties {ties}, mismatches outside the band {bad}")
    assert bad == 0
    # decode at N = 16384, B = 4 from random caches of every block
    lens = synth.make_seq_lens(cfg)
    bt, npg, caches = _random_cache_case(cfg, lens, 11, n_blocks=cfg.n_blocks)
    for t in (1, 6, 17, 32):
        beta = (t - 1) // cfg.Tc
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, caches[beta], bt, lens)
        ref = ref_decode(cfg, t, q, caches[beta], bt, lens, cb, requests=(0, 3), heads=(2, 13))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"deeploop decode t={t}: max err {err:.2e}")
        assert ratio <= 1.0


# ---------------------------------------------------------------- invariants and edge cases
def test_split_invariance_determinism_and_edges():
    cfg = synth.config_by_name("layer1p4b").replace(io_dtype="f32")
    lens = np.array([3000, 0, 1, 129])
    bt, npg, caches = _random_cache_case(cfg, lens, 3)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, 40000)
    q = synth.make_queries(cfg, len(lens), t=2)
    o1, l1 = layer.decode(2, q, caches[0], bt, lens)
    o1b, l1b = layer.decode(2, q, caches[0], bt, lens)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b), "run-to-run determinism"
    # a larger max_seq_len changes the split plan; the softmax merge must not care
    bt_wide = np.zeros((len(lens), 40000 // 64 + 1), dtype=np.int32)
    bt_wide[:, :bt.shape[1]] = bt
    o2, l2 = layer.decode(2, q, caches[0], bt_wide, lens, max_seq_len=40000)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=2e-6)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=2e-6)   # equal -inf entries compare equal
    ref = ref_decode(cfg, 2, q, caches[0], bt, lens, cb)
    err, ratio = compare(cfg, o1, l1, ref, lens)
    _note(f"fp32-output decode: max err {err:.2e}")
    assert err < 1e-4
    # explicit softmax scale and no lse output
    o3, l3 = layer.decode(2, q, caches[0], bt, lens, sm_scale=0.05, want_lse=False)
    assert l3 is None
    ref3 = ref_decode(cfg, 2, q, caches[0], bt, lens, cb, sm_scale=0.05)
    assert compare(cfg, o3, None, ref3, lens)[0] < 1e-4
    # empty batch entries only
    z = np.zeros(2, dtype=np.int32)
    oz, lz = layer.decode(2, q[:2], caches[0], bt[:2], z, max_seq_len=0)
    assert np.all(oz == 0) and np.all(np.isneginf(lz))


@pytest.mark.parametrize("page_size", [8, 256, 1024])   # 1024: the largest page size the boundary takes
def test_page_sizes(page_size):
    cfg = synth.config_by_name("layer1p4b").replace(page_size=page_size, H_kv=4, H_q=4)
    lens = np.array([1500, 37])                # with 1024-token pages: one full page and a partial one
    bt, npg, caches = _random_cache_case(cfg, lens, 21)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    layer = GpuLayer(cfg, cb, 1500)
    q = synth.make_queries(cfg, 2, t=3)
    o, lse = layer.decode(3, q, caches[0], bt, lens)
    ref = ref_decode(cfg, 3, q, caches[0], bt, lens, cb)
    assert compare(cfg, o, lse, ref, lens)[1] <= 1.0


@pytest.mark.parametrize("over,lens", [
    # fp32 queries and outputs on each K-side form: the duo's pairs share keys
    # (GQA), or not, with whole-step pages and with 8-token pages
    (dict(H_kv=4, H_q=8), [700, 1, 0, 300]),
    (dict(H_kv=4, H_q=8, page_size=8), [600, 37]),
    (dict(H_kv=4, H_q=4, page_size=8), [600, 37]),
])
def test_fp32_io_paths(over, lens):
    cfg = synth.config_by_name("layer1p4b").replace(io_dtype="f32", **over)
    lens = np.array(lens)
    bt, npg, caches = _random_cache_case(cfg, lens, 31)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=4)
    _note(f"fp32 io decode {over} lens={list(lens)}")
    o, lse = layer.decode(4, q, caches[0], bt, lens)
    ref = ref_decode(cfg, 4, q, caches[0], bt, lens, cb)
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"fp32 io decode {over}: max err {err:.2e}")
    assert err < 1e-4


def test_two_channels_eight_steps_64_groups_per_token():
    # c = 2 channels over Tc = 8 loop steps (G = 16): 64 groups per token, so
    # a 32-vector encoder unit is half a token (the one-token instance with
    # per-unit row slots) and an index row holds 64 codes
    cfg = synth.config_by_name("layer1p4b").replace(c=2, Tc=8, T=8, rhos=(0.8,) * 7, H_kv=2, H_q=2)
    lens = np.array([300, 45])
    ntot = int(lens.sum())
    xk, xv = synth.make_kv(cfg, ntot, seed=5)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    bt, npg = synth.make_block_table(cfg, lens)
    slots = np.concatenate([synth.slot_mapping_for(bt, b, int(n), cfg.page_size) for b, n in enumerate(lens)])
    layer = GpuLayer(cfg, cb, int(lens.max()))
    got = _encode_gpu(cfg, layer, xk, xv, slots, npg)
    ties, bad = check_codes(cfg, got, xk, xv, cb, slots)
    _note(f"c=2 Tc=8 encode: near-ties {ties}, mismatches outside the band {bad}")
    assert bad == 0
    ref_cache, _ = make_cache_from_data(cfg, xk, xv, cb, lens, bt, npg)
    for t in (1, 5, 8):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, ref_cache[0], bt, lens)
        ref = ref_decode(cfg, t, q, ref_cache[0], bt, lens, cb)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"c=2 Tc=8 decode t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_per_step_coding_runs_on_the_same_kernels():
    # Tc = 1: every loop step has its own codebook and its own cache block
    cfg = synth.config_by_name("layer1p4b").replace(Tc=1, c=8, H_kv=2, H_q=2,
                                                    x_dtype="f32")
    # G = c * Tc = 8 with fp32 input (split into two fp16 terms)
    n = 300
    xk, xv = synth.make_kv(cfg, n)
    cb = synth.make_codebooks(cfg.replace(n_calib=200))
    lens = np.array([n])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n, cfg.page_size)
    layer = GpuLayer(cfg, cb, n)
    got = _encode_gpu(cfg, layer, xk, xv, slots, npg)
    ties, bad = check_codes(cfg, got, xk, xv, cb, slots)
    _note(f"per-step encode: near-ties {ties}, mismatches {bad}")
    assert bad == 0
    ref_cache, _ = make_cache_from_data(cfg, xk, xv, cb, lens, bt, npg)
    for t in (1, 4):
        q = synth.make_queries(cfg, 1, t=t)
        o, lse = layer.decode(t, q, ref_cache[t - 1], bt, lens)
        ref = ref_decode(cfg, t, q, ref_cache[t - 1], bt, lens, cb)
        assert compare(cfg, o, lse, ref, lens)[1] <= 1.0


def test_combine_ignores_stale_partials():
    # The combine loads a whole batch of chunk partials before it knows the
    # request's own chunk count, then drops the chunks past that count.  With
    # every workspace byte set to 0xff beforehand (NaN in each partial the
    # split does not write), the short requests' outputs must still match the
    # oracle, and an empty request must give zeros and lse = -inf.
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=4, H_q=4)
    lens = np.array([4096, 3, 0, 130, 2047, 64])
    bt, npg, caches = _random_cache_case(cfg, lens, 17)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    layer = GpuLayer(cfg, cb, int(lens.max()))
    B, msl = len(lens), int(lens.max())
    q = synth.make_queries(cfg, B, t=2)
    ws = torch.full((lv.loopvq_decode_workspace_bytes(layer.dims, B, msl),), 0xff, dtype=torch.uint8,
                    device="cuda")
    out = torch.empty((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, cfg.H_q), dtype=torch.float32, device="cuda")
    bt_d, seq_d = to_dev(bt.astype(np.int32)), to_dev(lens.astype(np.int32))
    lv.loopvq_decode_split(layer.dims, 2, io_tensor(cfg, q), to_dev(caches[0]), layer.slices, layer.rope, bt_d,
                           seq_d, msl, ws, max_pos=layer.max_pos)
    lv.loopvq_decode_combine(layer.dims, B, seq_d, msl, ws, out, lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), "a stale partial reached the output"
    assert np.all(o[2] == 0) and np.all(np.isneginf(l[2]))
    ref = ref_decode(cfg, 2, q, caches[0], bt, lens, cb)
    err, ratio = compare(cfg, o, l, ref, lens)
    _note(f"combine over stale partials: max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0
