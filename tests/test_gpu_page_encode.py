"""GPU parity of decode-time page encoding (loopvq_encode_pages) and of
block-by-block prefill encoding, and an end-to-end run in which the bf16
window moves on and its oldest page is coded every 8 tokens.

Bars: codes bit-exact against the dense encoder on the same values, and
against the oracle except inside its near-tie band; decode outputs within
2e-3 (+ half a bf16 ulp for bf16 output), lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuLayer, check_codes, compare, ref_decode_window, to_dev, x_tensor

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401


def _note(msg):
    print(msg, flush=True)


def _pools_from_dense(xk, xv, n_pages, src_slot):
    """bf16 page pools [steps][n_pages][H][2][8][D] holding token j at page src_slot[j] // 8."""
    T, n, H, D = xk.shape
    pools = np.zeros((T, n_pages, H, 2, 8, D), np.float32)
    pg, sl = src_slot // 8, src_slot % 8
    pools[:, pg, :, 0, sl, :] = np.transpose(xk, (1, 0, 2, 3))
    pools[:, pg, :, 1, sl, :] = np.transpose(xv, (1, 0, 2, 3))
    return pools


@pytest.mark.parametrize("name,over,n_tok", [
    ("layer1p4b", dict(), 200),
    ("deeploop", dict(), 64),
    ("gqa_ragged", dict(), 72),                                  # 16 groups per token
    ("layer1p4b", dict(c=2, Tc=8, T=8, rhos=(0.8,) * 7, H_kv=2, H_q=2), 120),   # 64 groups per token
])
def test_encode_pages_equals_dense_encode(name, over, n_tok):
    cfg = synth.config_by_name(name).replace(**over)
    xk, xv = synth.make_kv(cfg, n_tok, seed=cfg.index + 70)
    cb = synth.make_codebooks(cfg.replace(n_calib=400))
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n_tok, cfg.page_size)
    layer = GpuLayer(cfg, cb, 16)
    rng = np.random.default_rng(71)
    n_pages = (n_tok + 7) // 8 + 3
    src_slot = rng.permutation(n_pages * 8)[:n_tok].astype(np.int32)   # scattered page slots
    pools = to_dev(_pools_from_dense(xk, xv, n_pages, src_slot), torch.bfloat16)
    shape = (cfg.n_blocks, npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes)
    dense = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    paged = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    slots_d = to_dev(slots.astype(np.int32))
    lv.loopvq_encode(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), layer.cb, layer.hsq, slots_d, dense,
                     n_blocks=cfg.n_blocks, block_stride_bytes=dense[0].numel())
    lv.loopvq_encode_pages(layer.dims, pools, to_dev(src_slot), layer.cb, layer.hsq, slots_d, paged,
                           n_blocks=cfg.n_blocks, block_stride_bytes=paged[0].numel())
    torch.cuda.synchronize()
    got = paged.cpu().numpy()
    assert np.array_equal(got, dense.cpu().numpy()), "paged and dense inputs must give the same codes"
    ties, bad = check_codes(cfg, got, xk, xv, cb, slots, heads=[0, cfg.H_kv - 1])
    _note(f"{name} {over} page encode: near-ties {ties}, mismatches outside the band {bad}")
    assert bad == 0


def test_block_by_block_prefill_equals_one_call():
    # prefill holds each block's loop steps until the block's last step, then
    # codes that block alone; the result equals coding all blocks at once
    cfg = synth.config_by_name("deeploop")
    n = 96
    xk, xv = synth.make_kv(cfg, n, seed=80)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    lens = np.array([n])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = to_dev(synth.slot_mapping_for(bt, 0, n, cfg.page_size).astype(np.int32))
    layer = GpuLayer(cfg, cb, 16)
    shape = (cfg.n_blocks, npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes)
    whole = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    parts = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    xk_d, xv_d = x_tensor(cfg, xk), x_tensor(cfg, xv)
    lv.loopvq_encode(layer.dims, xk_d, xv_d, layer.cb, layer.hsq, slots, whole, n_blocks=cfg.n_blocks,
                     block_stride_bytes=whole[0].numel())
    for beta in range(cfg.n_blocks):
        steps = slice(beta * cfg.Tc, (beta + 1) * cfg.Tc)
        lv.loopvq_encode(layer.dims, xk_d[steps].contiguous(), xv_d[steps].contiguous(), layer.cb, layer.hsq,
                         slots, parts[beta], first_block=beta, n_blocks=1)
    torch.cuda.synchronize()
    assert torch.equal(whole, parts)


def test_window_moves_on_and_pages_are_coded():
    # one request grows token by token.  New tokens go to bf16 window pages;
    # whenever the window holds n_r + 8 tokens its oldest page is coded into
    # the quantised cache (all loop steps at once) and leaves the window.
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=4, H_q=4)
    N0, N, n_s, n_r = 200, 400, 8, 64
    xk, xv = synth.make_kv(cfg, N, seed=90)                 # [T, N, H, D] bf16 values
    cb = synth.make_codebooks(cfg.replace(n_calib=400))
    lens = np.array([N])
    bt, npg = synth.make_block_table(cfg, lens)
    layer = GpuLayer(cfg, cb, N)
    P = cfg.page_size
    cache = torch.zeros((npg, cfg.H_kv, 2, P, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    n_pool = 16
    pool = torch.zeros((cfg.T, n_pool, cfg.H_kv, 2, 8, cfg.D), dtype=torch.bfloat16, device="cuda")
    xk_d, xv_d = x_tensor(cfg, xk), x_tensor(cfg, xv)
    free = list(range(n_pool))
    win_pages = []                                            # sink page(s) first, then window pages

    def put(pos, page):
        pool[:, page, :, 0, pos % 8, :] = xk_d[:, pos].to(torch.bfloat16)
        pool[:, page, :, 1, pos % 8, :] = xv_d[:, pos].to(torch.bfloat16)

    # prefill of N0 tokens: sink and window in bf16, the rest coded at once
    ws = max(n_s, (N0 - n_r) // 8 * 8)
    for pos in list(range(n_s)) + list(range(ws, N0)):
        if (pos < n_s and pos % 8 == 0) or (pos >= ws and (pos - ws) % 8 == 0):
            win_pages.append(free.pop(0))
        put(pos, win_pages[-1])
    coded = slice(n_s, ws)
    slots = synth.slot_mapping_for(bt, 0, ws - n_s, P, start=n_s)
    lv.loopvq_encode(layer.dims, xk_d[:, coded].contiguous(), xv_d[:, coded].contiguous(), layer.cb, layer.hsq,
                     to_dev(slots), cache)
    # the expected codes of every position, from the oracle
    ref_cache, _, _ = oracle.build_index_cache(xk, xv, cb, cfg.Tc, cfg.c, cfg.bits,
                                               synth.slot_mapping_for(bt, 0, N, P), npg, P)
    n_sink_pages = (n_s + 7) // 8
    checks = 0
    for n in range(N0, N + 1):
        if n > N0:                                            # token n-1 arrives
            pos = n - 1
            if (pos - ws) % 8 == 0:
                win_pages.append(free.pop(0))
            put(pos, win_pages[-1])
            if n - ws >= n_r + 8:                             # code the oldest window page
                page = win_pages.pop(n_sink_pages)
                src = np.arange(8, dtype=np.int32) + page * 8
                slots = synth.slot_mapping_for(bt, 0, 8, P, start=ws)
                lv.loopvq_encode_pages(layer.dims, pool, to_dev(src), layer.cb, layer.hsq, to_dev(slots), cache)
                free.append(page)
                ws += 8
        if n in (N0, 233, 300, N):
            torch.cuda.synchronize()
            got = cache.cpu().numpy()
            # the rows coded so far hold the oracle's nearest entries (an other
            # code only for a vector inside the oracle's near-tie band)
            cslots = synth.slot_mapping_for(bt, 0, ws - n_s, P, start=n_s)
            ties, bad = check_codes(cfg, got[None], xk[:, n_s:ws], xv[:, n_s:ws], cb, cslots)
            assert bad == 0
            same = all(np.array_equal(got[s // P, :, :, s % P], ref_cache[0][s // P, :, :, s % P]) for s in cslots)
            # decode reads the GPU-coded rows when they equal the oracle's, else the oracle's rows
            dcache = cache if same else to_dev(ref_cache[0])
            pt = np.array([win_pages], dtype=np.int32)
            for t in (1, 4):
                q = synth.make_queries(cfg, 1, t=t)
                o, lse = layer.decode_window(t, q, dcache, bt, np.array([n]), pool[t - 1], pt,
                                             np.array([n_s]), np.array([ws]), max_seq_len=N)
                ref = ref_decode_window(cfg, t, q, ref_cache[0], bt, np.array([n]), cb, [n_s], [ws],
                                        lambda b, h: (xk[t - 1, :n, h], xv[t - 1, :n, h]))
                err, ratio = compare(cfg, o, lse, ref, np.array([n]))
                _note(f"rollover n={n} (window from {ws}, near-ties {ties}, GPU rows read: {same}) t={t}: "
                      f"max err {err:.2e}")
                assert ratio <= 1.0
                checks += 1
    assert checks == 8
