"""GPU parity of decode attention over a bf16 sink and recent window plus coded
pages (loopvq_decode_attn_window) against the fp64 oracle.

Same bars as the coded-only path: outputs within 2e-3 max-abs (+ half a bf16
ulp for bf16 output), lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuLayer, compare, ref_decode_window, to_dev

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _random_bf16_kv(cfg, lens, seed):
    """Per-request pre-RoPE bf16 keys and values [len, H_kv, D] for the window tokens."""
    rng = np.random.default_rng(seed)
    ks = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    vs = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    return ks, vs


def _pages(cfg, lens, ns, ws, pt, npg, ks, vs):
    return synth.fill_window_pages(npg, pt, ns, ws, lens, lambda b, pos: ks[b][pos], lambda b, pos: vs[b][pos],
                                   cfg.H_kv, cfg.D)


@pytest.mark.parametrize("n_sink,n_recent", [(8, 64), (64, 64)])
def test_window_tiny_every_loop_step(n_sink, n_recent):
    # fp32 queries and output, D = 64, 4-bit codes; the coded part comes from
    # the oracle's own encoding of the same data, the bf16 part is that data
    cfg = synth.config_by_name("tiny")
    N = cfg.seq_len
    xk, xv = synth.make_kv(cfg, N)
    cb = synth.make_codebooks(cfg)
    lens = np.array([N])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, N, cfg.page_size)
    caches, _, _ = oracle.build_index_cache(xk, xv, cb, cfg.Tc, cfg.c, cfg.bits, slots, npg, cfg.page_size)
    ns, ws, pt, nwp = synth.make_window(cfg, lens, n_sink, n_recent)
    layer = GpuLayer(cfg, cb, N)
    for t in range(1, cfg.T + 1):
        kb = synth.round_to_bf16(xk[t - 1])
        vb = synth.round_to_bf16(xv[t - 1])
        pages = _pages(cfg, lens, ns, ws, pt, nwp, [kb], [vb])
        q = synth.make_queries(cfg, 1, t=t)
        beta = (t - 1) // cfg.Tc
        o, lse = layer.decode_window(t, q, caches[beta], bt, lens, pages, pt, ns, ws)
        ref = ref_decode_window(cfg, t, q, caches[beta], bt, lens, cb, ns, ws,
                                lambda b, h: (kb[:, h], vb[:, h]))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"tiny window ({n_sink}, {n_recent}) t={t}: max err {err:.2e}")
        assert ratio <= 1.0


@pytest.mark.parametrize("n_sink,n_recent", [(8, 64), (64, 256)])
def test_window_ragged_batch(n_sink, n_recent):
    # 16 ragged requests (eight duos per head: the workgroup-shared RoPE path),
    # including empty, one-token and all-bf16 requests
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([1000, 1, 257, 64, 72, 0, 1003, 500, 8, 9, 300, 2048, 71, 600, 128, 5])
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 31)
    cb = synth.make_codebooks(cfg)
    ns, ws, pt, nwp = synth.make_window(cfg, lens, n_sink, n_recent)
    ks, vs = _random_bf16_kv(cfg, lens, 32)
    pages = _pages(cfg, lens, ns, ws, pt, nwp, ks, vs)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    for t in (1, 3):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode_window(t, q, cache, bt, lens, pages, pt, ns, ws)
        ref = ref_decode_window(cfg, t, q, cache, bt, lens, cb, ns, ws,
                                lambda b, h: (ks[b][:, h], vs[b][:, h]), heads=(0, 5, 15))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"layer window ({n_sink}, {n_recent}) t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_window_gqa_and_small_pages():
    # GQA group 4 (pairs of one request share a stream), then 8-token pages
    cfg = synth.config_by_name("gqa_ragged")
    lens = np.array([1500, 1, 0, 700, 64, 2049])
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 41)
    cb = synth.make_codebooks(cfg)
    ns, ws, pt, nwp = synth.make_window(cfg, lens, 16, 64)
    ks, vs = _random_bf16_kv(cfg, lens, 42)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=2)
    o, lse = layer.decode_window(2, q, cache, bt, lens, _pages(cfg, lens, ns, ws, pt, nwp, ks, vs), pt, ns, ws)
    ref = ref_decode_window(cfg, 2, q, cache, bt, lens, cb, ns, ws, lambda b, h: (ks[b][:, h], vs[b][:, h]))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"gqa window: max err {err:.2e}")
    assert ratio <= 1.0

    cfg = synth.config_by_name("layer1p4b").replace(page_size=8, H_kv=4, H_q=4)
    lens = np.array([600, 37, 90])
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 43)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    ns, ws, pt, nwp = synth.make_window(cfg, lens, 24, 40)
    ks, vs = _random_bf16_kv(cfg, lens, 44)
    layer = GpuLayer(cfg, cb, 600)
    q = synth.make_queries(cfg, len(lens), t=4)
    o, lse = layer.decode_window(4, q, cache, bt, lens, _pages(cfg, lens, ns, ws, pt, nwp, ks, vs), pt, ns, ws)
    ref = ref_decode_window(cfg, 4, q, cache, bt, lens, cb, ns, ws, lambda b, h: (ks[b][:, h], vs[b][:, h]))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"8-token pages window: max err {err:.2e}")
    assert ratio <= 1.0


def test_empty_window_is_the_coded_decode_bit_for_bit():
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([1000, 257, 1, 0])
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 51)
    cb = synth.make_codebooks(cfg)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=1)
    # no sink and the window starting at the end: every token is coded
    ns = np.zeros(len(lens), np.int32)
    ws = lens.astype(np.int32)
    pt = np.zeros((len(lens), 1), np.int32)
    pages = np.zeros((1, cfg.H_kv, 2, 8, cfg.D), np.float32)
    o1, l1 = layer.decode(1, q, cache, bt, lens)
    o2, l2 = layer.decode_window(1, q, cache, bt, lens, pages, pt, ns, ws)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_window_full_size_sampled():
    # the 32K-context batch of 16 with a 64-token sink and a 256-token window
    cfg = synth.config_by_name("longctx32k")
    lens = synth.make_seq_lens(cfg)
    bt, npg = synth.make_block_table(cfg, lens)
    cache = to_dev(synth.random_index_cache(cfg, npg, 61))
    cb = synth.make_codebooks(cfg)
    ns, ws, pt, nwp = synth.make_window(cfg, lens, 64, 256)
    rng = np.random.default_rng(62)
    # bf16 values only at the bf16 positions (the rest is never read)
    nb = int(ns[0] + lens[0] - ws[0])
    kw = synth.round_to_bf16(rng.standard_normal((len(lens), nb, cfg.H_kv, cfg.D), dtype=np.float32))
    vw = synth.round_to_bf16(rng.standard_normal((len(lens), nb, cfg.H_kv, cfg.D), dtype=np.float32))

    def dense(b, h, src):
        full = np.zeros((int(lens[b]), cfg.D), np.float32)
        full[synth.window_positions(int(ns[b]), int(ws[b]), int(lens[b]))] = src[b, :, h]
        return full
    pages = synth.fill_window_pages(
        nwp, pt, ns, ws, lens,
        lambda b, pos: kw[b, np.searchsorted(synth.window_positions(int(ns[b]), int(ws[b]), int(lens[b])), pos)],
        lambda b, pos: vw[b, np.searchsorted(synth.window_positions(int(ns[b]), int(ws[b]), int(lens[b])), pos)],
        cfg.H_kv, cfg.D)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    cache_np = cache.cpu().numpy()
    for t in (1, 4):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode_window(t, q, cache, bt, lens, pages, pt, ns, ws)
        ref = ref_decode_window(cfg, t, q, cache_np, bt, lens, cb, ns, ws,
                                lambda b, h: (dense(b, h, kw), dense(b, h, vw)),
                                requests=(0, 15), heads=(0, 15))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"longctx32k window t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0
