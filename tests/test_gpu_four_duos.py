"""GPU parity of decode with four duos of (request, query head) pairs per KV
head against the fp64 oracle.

Four duos per head is the shape of the 1.4B-layer batch (eight requests, one
query head per KV head) and of four requests with a GQA group of two: the
eight waves of a workgroup then hold two chunks, and each wave reads its own
RoPE rows.  The cases cover ragged lengths (an empty request, one ending in
its first step), 16-token pages, a GQA pair and a bf16 sink and window.  Same
bars as the other decode tests: outputs within 2e-3 max-abs (+ half a bf16
ulp for bf16 output), lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import GpuLayer, compare, ref_decode, ref_decode_window

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _case(cfg, lens, seed):
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, seed)
    cb = synth.make_codebooks(cfg)
    return bt, cache, cb


@pytest.mark.parametrize("page_size,lens", [
    # ragged: the two chunk groups of a workgroup have different step counts,
    # one request ends inside its first step, one is empty
    (64, [4096, 1, 700, 2049, 64, 1500, 3333, 0]),
    # 16-token pages: a chunk spans eight pages
    (16, [1025, 300, 17, 1024, 999, 128, 2, 640]),
])
def test_four_duos_ragged(page_size, lens):
    cfg = synth.config_by_name("layer1p4b").replace(page_size=page_size)
    lens = np.array(lens)
    assert len(lens) == 8 and cfg.H_q == cfg.H_kv          # four duos per head
    bt, cache, cb = _case(cfg, lens, 41 + page_size)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    for t in (1, 4):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, cache, bt, lens)
        ref = ref_decode(cfg, t, q, cache, bt, lens, cb, heads=(0, 9, 15))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"four duos per head P={page_size} t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_four_duos_gqa_pairs():
    # a GQA group of two: a duo is two query heads of one request (shared keys)
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=8, H_q=16)
    lens = np.array([2000, 513, 4096, 77])
    bt, cache, cb = _case(cfg, lens, 43)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=2)
    o, lse = layer.decode(2, q, cache, bt, lens)
    ref = ref_decode(cfg, 2, q, cache, bt, lens, cb, heads=(0, 7))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"four duos per head, GQA 2: max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


def test_four_duos_with_window():
    # coded positions start after a bf16 sink (past the first chunk's first
    # page) and end before a bf16 recent window
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([3000, 90, 1200, 4096, 333, 64, 2500, 700])
    bt, cache, cb = _case(cfg, lens, 44)
    ns, ws, pt, nwp = synth.make_window(cfg, lens, 72, 100)
    rng = np.random.default_rng(45)
    ks = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    vs = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    pages = synth.fill_window_pages(nwp, pt, ns, ws, lens, lambda b, pos: ks[b][pos], lambda b, pos: vs[b][pos],
                                    cfg.H_kv, cfg.D)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=3)
    o, lse = layer.decode_window(3, q, cache, bt, lens, pages, pt, ns, ws)
    ref = ref_decode_window(cfg, 3, q, cache, bt, lens, cb, ns, ws, lambda b, h: (ks[b][:, h], vs[b][:, h]),
                            heads=(0, 15))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"four duos per head with a bf16 window: max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


def test_four_duos_deterministic():
    # two calls on the same inputs give the same bits (no order-dependent sums)
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([1500, 3000, 7, 2222, 4096, 640, 1, 1111])
    bt, cache, cb = _case(cfg, lens, 46)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=1)
    o1, l1 = layer.decode(1, q, cache, bt, lens)
    o2, l2 = layer.decode(1, q, cache, bt, lens)
    torch.cuda.synchronize()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "decode not deterministic"
