"""GPU parity of the quad decode path (four query heads of one request per
wave) against the oracle, on the shapes that pick its code paths apart:
workgroup items taken in order of decreasing work (shared RoPE rows), chunk
edges, empty and one-token requests, a GQA group of eight (two quads per
request), the bf16 sink and window over quads, a batch too large to be put in
length order (index order instead), and head counts for which each
workgroup walks several items in turn.

Bars as in the other decode tests: outputs within 2e-3 (+ half a bf16 ulp of
the reference), lse within 1e-4 [LoopVQ paper, section "System
implementation", attention].
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import GpuLayer, compare, ref_decode, ref_decode_window

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _check(cfg, lens, seed, t, requests=None, heads=None):
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, seed)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    layer = GpuLayer(cfg, cb, max(int(lens.max()), 1))
    q = synth.make_queries(cfg, len(lens), t=t)
    o, lse = layer.decode(t, q, cache, bt, lens)
    ref = ref_decode(cfg, t, q, cache, bt, lens, cb, requests=requests, heads=heads)
    return compare(cfg, o, lse, ref, lens)


def test_quads_ordered_items_and_chunk_edges():
    # 16 requests -> 16 quads per KV head: shared RoPE rows, items in order of
    # decreasing work; lengths at and around the 512-position chunk edges
    cfg = synth.config_by_name("gqa_ragged")
    lens = np.array([0, 1, 511, 512, 513, 1023, 1024, 1025, 3000, 16, 17, 2048, 777, 64, 4099, 5])
    _note(f"quads, ordered items: lens {lens.tolist()}")
    err, ratio = _check(cfg, lens, 61, t=2)
    _note(f"max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


def test_quads_group_of_eight():
    # 8 KV heads, 64 query heads: two quads per request
    cfg = synth.config_by_name("gqa_ragged").replace(H_q=64)
    lens = np.array([900, 3, 2500, 0, 1200, 640, 4000, 1])
    _note(f"quads, group of 8: lens {lens.tolist()}")
    err, ratio = _check(cfg, lens, 62, t=4, heads=(0, 3, 7))
    _note(f"max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


def test_quads_with_bf16_window():
    # 8 requests: shared rows and ordered items with a bf16 sink and window
    cfg = synth.config_by_name("gqa_ragged")
    lens = np.array([1500, 40, 0, 700, 2049, 96, 1100, 513])
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 63)
    cb = synth.make_codebooks(cfg.replace(n_calib=300))
    ns, ws, pt, nwp = synth.make_window(cfg, lens, 16, 64)
    rng = np.random.default_rng(64)
    ks = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    vs = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    pages = synth.fill_window_pages(nwp, pt, ns, ws, lens, lambda b, pos: ks[b][pos], lambda b, pos: vs[b][pos],
                                    cfg.H_kv, cfg.D)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=3)
    o, lse = layer.decode_window(3, q, cache, bt, lens, pages, pt, ns, ws)
    ref = ref_decode_window(cfg, 3, q, cache, bt, lens, cb, ns, ws, lambda b, h: (ks[b][:, h], vs[b][:, h]))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"quads with window: max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


def test_quads_batch_beyond_the_length_order():
    # 520 requests: more than the kernel puts in length order, so quads go in
    # index order; short ragged lengths keep the oracle cheap
    cfg = synth.config_by_name("gqa_ragged").replace(H_kv=2, H_q=8)
    rng = np.random.default_rng(65)
    lens = rng.integers(0, 300, size=520).astype(np.int64)
    lens[7] = 2000
    _note("quads, 520 requests")
    err, ratio = _check(cfg, lens, 66, t=1, requests=(0, 7, 100, 311, 519))
    _note(f"max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0


@pytest.mark.parametrize("H_kv,B", [(40, 16), (100, 8)])
def test_quads_workgroups_walking_items(H_kv, B):
    # ordered items walked by CUs // H_kv workgroups per head (6 and 2 on
    # 256 CUs), so each workgroup takes several items in turn; 100 heads do
    # not divide the CU count; lengths up to six chunks, some empty
    cfg = synth.config_by_name("gqa_ragged").replace(H_kv=H_kv, H_q=4 * H_kv)
    rng = np.random.default_rng(67 + H_kv)
    lens = rng.integers(0, 2600, size=B).astype(np.int64)
    lens[1] = 0
    lens[2] = 1
    lens[3] = 2600
    _note(f"quads, H_kv={H_kv}, {B} requests, lens {lens.tolist()}")
    err, ratio = _check(cfg, lens, 68 + H_kv, t=3, requests=tuple(range(B)), heads=(0, H_kv // 2 + 1, H_kv - 1))
    _note(f"max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0
