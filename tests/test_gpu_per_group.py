"""GPU parity with one codebook per channel group (per_group = 1): encoder codes
against the oracle's nearest entries (outside its near-tie band), decode
attention against the oracle.  Same bars as the shared-codebook tests."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import GpuLayer, compare, dims_for, ref_decode, to_dev, x_tensor

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401


def _note(msg):
    print(msg, flush=True)


def _layer(cfg, cb, max_pos):
    return GpuLayer(cfg, cb, max_pos, dims=dims_for(cfg, per_group=1))


def _check_codes_pg(cfg, got_cache, xk, xv, cb, slots, heads):
    """(near-tie count, mismatches) of GPU rows against per-group nearest entries."""
    P = cfg.page_size
    slots = np.asarray(slots, np.int64)
    ties = bad = 0
    for beta in range(cfg.n_blocks):
        for h in heads:
            for kv, x in enumerate((xk, xv)):
                rows = got_cache[beta][slots // P, h, kv, slots % P, :]
                got = oracle.slots_to_groups(oracle.unpack_rows(rows, cfg.bits, cfg.n_groups))
                z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, beta)
                for g in range(cfg.n_groups):
                    E = cb[beta, h, kv, g].astype(np.float64)
                    res = oracle.nearest_entry(z[:, g, :], E, method="gemm")
                    ties += int(res.near_tie.sum())
                    bad += int((~oracle.accepts(z[:, g, :], E, res, got[:, g])).sum())
    return ties, bad


@pytest.mark.parametrize("name,over,n_tok", [
    ("layer1p4b", dict(H_kv=4, H_q=4), 300),                         # bf16, c = 4, G = 16
    ("gqa_ragged", dict(H_kv=2, H_q=8), 200),                        # bf16, c = 8, G = 32
    ("tiny", dict(bits=8, D=64, c=2, Tc=4), 256),                    # fp32 input, G = 8
])
def test_per_group_encode(name, over, n_tok):
    cfg = synth.config_by_name(name).replace(n_calib=400, **over)
    xk, xv = synth.make_kv(cfg, n_tok, seed=cfg.index + 90)
    cb = synth.make_codebooks_per_group(cfg)
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n_tok, cfg.page_size)
    layer = _layer(cfg, cb, 16)
    cache = torch.zeros((cfg.n_blocks, npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8,
                        device="cuda")
    lv.loopvq_encode(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), layer.cb, layer.hsq,
                     to_dev(slots.astype(np.int32)), cache, n_blocks=cfg.n_blocks, block_stride_bytes=cache[0].numel())
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    ties, bad = _check_codes_pg(cfg, got, xk, xv, cb, slots, heads=range(cfg.H_kv))
    _note(f"{name} per-group encode: near-ties {ties}, mismatches outside the band {bad}")
    assert bad == 0
    # hsq of every group's entries
    hsq = layer.hsq.cpu().numpy()
    np.testing.assert_allclose(hsq, 0.5 * (cb.astype(np.float64) ** 2).sum(-1), rtol=2 ** -24, atol=0)


@pytest.mark.parametrize("name,over,lens", [
    ("layer1p4b", {}, [1000, 1, 257, 64, 72, 0, 1003, 500, 8, 9, 300, 2048, 71, 600, 128, 5]),   # shared rows
    ("layer1p4b", dict(io_dtype="f32"), [3000, 0, 1, 129]),
    ("gqa_ragged", {}, [1500, 1, 0, 700, 64, 2049]),                                          # pairs share a stream
    ("layer1p4b", dict(page_size=8, H_kv=4, H_q=4), [600, 37]),
])
def test_per_group_decode(name, over, lens):
    cfg = synth.config_by_name(name).replace(**over)
    lens = np.array(lens)
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 95)
    cb = synth.make_codebooks_per_group(cfg.replace(n_calib=400))
    layer = _layer(cfg, cb, int(lens.max()))
    for t in (1, 4):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode(t, q, cache, bt, lens)
        ref = ref_decode(cfg, t, q, cache, bt, lens, cb, heads=(0, cfg.H_kv - 1))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"{name} per-group decode t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_per_group_encode_then_decode_and_full_size():
    # GPU encoder's cache into the GPU decoder, checked against the oracle
    # on the oracle's own cache of the same data (identical when no near-ties)
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=2, H_q=2, n_calib=400)
    n = 500
    xk, xv = synth.make_kv(cfg, n, seed=97)
    cb = synth.make_codebooks_per_group(cfg)
    lens = np.array([n])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = synth.slot_mapping_for(bt, 0, n, cfg.page_size)
    layer = _layer(cfg, cb, n)
    cache = torch.zeros((npg, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    lv.loopvq_encode(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), layer.cb, layer.hsq,
                     to_dev(slots.astype(np.int32)), cache)
    ref_cache, ties, _ = oracle.build_index_cache(xk, xv, cb, cfg.Tc, cfg.c, cfg.bits, slots, npg, cfg.page_size,
                                                  method="gemm")
    got = cache.cpu().numpy()
    same = np.array_equal(got, ref_cache[0])
    assert same or ties > 0
    for t in (2, 3):
        q = synth.make_queries(cfg, 1, t=t)
        o, lse = layer.decode(t, q, cache if same else to_dev(ref_cache[0]), bt, lens)
        ref = ref_decode(cfg, t, q, ref_cache[0], bt, lens, cb)
        assert compare(cfg, o, lse, ref, lens)[1] <= 1.0
    # the 32K batch with per-group codebooks, sampled
    cfg = synth.config_by_name("longctx32k")
    lens = synth.make_seq_lens(cfg)
    bt, npg = synth.make_block_table(cfg, lens)
    cache = to_dev(synth.random_index_cache(cfg, npg, 98))
    cb = synth.make_codebooks_per_group(cfg.replace(n_calib=400))
    layer = _layer(cfg, cb, int(lens.max()))
    q = synth.make_queries(cfg, len(lens), t=1)
    o, lse = layer.decode(1, q, cache, bt, lens)
    ref = ref_decode(cfg, 1, q, cache.cpu().numpy(), bt, lens, cb, requests=(0, 15), heads=(0, 15))
    err, ratio = compare(cfg, o, lse, ref, lens)
    _note(f"longctx32k per-group decode: max err {err:.2e} (bound ratio {ratio:.2f})")
    assert ratio <= 1.0
