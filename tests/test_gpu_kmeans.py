"""GPU parity of plain k-means on coupled vectors against the fp64 oracle: one
Lloyd iteration is loopvq_encode (assignment) then loopvq_kmeans_update (each
entry to the mean of its vectors, rounded to fp16); and the Fig. 2c
comparison of the LoopVQ paper (section "Redundancy along the loop axis")
run on the GPU.

Bars: codes equal the oracle's nearest entries outside its near-tie band; the
updated entries equal fp16(mean) of the oracle's assignment bit for bit (fp64
sums of bf16 values are exact on both sides), entries touched by a near-tie
excepted; error sums within 1e-9 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dims_for, to_dev, x_tensor

pytestmark = pytest.mark.gpu
tq = oracle.tasq_ref

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401


def _note(msg):
    print(msg, flush=True)


def _channel_cfg(cfg):
    """G = c*Tc channels of one loop step: c = G, Tc = 1, the Tc steps laid end to end as tokens."""
    return cfg.replace(c=cfg.G, Tc=1, T=1, rhos=())


def _gpu_iteration(cfg, xk_d, xv_d, cb_d, n_tok):
    """One Lloyd iteration on the GPU; returns (codes [n_tok, H, 2, n_groups] in group order, cb_out, err)."""
    dims = dims_for(cfg)
    P = cfg.page_size
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    slots = to_dev(synth.slot_mapping_for(bt, 0, n_tok, P))
    _, hsq = lv.loopvq_build_codebook_slices(dims, cb_d)
    cache = torch.zeros((npg, cfg.H_kv, 2, P, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    lv.loopvq_encode(dims, xk_d, xv_d, cb_d, hsq, slots, cache)
    cb_out, err = lv.loopvq_kmeans_update(dims, xk_d, xv_d, slots, cache, cb_d)
    torch.cuda.synchronize()
    s = synth.slot_mapping_for(bt, 0, n_tok, P).astype(np.int64)
    rows = cache.cpu().numpy()[s // P, :, :, s % P, :]
    codes = np.empty((n_tok, cfg.H_kv, 2, cfg.n_groups), np.int64)
    for h in range(cfg.H_kv):
        for kv in range(2):
            codes[:, h, kv] = oracle.slots_to_groups(oracle.unpack_rows(rows[:, h, kv], cfg.bits, cfg.n_groups))
    return codes, cb_out.cpu().numpy(), err.cpu().numpy()


def _check_iteration(cfg, x, cb0, codes, cb1, err):
    """x = (xk, xv) [T, n, H, D] in cfg's layout; one block."""
    touched_total = 0
    ties_total = 0
    for h in range(cfg.H_kv):
        for kv in range(2):
            z = oracle.coupled_vectors(x[kv][:, :, h, :], cfg.Tc, cfg.c, 0).reshape(-1, cfg.G)
            E = cb0[0, h, kv].astype(np.float64)
            res = oracle.nearest_entry(z, E, method="gemm")
            got = codes[:, h, kv].reshape(-1)
            assert oracle.accepts(z, E, res, got).all()
            ties_total += int(res.near_tie.sum())
            want = tq.f16_round(tq.kmeans_update(z, res.idx, E))
            differ = got != res.idx
            touched = np.unique(np.concatenate([got[differ], res.idx[differ]]))
            keep = np.ones(cfg.K, bool)
            keep[touched] = False
            touched_total += int((~keep).sum())
            np.testing.assert_array_equal(cb1[0, h, kv][keep].astype(np.float64), want[keep])
            d = z - E[res.idx]
            np.testing.assert_allclose(err[0, h, kv, 0], (d * d).sum(), rtol=1e-9)
            np.testing.assert_allclose(err[0, h, kv, 1], (z * z).sum(), rtol=1e-12)
    return ties_total, touched_total


@pytest.mark.parametrize("name,over,n_tok", [
    ("layer1p4b", dict(H_kv=2, H_q=2), 1500),        # loop grouping: c = 4 channels x Tc = 4 steps
    ("gqa_ragged", dict(H_kv=1, H_q=4), 900),         # c = 8, G = 32
    ("tiny", {}, 256),                                # 4-bit, fp32 data, G = 8
])
def test_kmeans_iteration_loop_grouping(name, over, n_tok):
    cfg = synth.config_by_name(name).replace(n_calib=400, **over)
    xk, xv = synth.make_kv(cfg, n_tok, seed=cfg.index + 160)
    cb0 = synth.make_codebooks(cfg)
    codes, cb1, err = _gpu_iteration(cfg, x_tensor(cfg, xk), x_tensor(cfg, xv), to_dev(cb0), n_tok)
    ties, touched = _check_iteration(cfg, (xk, xv), cb0, codes, cb1, err)
    _note(f"{name} k-means iteration: near-ties {ties}, entries excluded {touched}")


def test_kmeans_iteration_channel_grouping():
    # 16 channels of one step, one codebook shared by the 4 steps of the block
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=2, H_q=2, n_calib=400)
    n = 1200
    xk, xv = synth.make_kv(cfg, n, seed=170)
    ch = _channel_cfg(cfg)
    xkr, xvr = (a.reshape(1, cfg.T * n, cfg.H_kv, cfg.D) for a in (xk, xv))
    cb0 = synth.codebooks_from_vectors(ch, xkr, xvr, seed=171)
    codes, cb1, err = _gpu_iteration(ch, x_tensor(ch, xkr), x_tensor(ch, xvr), to_dev(cb0), cfg.T * n)
    ties, touched = _check_iteration(ch, (xkr, xvr), cb0, codes, cb1, err)
    _note(f"channel grouping k-means iteration: near-ties {ties}, entries excluded {touched}")


def test_fig2c_on_the_gpu():
    # same bit width (8-bit code per 16 coordinates), one codebook per cache
    # under both groupings, 8 Lloyd iterations from K distinct data vectors:
    # the loop-axis grouping reconstructs markedly better; the GPU's error
    # follows the oracle's k-means (fp16 entries after every update)
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=1, H_q=1, n_calib=400)
    n, iters = 1024, 8
    xk, xv = synth.make_kv(cfg, n, seed=180)
    out = {}
    for grouping in ("loop", "channel"):
        c2 = cfg if grouping == "loop" else _channel_cfg(cfg)
        xs = (xk, xv) if grouping == "loop" else tuple(a.reshape(1, cfg.T * n, 1, cfg.D) for a in (xk, xv))
        ntok = xs[0].shape[1]
        cb = synth.codebooks_from_vectors(c2, xs[0], xs[1], seed=181)
        xd = tuple(x_tensor(c2, a) for a in xs)
        cbd = to_dev(cb)
        for _ in range(iters):
            _, cbn, err = _gpu_iteration(c2, xd[0], xd[1], cbd, ntok)
            cbd = to_dev(cbn)
        _, _, err = _gpu_iteration(c2, xd[0], xd[1], cbd, ntok)
        gpu_nmse = err[0, 0, :, 0] / err[0, 0, :, 1]               # K and V
        # the oracle's Lloyd iterations from the same start, entries rounded to fp16
        ref = []
        for kv in range(2):
            z = oracle.coupled_vectors(xs[kv][:, :, 0, :], c2.Tc, c2.c, 0).reshape(-1, c2.G)
            C = cb[0, 0, kv].astype(np.float64)
            for _ in range(iters):
                C = tq.f16_round(tq.kmeans_update(z, tq.kmeans_assign(z, C), C))
            ref.append(tq.nmse(z, C[tq.kmeans_assign(z, C)]))
        out[grouping] = gpu_nmse
        _note(f"Fig. 2c on the GPU, {grouping} grouping: NMSE K {gpu_nmse[0]:.4f} V {gpu_nmse[1]:.4f} "
              f"(oracle {ref[0]:.4f} {ref[1]:.4f})")
        np.testing.assert_allclose(gpu_nmse, ref, rtol=0.02)
    assert np.all(out["loop"] < 0.8 * out["channel"])
