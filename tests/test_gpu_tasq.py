"""GPU parity of the TaSQ+LoopVQ key path against the fp64 oracle: the key
transform and coding (loopvq_encode_tasq) and decode attention over
TaSQ-coded keys (loopvq_decode_attn_tasq), with and without the bf16 window.

Bars: sigma bit-exact in fp16, except where the exact RMS lies within 2e-6
relative of an fp16 rounding midpoint (then either neighbour is accepted);
key and value codes equal the oracle's nearest entries outside its near-tie
band (tokens with a midpoint sigma excluded from the key check, their u
differs by an ulp of sigma); decode outputs within 2e-3 max-abs (+ half a
bf16 ulp for bf16 output), lse within 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (GpuLayer, check_codes, compare, ref_decode_tasq, sigma_at_positions, to_dev,
                      x_tensor)

pytestmark = pytest.mark.gpu
tq = oracle.tasq_ref

if torch.cuda.is_available():
    import decode_attention_loopvq_amd as lv  # noqa: F401


def _note(msg):
    print(msg, flush=True)


def _tasq_codebooks(cfg, w, perm, seed):
    """K codebooks sampled from u of calibration keys (the oracle's transform), V from the values."""
    ck, cv = synth.make_kv(cfg, cfg.n_calib, seed=seed)
    cu, _ = tq.tasq_transform(ck, w, perm, cfg.Tc)
    return synth.codebooks_from_vectors(cfg, cu, cv, seed=seed + 1)


def _random_sigma(cfg, n_slots, seed):
    return np.stack([synth.make_sigma(n_slots, seed + t) for t in range(cfg.T)])


@pytest.mark.parametrize("name,over,n_tok", [
    ("layer1p4b", dict(H_kv=4, H_q=4), 300),
    ("gqa_ragged", dict(H_kv=2, H_q=8), 200),        # c = 8
    ("tiny", dict(bits=8), 256),                     # D = 64, c = 2, fp32 input
    ("deeploop", dict(H_kv=2, H_q=2), 64),           # eight blocks
    # 32 loop steps share the transform's workgroups, so each walks several
    # groups of four tokens (the last one partial)
    ("deeploop", dict(H_kv=2, H_q=2), 300),
])
def test_tasq_encode(name, over, n_tok):
    cfg = synth.config_by_name(name).replace(n_calib=400, **over)
    xk, xv = synth.make_kv(cfg, n_tok, seed=cfg.index + 110)
    w, perm = synth.make_tasq(cfg)
    u, s16 = tq.tasq_transform(xk, w, perm, cfg.Tc)
    cb = _tasq_codebooks(cfg, w, perm, cfg.index + 1110)
    lens = np.array([n_tok])
    bt, npg = synth.make_block_table(cfg, lens)
    P = cfg.page_size
    slots = synth.slot_mapping_for(bt, 0, n_tok, P)
    layer = GpuLayer(cfg, cb, 16)
    cache = torch.zeros((cfg.n_blocks, npg, cfg.H_kv, 2, P, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    sigma = torch.zeros((cfg.T, npg * P), dtype=torch.float16, device="cuda")
    _note(f"{name}: encode_tasq n_tok={n_tok} H_kv={cfg.H_kv} blocks={cfg.n_blocks}")
    lv.loopvq_encode_tasq(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), to_dev(w), to_dev(perm), sigma,
                          layer.cb, layer.hsq, to_dev(slots), cache, n_blocks=cfg.n_blocks,
                          block_stride_bytes=cache[0].numel())
    torch.cuda.synchronize()
    # sigma: the fp16 RMS at each token's slot
    got_sig = sigma.cpu().numpy().astype(np.float64)[:, slots]
    exact = np.stack([tq.tasq_sigma(xk[t], w[t]) for t in range(cfg.T)])
    mid = tq.f16_near_midpoint(exact)
    assert np.array_equal(got_sig[~mid], s16[~mid])
    ulp = np.spacing(s16[mid].astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got_sig[mid] - exact[mid]) <= ulp)
    # codes: keys against the oracle's u, values as usual
    got = cache.cpu().numpy()
    ties_all = 0
    for beta in range(cfg.n_blocks):
        ok = ~mid[beta * cfg.Tc:(beta + 1) * cfg.Tc].any(axis=0)
        ties, bad = check_codes(cfg, got, u[:, ok], xv[:, ok], cb, slots[ok], blocks=[beta])
        ties_all += ties
        assert bad == 0, (beta, bad)
    _note(f"{name} TaSQ encode: midpoint sigmas {int(mid.sum())}, near-ties {ties_all}, no mismatches")


@pytest.mark.parametrize("name,over,lens", [
    ("layer1p4b", {}, [1000, 1, 257, 64, 72, 0, 1003, 500, 8, 9, 300, 2048, 71, 600, 128, 5]),  # shared rows
    ("gqa_ragged", {}, [1500, 1, 0, 700]),              # shared rows, the duo's pairs share keys
    ("gqa_ragged", {}, [1500, 1, 0, 700, 64, 2049]),    # per-wave rows, shared keys
    ("layer1p4b", dict(io_dtype="f32"), [3000, 0, 1, 129]),
    ("layer1p4b", dict(page_size=8, H_kv=4, H_q=4), [600, 37]),
    ("tiny", dict(bits=8), [256]),                      # D = 64, c = 2, fp32 queries
])
def test_tasq_decode(name, over, lens):
    cfg = synth.config_by_name(name).replace(**over)
    lens = np.array(lens)
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 120)
    cb = synth.make_codebooks(cfg.replace(n_calib=400))
    w, perm = synth.make_tasq(cfg)
    sigma = _random_sigma(cfg, npg * cfg.page_size, 121)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    heads = (0, cfg.H_kv - 1) if cfg.H_kv > 2 else None
    for t in sorted({1, cfg.T}):
        q = synth.make_queries(cfg, len(lens), t=t)
        _note(f"{name} TaSQ decode t={t} lens={lens.tolist()}")
        o, lse = layer.decode_tasq(t, q, cache, bt, lens, w, perm, sigma)
        ref = ref_decode_tasq(cfg, t, q, cache, bt, lens, cb, w, perm, sigma, heads=heads)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"  max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_tasq_encode_then_decode():
    # the GPU-coded cache and sigma into the GPU decoder, checked against the
    # oracle on the oracle's own cache and sigma (identical when no near-ties)
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=2, H_q=2, n_calib=400)
    n = 500
    xk, xv = synth.make_kv(cfg, n, seed=130)
    w, perm = synth.make_tasq(cfg)
    u, s16 = tq.tasq_transform(xk, w, perm, cfg.Tc)
    cb = _tasq_codebooks(cfg, w, perm, 131)
    lens = np.array([n])
    bt, npg = synth.make_block_table(cfg, lens)
    P = cfg.page_size
    slots = synth.slot_mapping_for(bt, 0, n, P)
    layer = GpuLayer(cfg, cb, n)
    cache = torch.zeros((npg, cfg.H_kv, 2, P, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    sigma = torch.zeros((cfg.T, npg * P), dtype=torch.float16, device="cuda")
    lv.loopvq_encode_tasq(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), to_dev(w), to_dev(perm), sigma,
                          layer.cb, layer.hsq, to_dev(slots), cache)
    ref_cache, ties, _ = oracle.build_index_cache(u, xv, cb, cfg.Tc, cfg.c, cfg.bits, slots, npg, P, method="gemm")
    ref_sigma = np.zeros((cfg.T, npg * P))
    ref_sigma[:, slots] = s16
    torch.cuda.synchronize()
    same = np.array_equal(cache.cpu().numpy(), ref_cache[0]) and \
        np.array_equal(sigma.cpu().numpy().astype(np.float64), ref_sigma)
    _note(f"TaSQ encode -> decode: GPU cache equals the oracle's: {same} (near-ties {ties})")
    for t in (1, 2, 3, 4):
        q = synth.make_queries(cfg, 1, t=t)
        o, lse = layer.decode_tasq(t, q, cache if same else to_dev(ref_cache[0]), bt, lens, w, perm,
                                   sigma if same else ref_sigma.astype(np.float16))
        ref = ref_decode_tasq(cfg, t, q, ref_cache[0], bt, lens, cb, w, perm, ref_sigma)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"  t={t}: max err {err:.2e}")
        assert ratio <= 1.0


def test_tasq_zero_keys_and_odd_token_counts():
    # tokens whose keys are zero at some loop steps get sigma = 0 and u = 0 there;
    # 37 tokens leave a partial workgroup of the transform and a partial encoder unit
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=2, H_q=2, n_calib=400)
    n = 37
    xk, xv = synth.make_kv(cfg, n, seed=190)
    xk[1, 3] = 0.0
    xk[:, 20] = 0.0
    w, perm = synth.make_tasq(cfg)
    u, s16 = tq.tasq_transform(xk, w, perm, cfg.Tc)
    assert s16[1, 3] == 0 and np.all(s16[:, 20] == 0)
    cb = _tasq_codebooks(cfg, w, perm, 191)
    lens = np.array([n])
    bt, npg = synth.make_block_table(cfg, lens)
    P = cfg.page_size
    slots = synth.slot_mapping_for(bt, 0, n, P)
    layer = GpuLayer(cfg, cb, n)
    cache = torch.zeros((npg, cfg.H_kv, 2, P, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    sigma = torch.full((cfg.T, npg * P), 7.0, dtype=torch.float16, device="cuda")
    lv.loopvq_encode_tasq(layer.dims, x_tensor(cfg, xk), x_tensor(cfg, xv), to_dev(w), to_dev(perm), sigma,
                          layer.cb, layer.hsq, to_dev(slots), cache)
    torch.cuda.synchronize()
    got_sig = sigma.cpu().numpy().astype(np.float64)
    exact = np.stack([tq.tasq_sigma(xk[t], w[t]) for t in range(cfg.T)])
    mid = tq.f16_near_midpoint(exact)
    assert np.array_equal(got_sig[:, slots][~mid], s16[~mid])
    untouched = np.setdiff1d(np.arange(npg * P), slots)
    assert np.all(got_sig[:, untouched] == 7.0)              # only the coded slots are written
    ok = ~mid.any(axis=0)
    ties, bad = check_codes(cfg, cache.cpu().numpy()[None], u[:, ok], xv[:, ok], cb, slots[ok])
    assert bad == 0
    ref_sigma = np.zeros((cfg.T, npg * P))
    ref_sigma[:, slots] = s16
    ref_cache, _, _ = oracle.build_index_cache(u, xv, cb, cfg.Tc, cfg.c, cfg.bits, slots, npg, P, method="gemm")
    for t in (1, 2):
        q = synth.make_queries(cfg, 1, t=t)
        o, lse = layer.decode_tasq(t, q, to_dev(ref_cache[0]), bt, lens, w, perm, ref_sigma.astype(np.float16))
        ref = ref_decode_tasq(cfg, t, q, ref_cache[0], bt, lens, cb, w, perm, ref_sigma)
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"zero-key tokens t={t}: max err {err:.2e}")
        assert ratio <= 1.0


@pytest.mark.parametrize("n_sink,n_recent", [(8, 64), (64, 256)])
def test_tasq_decode_with_window(n_sink, n_recent):
    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([1000, 1, 257, 64, 72, 0, 1003, 500, 8, 9, 300, 2048, 71, 600, 128, 5])
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 140)
    cb = synth.make_codebooks(cfg)
    w, perm = synth.make_tasq(cfg)
    sigma = _random_sigma(cfg, npg * cfg.page_size, 141)
    ns, ws, pt, nwp = synth.make_window(cfg, lens, n_sink, n_recent)
    rng = np.random.default_rng(142)
    ks = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    vs = [synth.round_to_bf16(rng.standard_normal((int(n), cfg.H_kv, cfg.D), dtype=np.float32)) for n in lens]
    pages = synth.fill_window_pages(nwp, pt, ns, ws, lens, lambda b, pos: ks[b][pos], lambda b, pos: vs[b][pos],
                                    cfg.H_kv, cfg.D)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    for t in (1, 3):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode_tasq(t, q, cache, bt, lens, w, perm, sigma, window=(pages, pt, ns, ws))
        ref = ref_decode_tasq(cfg, t, q, cache, bt, lens, cb, w, perm, sigma, heads=(0, 7, 15),
                              window=(ns, ws, lambda b, h: (ks[b][:, h], vs[b][:, h])))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"TaSQ + window ({n_sink}, {n_recent}) t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0


def test_tasq_decode_full_size_sampled():
    # the 32K-context batch of 16 requests, 16 KV heads, TaSQ-coded keys
    cfg = synth.config_by_name("longctx32k")
    lens = synth.make_seq_lens(cfg)
    bt, npg = synth.make_block_table(cfg, lens)
    cache = to_dev(synth.random_index_cache(cfg, npg, 150))
    cb = synth.make_codebooks(cfg)
    w, perm = synth.make_tasq(cfg)
    sigma = _random_sigma(cfg, npg * cfg.page_size, 151)
    layer = GpuLayer(cfg, cb, int(lens.max()))
    cache_np = cache.cpu().numpy()
    for t in (2, 4):
        q = synth.make_queries(cfg, len(lens), t=t)
        o, lse = layer.decode_tasq(t, q, cache, bt, lens, w, perm, sigma)
        ref = ref_decode_tasq(cfg, t, q, cache_np, bt, lens, cb, w, perm, sigma, requests=(0, 15), heads=(0, 15))
        err, ratio = compare(cfg, o, lse, ref, lens)
        _note(f"longctx32k TaSQ decode t={t}: max err {err:.2e} (bound ratio {ratio:.2f})")
        assert ratio <= 1.0
