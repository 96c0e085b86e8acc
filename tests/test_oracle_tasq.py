"""Pins of the TaSQ+LoopVQ and k-means parts of the fp64 oracle.

Each pin is independent of the oracle's own code: hand-worked values,
exactly representable constructions whose answer is textbook attention,
closed forms, a library k-means (SciPy) and invariants.  The last tests run
the Fig. 2c comparison of the LoopVQ paper (section "Redundancy along the loop
axis") on synthetic loop-correlated caches.
"""
import math

import numpy as np
import pytest
import scipy.cluster.vq
import torch

import oracle
import synth

tq = oracle.tasq_ref


# ---------------------------------------------------------------- fp16 scale
def test_f16_round_ties_to_even_and_midpoint_band():
    u = 2.0 ** -10                                   # fp16 spacing on [1, 2)
    assert tq.f16_round(np.array([1 + u / 2]))[0] == 1.0          # tie -> even (1.0)
    assert tq.f16_round(np.array([1 + 3 * u / 2]))[0] == 1 + 2 * u   # tie -> even (1 + 2u)
    assert tq.f16_round(np.array([1 + 0.49 * u]))[0] == 1.0
    near = tq.f16_near_midpoint(np.array([1 + u / 2, 1 + u / 2 + 1e-7, 1 + u / 4, 3.0]))
    assert near.tolist() == [True, True, False, False]


def test_sigma_is_the_rms_of_weighted_keys():
    # fifteen entries of magnitude 1 and one of magnitude 7 over H*D = 16:
    # mean square (15 + 49) / 16 = 4, so sigma = 2 exactly
    rng = np.random.default_rng(0)
    H, D = 2, 8
    w = 2.0 ** rng.integers(-2, 3, size=(H, D))
    y = rng.choice([-1.0, 1.0], size=(3, H * D))
    for j in range(3):
        y[j, rng.integers(H * D)] *= 7
    k = y.reshape(3, H, D) / w[None]
    np.testing.assert_array_equal(tq.tasq_sigma(k, w), [2.0, 2.0, 2.0])
    # against a library norm on random data
    k = rng.standard_normal((5, 4, 16))
    w = rng.random((4, 16)) + 0.5
    want = torch.linalg.vector_norm(torch.tensor(k * w[None]).reshape(5, -1), dim=1) / math.sqrt(64)
    np.testing.assert_allclose(tq.tasq_sigma(k, w), want.numpy(), rtol=1e-14)


# ---------------------------------------------------------------- permutation
def test_pair_sources_hand_worked():
    np.testing.assert_array_equal(tq.pair_source_channels(np.array([2, 0, 3, 1]), 8),
                                  [2, 6, 0, 4, 3, 7, 1, 5])


@pytest.mark.parametrize("c", [2, 4, 8])
def test_every_code_holds_whole_rope_pairs(c):
    rng = np.random.default_rng(c)
    D = 64
    src = tq.pair_source_channels(rng.permutation(D // 2), D)
    assert np.array_equal(np.sort(src), np.arange(D))
    for g in range(D // c):
        ch = src[g * c:(g + 1) * c]
        # c/2 frequencies, each present with both of its channels f and f + D/2
        f = ch % (D // 2)
        vals, cnt = np.unique(f, return_counts=True)
        assert len(vals) == c // 2 and np.all(cnt == 2)
        assert set(ch) == set(vals) | set(vals + D // 2)


# ---------------------------------------------------------------- transform
def test_transform_hand_worked():
    # one step, one token, H = 2, D = 8; w * k has fifteen +-1 and one 7, so
    # sigma = 2 and u = P(w k) / 2
    D, H = 8, 2
    wk = np.array([[1, -1, 1, 1, -1, 1, 1, -1], [1, 1, -1, 7, 1, -1, -1, 1]], dtype=np.float64)
    w = np.array([[1, 2, 0.5, 1, 4, 1, 0.25, 2], [2, 1, 1, 0.5, 1, 2, 1, 1]])
    k = (wk / w)[None, None]                            # [T=1, N=1, H, D]
    perm = np.array([[[1, 3, 0, 2], [0, 1, 2, 3]]])      # [n_blocks=1, H, D/2]
    u, s16 = tq.tasq_transform(k, w[None], perm, Tc=1)
    assert s16[0, 0] == 2.0
    # head 0: u = (wk[1], wk[5], wk[3], wk[7], wk[0], wk[4], wk[2], wk[6]) / 2
    np.testing.assert_array_equal(u[0, 0, 0], np.array([-1, 1, 1, -1, 1, -1, 1, 1]) / 2)
    # head 1: identity pairs: (wk[0], wk[4], wk[1], wk[5], ...) / 2
    np.testing.assert_array_equal(u[0, 0, 1], np.array([1, 1, 1, -1, -1, -1, 7, 1]) / 2)


def test_transform_inverse_round_trip_and_unit_rms():
    cfg = synth.config_by_name("layer1p4b").replace(H_kv=3, H_q=3)
    xk, _ = synth.make_kv(cfg, 40, seed=11)
    w, perm = synth.make_tasq(cfg)
    u, s16 = tq.tasq_transform(xk, w, perm, cfg.Tc)
    for t in range(cfg.T):
        s_exact = tq.tasq_sigma(xk[t], w[t])
        # the transform is scale-free: the RMS of u over heads and channels is sigma / fp16(sigma)
        rms = np.sqrt((u[t] ** 2).mean(axis=(1, 2)))
        np.testing.assert_allclose(rms, s_exact / s16[t], rtol=1e-13)
        assert np.all(np.abs(s16[t] / s_exact - 1) <= 2.0 ** -11)
        for h in range(cfg.H_kv):
            k_back = tq.tasq_inverse(u[t, :, h], w[t, h], perm[t // cfg.Tc, h], s16[t])
            np.testing.assert_allclose(k_back, xk[t, :, h], rtol=1e-14, atol=1e-14)


def test_zero_key_has_zero_sigma_and_zero_u():
    k = np.zeros((1, 2, 1, 8))
    k[0, 1, 0, 3] = 1.0
    u, s16 = tq.tasq_transform(k, np.ones((1, 1, 8)), np.array([[[0, 1, 2, 3]]]), Tc=1)
    assert s16[0, 0] == 0.0 and np.all(u[0, 0] == 0)
    assert s16[0, 1] == tq.f16_round(np.array([math.sqrt(1 / 8)]))[0]


# ---------------------------------------------------------------- decode
def _exact_tasq_case(rng, T, N, H, D):
    """Keys whose weighted values per (step, token) are fifteen-of-sixteen +-1
    and one +-7 per 16 entries (sigma = 2 exactly), with power-of-two weights:
    every u value is +-0.5 or +-3.5, exactly representable in fp16."""
    w = 2.0 ** rng.integers(-2, 3, size=(T, H, D)).astype(np.float64)
    y = rng.choice([-1.0, 1.0], size=(T, N, H * D))
    for t in range(T):
        for j in range(N):
            for blk in range(H * D // 16):
                y[t, j, 16 * blk + rng.integers(16)] *= 7
    k = y.reshape(T, N, H, D) / w[:, None]
    return k, w


def test_tasq_decode_lossless_equals_textbook_attention():
    # the codebook holds every coupled vector of u, so coding is lossless and
    # decode equals softmax attention over the RoPE'd original keys
    rng = np.random.default_rng(21)
    T, Tc, c, D, N, bits, H = 4, 4, 2, 16, 4, 8, 1
    k, w = _exact_tasq_case(rng, T, N, H, D)
    v = rng.standard_normal((T, N, H, D)).astype(np.float16).astype(np.float64)
    perm = np.array([[rng.permutation(D // 2)]])
    u, s16 = tq.tasq_transform(k, w, perm, Tc)
    assert np.all(s16 == 2.0)
    cb = np.zeros((1, H, 2, 256, c * Tc), dtype=np.float16)
    for kv, x in enumerate((u, v)):
        z = oracle.coupled_vectors(x[:, :, 0, :], Tc, c, 0).reshape(-1, c * Tc)
        fill = 100.0 + np.arange(256 - len(z))[:, None] + rng.random((256 - len(z), c * Tc))
        cb[0, 0, kv] = np.concatenate([z, fill]).astype(np.float16)
        assert np.array_equal(cb[0, 0, kv, :len(z)].astype(np.float64), z)
    P = 8
    bt = np.array([[0]], dtype=np.int32)
    slots = synth.slot_mapping_for(bt, 0, N, P)
    caches, ties, _ = oracle.build_index_cache(u, v, cb, Tc, c, bits, slots, 1, P)
    assert ties == 0
    for t in range(1, T + 1):
        q = rng.standard_normal((1, D))
        o, lse = tq.decode_attention_tasq(q, caches[0], bt[0], N, cb[0], t, Tc, c, bits, 1e4,
                                          w[t - 1], perm[0], s16[t - 1])
        krot = oracle.rope(k[t - 1, :, 0, :], np.arange(N), 1e4)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None], torch.tensor(krot)[None, None],
            torch.tensor(v[t - 1, :, 0, :])[None, None])[0, 0, 0].numpy()
        np.testing.assert_allclose(o[0], want, rtol=0, atol=1e-12)
        s = (krot @ q[0]) / math.sqrt(D)
        assert abs(lse[0] - (s.max() + math.log(np.exp(s - s.max()).sum()))) < 1e-12


def test_tasq_decode_scale_invariances():
    # sigma multiplies every rebuilt key; 1/w divides channel-wise; doubling
    # sigma (or halving w) is the same as doubling the softmax scale
    cfg = synth.config_by_name("tiny").replace(bits=8)
    rng = np.random.default_rng(22)
    N, P = 70, 64
    cache = rng.integers(0, 256, size=(2, 1, 2, P, cfg.row_bytes), dtype=np.uint8)
    bt = np.array([1, 0], dtype=np.int32)
    cbb = rng.standard_normal((1, 2, 256, cfg.G)).astype(np.float16)
    w, perm = synth.make_tasq(cfg)
    sig = synth.make_sigma(N, 5).astype(np.float64)
    q = rng.standard_normal((1, cfg.D))
    args = (cache, bt, N, cbb, 3, cfg.Tc, cfg.c, 8, 1e4)
    o1, l1 = tq.decode_attention_tasq(q, *args, w[2], perm[0], sig, sm_scale=0.2)
    o2, l2 = tq.decode_attention_tasq(q, *args, w[2], perm[0], 2 * sig, sm_scale=0.1)
    o3, l3 = tq.decode_attention_tasq(q, *args, 2 * w[2], perm[0], sig, sm_scale=0.4)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o3, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose([l2[0], l3[0]], [l1[0], l1[0]], rtol=0, atol=1e-13)


def test_tasq_decode_permutation_acts_on_pairs():
    # relabelling the u pairs (perm -> perm[s]) together with the u channels of
    # the codebook entries (pairs moved as units) leaves the output unchanged
    D, c, Tc, N, P = 32, 4, 2, 9, 16
    rng = np.random.default_rng(23)
    perm = rng.permutation(D // 2)
    w = rng.random((1, D)) + 0.5
    sig = synth.make_sigma(N, 7).astype(np.float64)
    q = rng.standard_normal((1, D))
    ng = D // c
    # a cache where token j's code of group g is codes[j, g] (row slot order applied)
    codes = rng.integers(0, 16, size=(N, ng))
    cb = rng.standard_normal((1, 2, 256, c * Tc)).astype(np.float16)
    # group-swap relabelling: u groups g <-> sg[g] (whole groups hold whole pairs)
    sg = rng.permutation(ng)
    perm2 = np.empty_like(perm)
    for g in range(ng):
        perm2[sg[g] * c // 2:(sg[g] + 1) * c // 2] = perm[g * c // 2:(g + 1) * c // 2]
    codes2 = np.empty_like(codes)
    codes2[:, sg] = codes
    def cache_of(cd):
        cache = np.zeros((1, 1, 2, P, ng), dtype=np.uint8)
        cache[0, 0, 0, :N] = oracle.groups_to_slots(cd)
        cache[0, 0, 1, :N] = oracle.groups_to_slots(codes)
        return cache
    bt = np.array([0], dtype=np.int32)
    o1, l1 = tq.decode_attention_tasq(q, cache_of(codes), bt, N, cb, 2, Tc, c, 8, 1e4, w, perm[None], sig)
    o2, l2 = tq.decode_attention_tasq(q, cache_of(codes2), bt, N, cb, 2, Tc, c, 8, 1e4, w, perm2[None], sig)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


@pytest.mark.parametrize("split", ["all_coded", "all_bf16", "mixed"])
def test_tasq_window_reduces_to_its_parts(split):
    # no bf16 tokens: the TaSQ decode; no coded tokens: the plain bf16-window
    # decode (the transform never touches bf16 keys); mixed: the coded part
    # through the TaSQ rebuild and the bf16 part as stored (lossless codebook
    # case -> textbook attention over the original keys)
    rng = np.random.default_rng(24)
    T, Tc, c, D, N, bits, H = 4, 4, 2, 16, 6, 8, 1
    k, w = _exact_tasq_case(rng, T, N, H, D)
    v = rng.standard_normal((T, N, H, D)).astype(np.float16).astype(np.float64)
    perm = np.array([[rng.permutation(D // 2)]])
    u, s16 = tq.tasq_transform(k, w, perm, Tc)
    cb = np.zeros((1, H, 2, 256, c * Tc), dtype=np.float16)
    for kv, x in enumerate((u, v)):
        z = oracle.coupled_vectors(x[:, :, 0, :], Tc, c, 0).reshape(-1, c * Tc)
        fill = 100.0 + np.arange(256 - len(z))[:, None] + rng.random((256 - len(z), c * Tc))
        cb[0, 0, kv] = np.concatenate([z, fill]).astype(np.float16)
    P = 8
    bt = np.array([[0]], dtype=np.int32)
    caches, _, _ = oracle.build_index_cache(u, v, cb, Tc, c, bits, synth.slot_mapping_for(bt, 0, N, P), 1, P)
    ns, ws = {"all_coded": (0, N), "all_bf16": (N, N), "mixed": (2, 4)}[split]
    t = 3
    q = rng.standard_normal((1, D))
    o, lse = tq.decode_attention_tasq_window(q, caches[0], bt[0], N, ns, ws, k[t - 1], v[t - 1], cb[0], t, Tc, c,
                                             bits, 1e4, w[t - 1], perm[0], s16[t - 1])
    if split == "all_coded":
        o2, l2 = tq.decode_attention_tasq(q, caches[0], bt[0], N, cb[0], t, Tc, c, bits, 1e4, w[t - 1], perm[0],
                                          s16[t - 1])
    elif split == "all_bf16":
        o2, l2 = oracle.decode_attention_window(q, caches[0], bt[0], N, N, N, k[t - 1], v[t - 1], cb[0], t, Tc,
                                                c, bits, 1e4)
    else:
        krot = oracle.rope(k[t - 1, :, 0, :], np.arange(N), 1e4)
        o2 = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None], torch.tensor(krot)[None, None],
            torch.tensor(v[t - 1, :, 0, :])[None, None])[0, 0].numpy()
        s = (krot @ q[0]) / math.sqrt(D)
        l2 = [s.max() + math.log(np.exp(s - s.max()).sum())]
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- k-means
def test_kmeans_hand_worked():
    z = np.array([[0.0], [1.0], [10.0], [11.0]])
    C1 = tq.kmeans_update(z, tq.kmeans_assign(z, np.array([[0.0], [1.0]])), np.array([[0.0], [1.0]]))
    np.testing.assert_allclose(C1, [[0.0], [22.0 / 3.0]], rtol=1e-15)
    C2, idx = tq.kmeans(z, np.array([[0.0], [1.0]]), iters=2)
    np.testing.assert_allclose(C2, [[0.5], [10.5]], rtol=1e-15)
    assert idx.tolist() == [0, 0, 1, 1]
    # a centre that gets no rows stays; ties go to the lowest index
    C, idx = tq.kmeans(z, np.array([[5.5], [5.5], [100.0]]), iters=1)
    assert idx.tolist() == [0, 0, 0, 0] and C[1, 0] == 5.5 and C[2, 0] == 100.0


def test_kmeans_matches_scipy_lloyd():
    rng = np.random.default_rng(31)
    z = np.concatenate([rng.standard_normal((300, 6)) + 3 * rng.standard_normal(6) for _ in range(5)])
    init = z[rng.choice(len(z), 12, replace=False)]
    C, idx = tq.kmeans(z, init, iters=7)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        Cs, idx_s = scipy.cluster.vq.kmeans2(z, init.copy(), iter=7, minit="matrix", missing="warn")
    np.testing.assert_allclose(C, Cs, rtol=1e-12, atol=1e-12)
    # SciPy returns the labels of its last assignment (before the last update);
    # the nearest-centre rule itself against SciPy's vq on the final centres
    np.testing.assert_array_equal(idx, scipy.cluster.vq.vq(z, Cs)[0])


def test_kmeans_objective_never_increases():
    rng = np.random.default_rng(32)
    z = rng.standard_normal((500, 4)) ** 3
    C = z[:16].copy()
    prev = np.inf
    for _ in range(8):
        idx = tq.kmeans_assign(z, C)
        err = ((z - C[idx]) ** 2).sum()
        assert err <= prev * (1 + 1e-12)
        prev = err
        C = tq.kmeans_update(z, idx, C)


def test_nmse_closed_form():
    assert tq.nmse(np.array([[3.0, 4.0]]), np.array([[0.0, 4.0]])) == pytest.approx(9 / 25, rel=1e-15)
    assert tq.nmse(np.ones((3, 2)), np.ones((3, 2))) == 0.0


def test_grouped_vectors_hand_worked():
    # Tc = 2 steps, N = 1 token, D = 4 channels, G = 4
    x = np.array([[[1, 2, 3, 4]], [[5, 6, 7, 8]]], dtype=np.float64)
    np.testing.assert_array_equal(tq.grouped_vectors(x, 4, "channel"), [[1, 2, 3, 4], [5, 6, 7, 8]])
    # loop grouping: c = 2 channels at 2 steps, coordinate i*Tc + m
    np.testing.assert_array_equal(tq.grouped_vectors(x, 4, "loop"), [[1, 5, 2, 6], [3, 7, 4, 8]])


# ---------------------------------------------------------------- Fig. 2c
def _fig2c_nmse(x, G, K, seed, iters=10):
    out = {}
    for grouping in ("channel", "loop"):
        z = tq.grouped_vectors(x, G, grouping)
        pick = np.random.default_rng(seed).choice(len(z), K, replace=False)
        C, idx = tq.kmeans(z, z[pick], iters)
        out[grouping] = tq.nmse(z, C[idx])
    return out


@pytest.mark.parametrize("bits,kv", [(8, 0), (8, 1), (4, 0)])
def test_fig2c_loop_grouping_lowers_kmeans_error(bits, kv):
    # the same bit width (one b-bit code per G = 16 coordinates) and one
    # codebook per cache under both groupings; only which coordinates share a
    # code changes.  On loop-correlated synthetic keys/values the loop-axis
    # grouping must reconstruct markedly better (the pages report roughly half
    # the error at 0.5 bit on their model).
    cfg = synth.config_by_name("layer1p4b")
    xk, xv = synth.make_kv(cfg, 1024, seed=41, heads=[3])
    x = (xk, xv)[kv][:, :, 0, :]
    r = _fig2c_nmse(x, 16, 1 << bits, seed=42)
    print(f"Fig. 2c check, {bits}-bit, {'KV'[kv]}: channel {r['channel']:.4f}, loop {r['loop']:.4f} "
          f"(ratio {r['loop'] / r['channel']:.3f})")
    assert r["loop"] < 0.8 * r["channel"]


def test_fig2c_control_without_loop_correlation():
    # with independent loop steps and no channel scales the two groupings see
    # identically distributed coordinates: no gain either way
    cfg = synth.config_by_name("layer1p4b").replace(rhos=(0.0, 0.0, 0.0), scale_sigma=0.0)
    xk, _ = synth.make_kv(cfg, 1024, seed=43, heads=[0])
    r = _fig2c_nmse(xk[:, :, 0, :], 16, 256, seed=44)
    assert abs(r["loop"] / r["channel"] - 1) < 0.05
