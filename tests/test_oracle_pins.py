"""Pins of the fp64 oracle against things other than itself.

Every pin here is independent of the oracle's own code: hand-worked fixtures
(tests/golden/), closed forms stated on the pages, exact rational brute force,
library routines (SciPy, PyTorch CPU) and invariants of the mathematics.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.cluster.vq
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- coupling
def test_coupling_hand_worked():
    g = _golden("coupling_tiny.json")
    for case in g["cases"]:
        x = np.array(case["x"], dtype=np.float64)
        z = oracle.coupled_vectors(x, g["Tc"], g["c"], case["beta"])
        np.testing.assert_array_equal(z, np.array(case["z"], dtype=np.float64))


def test_loop_slices_hand_worked():
    g = _golden("coupling_tiny.json")
    s = g["slices"]
    E = np.array([s["entry"]], dtype=np.float64)
    np.testing.assert_array_equal(oracle.loop_slice(E, g["Tc"], g["c"], 0)[0], s["slice0"])
    np.testing.assert_array_equal(oracle.loop_slice(E, g["Tc"], g["c"], 1)[0], s["slice1"])


def test_slices_are_a_permutation_of_each_entry():
    rng = np.random.default_rng(5)
    for Tc, c in [(4, 4), (4, 8), (2, 2), (1, 4)]:
        E = rng.standard_normal((7, Tc * c))
        cat = np.concatenate([oracle.loop_slice(E, Tc, c, m) for m in range(Tc)], axis=1)
        np.testing.assert_array_equal(np.sort(cat, axis=1), np.sort(E, axis=1))


def test_codebook_holding_the_data_round_trips_exactly():
    # a codebook that contains every coupled vector of the data encodes each
    # vector to itself, and rebuilding loop step t returns x^(t) bit-exactly
    rng = np.random.default_rng(1)
    T, Tc, c, D, N = 8, 4, 2, 16, 5
    x = rng.standard_normal((T, N, D))
    for beta in range(T // Tc):
        z = oracle.coupled_vectors(x, Tc, c, beta).reshape(-1, c * Tc)
        E = np.concatenate([z[::-1], rng.standard_normal((3, c * Tc)) + 50.0])
        idx, res = oracle.encode_stream(x, E, Tc, c, beta)
        assert (res.d1 == 0).all()
        for m in range(Tc):
            xr = oracle.rebuild(idx, E, Tc, c, m)
            np.testing.assert_array_equal(xr, x[beta * Tc + m])


# ---------------------------------------------------------------- argmin
def _exact_argmin(z, E):
    zq = [[Fraction(float(v)) for v in row] for row in z]
    Eq = [[Fraction(float(v)) for v in row] for row in E]
    out = []
    for row in zq:
        d = [sum((a - b) ** 2 for a, b in zip(row, e)) for e in Eq]
        best = min(d)
        out.append(d.index(best))  # lowest index among exact ties
    return np.array(out)


def test_argmin_matches_exact_rational_bruteforce():
    cfg = synth.config_by_name("tiny")
    xk, _ = synth.make_kv(cfg, 64)
    cb = synth.make_codebooks(cfg)
    z = oracle.coupled_vectors(xk[:, :, 0, :], cfg.Tc, cfg.c, 0).reshape(-1, cfg.G)[:512]
    E = cb[0, 0, 0].astype(np.float64)
    want = _exact_argmin(z, E)
    for method in ("direct", "gemm"):
        res = oracle.nearest_entry(z, E, method=method)
        np.testing.assert_array_equal(res.idx, want)


def test_argmin_exact_ties_take_lowest_index():
    E = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0], [-1.0, 0.0]])
    z = np.array([[1.0, 0.0],      # equal to entries 0 and 2 -> 0
                  [0.5, 0.5],      # equidistant from 0, 1 and 2 -> 0
                  [-0.5, 0.5],     # equidistant from 1 and 3 -> 1
                  [-2.0, 0.0]])    # nearest 3
    want = _exact_argmin(z, E)
    np.testing.assert_array_equal(want, [0, 0, 1, 3])
    for method in ("direct", "gemm"):
        res = oracle.nearest_entry(z, E, method=method)
        np.testing.assert_array_equal(res.idx, want)
        assert res.near_tie[:3].all() and not res.near_tie[3]


def test_per_step_coding_is_library_vq():
    # Tc = 1 is ordinary vector quantisation of contiguous c-channel
    # sub-vectors (the per-step baseline runs on the same kernel); SciPy's vq
    # assigns each observation to its nearest code.
    rng = np.random.default_rng(3)
    T, N, D, c = 2, 300, 32, 4
    x = rng.standard_normal((T, N, D))
    E = rng.standard_normal((64, c))
    for beta in range(T):
        idx, _ = oracle.encode_stream(x, E, 1, c, beta)
        codes, _ = scipy.cluster.vq.vq(x[beta].reshape(N * D // c, c), E)
        np.testing.assert_array_equal(idx.reshape(-1), codes)


def test_coupled_argmin_is_library_vq():
    cfg = synth.config_by_name("layer1p4b")
    xk, xv = synth.make_kv(cfg, 40, heads=[3])
    cb = synth.make_codebooks(cfg.replace(n_calib=64))
    for kv, x in enumerate((xk, xv)):
        z = oracle.coupled_vectors(x[:, :, 0, :], cfg.Tc, cfg.c, 0).reshape(-1, cfg.G)
        E = cb[0, 3, kv].astype(np.float64)
        codes, _ = scipy.cluster.vq.vq(z, E)
        for method in ("direct", "gemm"):
            np.testing.assert_array_equal(oracle.nearest_entry(z, E, method=method).idx, codes)


def test_accepts_near_tied_alternatives_only():
    E = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 3.0]])
    z = np.array([[0.5, 0.0], [0.1, 0.0]])
    res = oracle.nearest_entry(z, E)
    assert list(res.idx) == [0, 0]
    ok = oracle.accepts(z, E, res, np.array([1, 1]))
    assert list(ok) == [True, False]


# ---------------------------------------------------------------- index rows
def test_pack_4bit_hand_worked():
    g = _golden("pack_4bit.json")
    idx = np.array(g["indices"])
    rows = oracle.pack_rows(idx, 4)
    np.testing.assert_array_equal(rows, np.array(g["bytes"], dtype=np.uint8))
    np.testing.assert_array_equal(oracle.unpack_rows(rows, 4, idx.shape[1]), idx)


def test_pack_round_trip_8bit_and_4bit():
    rng = np.random.default_rng(2)
    for bits, ng in [(8, 32), (8, 16), (4, 32)]:
        idx = rng.integers(0, 1 << bits, size=(50, ng))
        rows = oracle.pack_rows(idx, bits)
        assert rows.shape == (50, ng * bits // 8)
        np.testing.assert_array_equal(oracle.unpack_rows(rows, bits, ng), idx)


def test_paged_scatter_gather_hand_worked():
    # explicit byte positions worked out by hand from the page / head / K|V /
    # offset strides, so a convention shared by scatter and gather (a swapped
    # axis, a wrong page lookup) cannot pass by round-tripping
    g = _golden("paged_rows.json")
    cache = np.zeros(g["shape"], dtype=np.uint8)
    for w in g["writes"]:
        oracle.scatter_rows(cache, np.array(w["rows"], np.uint8), np.array(w["slots"]), w["h"], w["kv"])
    want = np.zeros(cache.size, dtype=np.uint8)
    for off, val in g["nonzero_bytes"]:
        want[off] = val
    np.testing.assert_array_equal(cache.reshape(-1), want)
    for gg in g["gathers"]:
        got = oracle.gather_rows(cache, np.array(gg["block_table"]), gg["n"], gg["h"], gg["kv"])
        np.testing.assert_array_equal(got, np.array(gg["rows"], np.uint8))
    for gg in g["gathers_at"]:
        got = oracle.gather_rows_at(cache, np.array(gg["block_table"]), np.array(gg["pos"]), gg["h"], gg["kv"])
        np.testing.assert_array_equal(got, np.array(gg["rows"], np.uint8))
    u = g["unpack_8bit"]
    np.testing.assert_array_equal(oracle.unpack_rows(np.array(u["rows"], np.uint8), 8, 4), np.array(u["codes"]))


def test_paged_scatter_gather_round_trip():
    cfg = synth.config_by_name("tiny").replace(page_size=8)
    lens = np.array([13, 30, 1])
    bt, npages = synth.make_block_table(cfg, lens)
    assert sorted(bt[0, :2].tolist() + bt[1, :4].tolist() + bt[2, :1].tolist()) == list(range(npages))
    cache = np.zeros((npages, 1, 2, 8, 5), dtype=np.uint8)
    rng = np.random.default_rng(0)
    rows = {}
    for b, n in enumerate(lens):
        rows[b] = rng.integers(0, 256, size=(n, 5), dtype=np.uint8)
        oracle.scatter_rows(cache, rows[b], synth.slot_mapping_for(bt, b, n, 8), 0, 1)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(oracle.gather_rows(cache, bt[b], n, 0, 1), rows[b])


def test_storage_identities():
    g = _golden("identities.json")
    for e in g["bits_per_element"]:
        assert oracle.bits_per_element(e["bits"], e["G"]) == e["value"]
    assert 16 / oracle.bits_per_element(8, 16) == g["ratio_vs_bf16_at_half_bit"]["value"]
    for e in g["decode_bytes_fewer_than_bf16"]:
        D, c, bits = e["D"], e["c"], e["bits"]
        idx = np.zeros((1, D // c), dtype=np.int64)
        row_bytes = oracle.pack_rows(idx, bits).nbytes  # one K row; V is the same
        bf16_bytes = D * 2
        assert bf16_bytes // row_bytes == e["value"]
    w = g["worked_index_count"]
    c = w["G"] // w["Tc"]
    z = oracle.coupled_vectors(np.zeros((w["T"], 1, w["D"])), w["Tc"], c, 0)
    assert z.shape[1] * (w["T"] // w["Tc"]) == w["indices_per_token_head"]
    # per-step coding of the same token-head: D/G codes per step, T steps
    assert (w["D"] // w["G"]) * w["T"] == w["indices_per_token_head"]


# ---------------------------------------------------------------- RoPE
def test_rope_frequencies_closed_form():
    np.testing.assert_allclose(oracle.rope_frequencies(4, 10000.0), [1.0, 0.01], rtol=0, atol=1e-15)
    th = oracle.rope_frequencies(128, 10000.0)
    assert th[0] == 1.0 and abs(th[32] - 0.01) < 1e-15 and np.all(np.diff(th) < 0)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(4)
    D, N = 64, 40
    x = rng.standard_normal((N, D))
    pos = rng.integers(0, 65536, size=N)
    y = oracle.rope(x, pos, 10000.0)
    theta = oracle.rope_frequencies(D, 10000.0)
    zc = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos[:, None] * theta[None, :])
    np.testing.assert_allclose(y[:, :D // 2], zc.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[:, D // 2:], zc.imag, rtol=0, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(6)
    D = 128
    k = rng.standard_normal((10, D))
    q = rng.standard_normal((10, D))
    np.testing.assert_array_equal(oracle.rope(k, np.zeros(10), 1e4), k)
    pos = rng.integers(0, 40000, size=10)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(k, pos, 1e4), axis=1),
                               np.linalg.norm(k, axis=1), rtol=1e-13)
    # <RoPE(q, p), RoPE(k, p')> depends only on p - p'
    a = (oracle.rope(q, pos + 1000, 1e4) * oracle.rope(k, pos, 1e4)).sum(1)
    b = (oracle.rope(q, np.full(10, 1000), 1e4) * k).sum(1)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_rope_table_layout():
    t = oracle.rope_table(3, 4, 10000.0)
    np.testing.assert_allclose(t[1], [math.cos(1.0), math.cos(0.01), math.sin(1.0), math.sin(0.01)],
                               rtol=0, atol=1e-15)
    np.testing.assert_array_equal(t[0], [1, 1, 0, 0])


# ---------------------------------------------------------------- attention
def test_attention_matches_library_sdpa_and_logsumexp():
    rng = np.random.default_rng(7)
    N, D = 77, 32
    q = rng.standard_normal(D)
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    o, lse = oracle.attention(q, k, v, 0.3)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None, :], torch.tensor(k)[None, None],
        torch.tensor(v)[None, None], scale=0.3)[0, 0, 0].numpy()
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(0.3 * k @ q), rtol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    D = 16
    o, lse = oracle.attention(np.ones(D), np.zeros((0, D)), np.zeros((0, D)), 1.0)
    assert np.all(o == 0) and lse == -np.inf
    v = rng.standard_normal((1, D))
    o, lse = oracle.attention(rng.standard_normal(D), rng.standard_normal((1, D)), v, 1.0)
    np.testing.assert_array_equal(o, v[0])
    v = rng.standard_normal((9, D))
    o, lse = oracle.attention(np.zeros(D), rng.standard_normal((9, D)), v, 1.0)
    np.testing.assert_allclose(o, v.mean(0), rtol=0, atol=1e-14)
    assert abs(lse - math.log(9)) < 1e-14


def _fp16_exact(a):
    return a.astype(np.float16).astype(np.float64)


def test_decode_equals_dense_attention_when_codebook_holds_the_data():
    # D = 64, c = 2, Tc = 4, 8-bit codes, N = 4 tokens: 128 data sub-vectors
    # per (head, K|V) plus 128 distinct far-away fillers.  Encoding is then
    # lossless and quantised decode attention equals ordinary attention over
    # the RoPE'd original keys and the original values at every loop step.
    rng = np.random.default_rng(9)
    T, Tc, c, D, N, bits, H = 4, 4, 2, 64, 4, 8, 1
    xk = _fp16_exact(rng.standard_normal((T, N, H, D)))
    xv = _fp16_exact(rng.standard_normal((T, N, H, D)))
    cb = np.zeros((1, H, 2, 256, c * Tc), dtype=np.float16)
    for kv, x in enumerate((xk, xv)):
        z = oracle.coupled_vectors(x[:, :, 0, :], Tc, c, 0).reshape(-1, c * Tc)
        fill = 100.0 + np.arange(128)[:, None] + rng.random((128, c * Tc))
        E = np.concatenate([fill[:64], z, fill[64:]])
        cb[0, 0, kv] = E.astype(np.float16)
    P = 8
    bt = np.array([[0]], dtype=np.int32)
    slots = synth.slot_mapping_for(bt, 0, N, P)
    caches, ties, _ = oracle.build_index_cache(xk, xv, cb, Tc, c, bits, slots, 1, P)
    assert ties == 0
    for t in range(1, T + 1):
        q = rng.standard_normal((1, D))
        o, lse = oracle.decode_attention(q, caches[0], bt[0], N, cb[0], t, Tc, c, bits, 1e4)
        krot = oracle.rope(xk[t - 1, :, 0, :], np.arange(N), 1e4)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None], torch.tensor(krot)[None, None],
            torch.tensor(xv[t - 1, :, 0, :])[None, None])[0, 0, 0].numpy()
        np.testing.assert_allclose(o[0], want, rtol=0, atol=1e-12)


def test_gqa_heads_read_their_kv_head():
    rng = np.random.default_rng(10)
    H_kv, grp, D, c, Tc, bits, N, P = 2, 3, 32, 4, 4, 8, 20, 8
    cache = rng.integers(0, 256, size=(3, H_kv, 2, P, D // c), dtype=np.uint8)
    bt = np.array([2, 0, 1], dtype=np.int32)
    cbb = rng.standard_normal((H_kv, 2, 256, c * Tc)).astype(np.float16)
    q = rng.standard_normal((H_kv * grp, D))
    o, lse = oracle.decode_attention(q, cache, bt, N, cbb, 2, Tc, c, bits, 1e4)
    # swapping the two KV heads' data swaps which query group sees what
    o2, _ = oracle.decode_attention(q[[3, 4, 5, 0, 1, 2]], cache[:, ::-1], bt, N, cbb[::-1], 2,
                                    Tc, c, bits, 1e4)
    np.testing.assert_allclose(o2, o[[3, 4, 5, 0, 1, 2]], rtol=0, atol=1e-13)


def test_row_order_hand_worked():
    g = _golden("row_order.json")
    for n, order in g["orders"].items():
        np.testing.assert_array_equal(oracle.row_group_order(int(n)), order)
    ex = g["example_4bit"]
    codes = np.array([ex["codes"]])
    rows = oracle.pack_rows(oracle.groups_to_slots(codes), 4)
    np.testing.assert_array_equal(rows[0], ex["bytes"])
    back = oracle.slots_to_groups(oracle.unpack_rows(rows, 4, codes.shape[1]))
    np.testing.assert_array_equal(back, codes)


# ---------------------------------------------------------------- bf16 sink and recent window
def _rope_complex(x, pos, base):
    # rotate-half RoPE written as a complex rotation (an independent form)
    D = x.shape[1]
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * np.asarray(pos)[:, None] * theta[None, :])
    return np.concatenate([z.real, z.imag], axis=1)


def _sdpa(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None, :], torch.tensor(k)[None, None],
        torch.tensor(v)[None, None])[0, 0, 0].numpy()


def _lossless_window_case(seed):
    # values on a 1/8 grid in [-4, 4): exact in bf16 and in fp16.  The
    # codebook of each (head, K|V) holds every coupled vector of the data plus
    # far-away fillers, so the codes rebuild the data exactly.
    rng = np.random.default_rng(seed)
    T, Tc, c, D, N, H, bits, P = 4, 4, 4, 32, 24, 2, 8, 8
    xk = rng.integers(-32, 32, size=(T, N, H, D)) / 8.0
    xv = rng.integers(-32, 32, size=(T, N, H, D)) / 8.0
    cb = np.zeros((1, H, 2, 256, c * Tc), dtype=np.float16)
    for h in range(H):
        for kv, x in enumerate((xk, xv)):
            z = oracle.coupled_vectors(x[:, :, h, :], Tc, c, 0).reshape(-1, c * Tc)
            fill = 100.0 + np.arange(256 - len(z))[:, None] + rng.random((256 - len(z), c * Tc))
            cb[0, h, kv] = np.concatenate([z, fill]).astype(np.float16)
    npg = N // P
    bt = rng.permutation(npg).astype(np.int32)[None, :]
    slots = synth.slot_mapping_for(bt, 0, N, P)
    caches, ties, _ = oracle.build_index_cache(xk, xv, cb, Tc, c, bits, slots, npg, P)
    assert ties == 0
    return dict(xk=xk, xv=xv, cb=cb, bt=bt, cache=caches[0], Tc=Tc, c=c, bits=bits, N=N, H=H, D=D, T=T)


@pytest.mark.parametrize("n_sink,win_start", [(0, 24), (8, 16), (0, 0), (24, 24), (8, 8), (16, 24)])
def test_window_lossless_cache_is_dense_rope_attention(n_sink, win_start):
    # whatever split of the positions into bf16 and codes, a lossless cache
    # gives ordinary attention over the rotated original keys
    g = _lossless_window_case(11)
    rng = np.random.default_rng(12)
    for t in range(1, g["T"] + 1):
        q = rng.standard_normal((g["H"], g["D"]))
        o, lse = oracle.decode_attention_window(q, g["cache"], g["bt"][0], g["N"], n_sink, win_start,
                                                g["xk"][t - 1], g["xv"][t - 1], g["cb"][0], t, g["Tc"],
                                                g["c"], g["bits"], 1e4)
        for h in range(g["H"]):
            krot = _rope_complex(g["xk"][t - 1, :, h, :], np.arange(g["N"]), 1e4)
            want = _sdpa(q[h], krot, g["xv"][t - 1, :, h, :])
            np.testing.assert_allclose(o[h], want, rtol=0, atol=1e-12)
            s = (krot @ q[h]) / np.sqrt(g["D"])
            assert abs(lse[h] - scipy.special.logsumexp(s)) < 1e-12


def test_window_reads_bf16_rows_only_at_bf16_positions():
    # garbage codes under bf16 positions and garbage bf16 rows under coded
    # positions change nothing; the bf16 rows that are read are used as given
    g = _lossless_window_case(13)
    rng = np.random.default_rng(14)
    n_sink, win_start, t = 8, 16, 3
    N, H, D = g["N"], g["H"], g["D"]
    q = rng.standard_normal((H, D))
    cache = g["cache"].copy()
    bpos = np.r_[0:n_sink, win_start:N]
    P = cache.shape[3]
    for p in bpos:
        cache[g["bt"][0, p // P], :, :, p % P, :] = rng.integers(0, 256, size=cache.shape[-1])
    kb = g["xk"][t - 1].copy()
    vb = g["xv"][t - 1].copy()
    kb[n_sink:win_start] = rng.standard_normal((win_start - n_sink, H, D))
    vb[n_sink:win_start] = rng.standard_normal((win_start - n_sink, H, D))
    delta = rng.standard_normal((len(bpos), H, D))
    kb[bpos] += delta
    o, _ = oracle.decode_attention_window(q, cache, g["bt"][0], N, n_sink, win_start, kb, vb, g["cb"][0],
                                          t, g["Tc"], g["c"], g["bits"], 1e4)
    for h in range(H):
        k = g["xk"][t - 1, :, h, :].copy()
        k[bpos] += delta[:, h, :]
        want = _sdpa(q[h], _rope_complex(k, np.arange(N), 1e4), g["xv"][t - 1, :, h, :])
        np.testing.assert_allclose(o[h], want, rtol=0, atol=1e-12)


def test_window_without_bf16_tokens_is_the_quantised_decode():
    rng = np.random.default_rng(15)
    H_kv, grp, D, c, Tc, bits, N, P = 2, 2, 32, 4, 4, 8, 40, 8
    cache = rng.integers(0, 256, size=(5, H_kv, 2, P, D // c), dtype=np.uint8)
    bt = np.array([3, 1, 4, 0, 2], dtype=np.int32)
    cbb = rng.standard_normal((H_kv, 2, 256, c * Tc)).astype(np.float16)
    q = rng.standard_normal((H_kv * grp, D))
    junk = rng.standard_normal((N, H_kv, D))
    o, lse = oracle.decode_attention_window(q, cache, bt, N, 0, N, junk, junk, cbb, 2, Tc, c, bits, 1e4)
    o2, lse2 = oracle.decode_attention(q, cache, bt, N, cbb, 2, Tc, c, bits, 1e4)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


# ---------------------------------------------------------------- one codebook per channel group
def _pg_case(seed, H=2):
    rng = np.random.default_rng(seed)
    T, Tc, c, D, N, bits = 4, 4, 4, 32, 40, 8
    ng = D // c
    xk = rng.standard_normal((T, N, H, D))
    xv = rng.standard_normal((T, N, H, D))
    shared = rng.standard_normal((1, H, 2, 256, c * Tc)).astype(np.float16)
    return rng, xk, xv, shared, T, Tc, c, D, N, bits, ng


def test_per_group_codebooks_all_equal_reduce_to_the_shared_one():
    rng, xk, xv, shared, T, Tc, c, D, N, bits, ng = _pg_case(21)
    pg = np.broadcast_to(shared[:, :, :, None], (1, 2, 2, ng) + shared.shape[3:]).copy()
    P = 8
    bt = rng.permutation(N // P).astype(np.int32)[None, :]
    slots = synth.slot_mapping_for(bt, 0, N, P)
    a, _, _ = oracle.build_index_cache(xk, xv, shared, Tc, c, bits, slots, N // P, P)
    b, _, _ = oracle.build_index_cache(xk, xv, pg, Tc, c, bits, slots, N // P, P)
    np.testing.assert_array_equal(a, b)
    q = rng.standard_normal((2, D))
    o1, l1 = oracle.decode_attention(q, a[0], bt[0], N, shared[0], 2, Tc, c, bits, 1e4)
    o2, l2 = oracle.decode_attention(q, b[0], bt[0], N, pg[0], 2, Tc, c, bits, 1e4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_per_group_codebooks_follow_a_per_group_entry_permutation():
    # group g's codebook is the shared one with its entries reordered by pi_g:
    # every code becomes pi_g^-1 of the shared code, and the rebuilt data match
    rng, xk, xv, shared, T, Tc, c, D, N, bits, ng = _pg_case(22, H=1)
    perms = [rng.permutation(256) for _ in range(ng)]
    pg = np.stack([shared[0, 0, 0][p] for p in perms])                       # [ng, K, G]
    x = xk[:, :, 0, :]
    i_sh, _ = oracle.encode_stream(x, shared[0, 0, 0], Tc, c, 0)
    i_pg, _ = oracle.encode_stream(x, pg, Tc, c, 0)
    for g in range(ng):
        inv = np.argsort(perms[g])
        np.testing.assert_array_equal(i_pg[:, g], inv[i_sh[:, g]])
    for m in range(Tc):
        np.testing.assert_array_equal(oracle.rebuild(i_pg, pg, Tc, c, m), oracle.rebuild(i_sh, shared[0, 0, 0], Tc, c, m))


def test_per_group_lossless_codebooks_give_dense_attention():
    # group g's codebook holds every coupled vector of group g: coding is
    # lossless and decode equals attention over the rotated original keys
    rng = np.random.default_rng(23)
    T, Tc, c, D, N, bits, H = 4, 4, 4, 32, 40, 8, 1
    ng = D // c
    xk = rng.integers(-32, 32, size=(T, N, H, D)) / 8.0
    xv = rng.integers(-32, 32, size=(T, N, H, D)) / 8.0
    cb = np.zeros((1, H, 2, ng, 256, c * Tc), dtype=np.float16)
    for kv, x in enumerate((xk, xv)):
        z = oracle.coupled_vectors(x[:, :, 0, :], Tc, c, 0)                  # [N, ng, G]
        for g in range(ng):
            fill = 100.0 + np.arange(256 - N)[:, None] + rng.random((256 - N, c * Tc))
            cb[0, 0, kv, g] = np.concatenate([z[:, g, :], fill]).astype(np.float16)
    P = 8
    bt = rng.permutation(N // P).astype(np.int32)[None, :]
    slots = synth.slot_mapping_for(bt, 0, N, P)
    caches, ties, _ = oracle.build_index_cache(xk, xv, cb, Tc, c, bits, slots, N // P, P)
    assert ties == 0
    for t in range(1, T + 1):
        q = rng.standard_normal((1, D))
        o, lse = oracle.decode_attention(q, caches[0], bt[0], N, cb[0], t, Tc, c, bits, 1e4)
        krot = _rope_complex(xk[t - 1, :, 0, :], np.arange(N), 1e4)
        np.testing.assert_allclose(o[0], _sdpa(q[0], krot, xv[t - 1, :, 0, :]), rtol=0, atol=1e-12)
