"""Plain fp64 CPU oracle for the TaSQ+LoopVQ key path and for plain k-means.

TEST INFRASTRUCTURE ONLY.  Only the tests, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import or call this module.  It shares no
code with the HIP library and imports nothing from it.

Sources ("the pages"):
  [P1] "LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers"
       (hub.valency.io/works/W_7srt5hed_v1): appendix "Orthogonal application
       with TaSQ" (subsections "Formulation", "Grouping under loop coupling",
       "Calibration and bitwidth"; eqs. (10)-(12) were lost in extraction and
       are rebuilt from the prose), and section "Redundancy along the loop
       axis" with Fig. 2c (k-means under two groupings).
  [P2] The jaehun.me summary post of the same paper, section 3.3 "Combining
       with TaSQ" and its restatement of Fig. 2c.

Readings taken where the pages are silent:
  * eq. (10): u = P(w (.) k / sigma_j): the pre-RoPE key of loop step t, head
    h and token j is weighted channel-wise by w^(t)_h, divided by the token's
    scale sigma^(t)_j and permuted by P_{beta,h} of its block;
  * sigma^(t)_j = RMS of w (.) k over all heads and channels of token j at
    step t (P1 "Formulation"), stored in fp16 (P1 "Calibration and
    bitwidth" counts it as 16/(H*D) bits of overhead per key element).  The
    fp16-rounded value (round
    to nearest even) is the one used on both sides: to form u and to rebuild
    the key.  A token whose fp16 sigma is 0 gets u = 0;
  * P keeps each RoPE pair {f, f + D/2} together and places whole pairs in a
    code (P1 "Grouping under loop coupling").  It is given as a pair
    permutation perm[p] (p < D/2): u channel 2p holds channel perm[p] and u
    channel 2p+1 holds channel perm[p] + D/2.  The coupled vectors (eq. (11))
    are then built from u exactly as from k (group g = u channels
    [g*c, (g+1)*c)), so a code covers c/2 whole RoPE pairs at Tc loop steps;
  * at decode the key is rebuilt in u space from the slice of its step, then
    k_hat = sigma * P^-1(u_hat) / w, then RoPE at the token's position;
  * Fig. 2c compares the groupings at an equal number of codebooks, read as one codebook per
    (head, K|V, block) under both groupings: the channel grouping codes G
    channels of each of the Tc steps with one codebook shared by the steps,
    the loop grouping codes G/Tc channels at the Tc steps (eq. (4)).  k-means
    is Lloyd's algorithm from given initial centres; an empty centre stays
    where it is; ties go to the lowest index.

Parity pins: tests/test_oracle_tasq.py checks every function here against
closed forms, exactly representable worked cases, a library k-means (scipy)
and textbook attention.  None is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .loopvq_ref import (attention, gather_rows, gather_rows_at, rebuild, rope, slots_to_groups,
                         unpack_rows, coupled_vectors)

# relative half-width of the band around an fp16 rounding midpoint inside
# which an fp32 evaluation of sigma may round to the other neighbour
SIGMA_MIDPOINT_REL = 2e-6


# --------------------------------------------------------------------------
# fp16 rounding of sigma  [P1 appendix "Calibration and bitwidth": sigma is
#                          kept in fp16]
# --------------------------------------------------------------------------
def f16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest fp16 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def f16_near_midpoint(x: np.ndarray, rel: float = SIGMA_MIDPOINT_REL) -> np.ndarray:
    """True where x lies within rel*|x| of a midpoint between two fp16 values,
    so that a slightly perturbed x may round to either neighbour."""
    x = np.asarray(x, dtype=np.float64)
    r = f16_round(x)
    lo = np.where(r <= x, r, np.nextafter(r.astype(np.float16), np.float16(-np.inf)).astype(np.float64))
    hi = np.where(r > x, r, np.nextafter(r.astype(np.float16), np.float16(np.inf)).astype(np.float64))
    mid = 0.5 * (lo + hi)
    return np.abs(x - mid) <= rel * np.abs(x)


# --------------------------------------------------------------------------
# the TaSQ key transform  [P1 appendix "Orthogonal application with TaSQ",
#   "Formulation" (eq. (10)) and "Grouping under loop coupling"; P2 3.3]
# --------------------------------------------------------------------------
def tasq_sigma(k_step: np.ndarray, w_step: np.ndarray) -> np.ndarray:
    """sigma_j = sqrt(mean over heads h and channels i of (w[h, i] * k[j, h, i])^2).

    k_step [N, H, D] keys of one loop step, w_step [H, D]; float64 [N], exact
    up to fp64 rounding (not yet rounded to fp16).
    """
    y = np.asarray(k_step, dtype=np.float64) * np.asarray(w_step, dtype=np.float64)[None]
    return np.sqrt((y * y).mean(axis=(1, 2)))


def pair_source_channels(perm_h: np.ndarray, D: int) -> np.ndarray:
    """Channel of the key that each u channel holds: u[2p] <- perm[p],
    u[2p + 1] <- perm[p] + D/2 (a RoPE pair stays together)."""
    perm_h = np.asarray(perm_h, dtype=np.int64)
    assert perm_h.shape == (D // 2,) and np.array_equal(np.sort(perm_h), np.arange(D // 2))
    src = np.empty(D, dtype=np.int64)
    src[0::2] = perm_h
    src[1::2] = perm_h + D // 2
    return src


def tasq_transform(k: np.ndarray, w: np.ndarray, perm: np.ndarray, Tc: int):
    """u = P(w (.) k / sigma) for every loop step, token and head.

    k [T, N, H, D] pre-RoPE keys, w [T, H, D] channel weights, perm
    [T // Tc, H, D/2] pair permutations of each block.  Returns (u [T, N, H, D]
    float64, sigma16 [T, N] float64 holding the fp16 values).
    """
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, N, H, D = k.shape
    u = np.zeros((T, N, H, D))
    s16 = np.zeros((T, N))
    for t in range(T):
        beta = t // Tc
        s16[t] = f16_round(tasq_sigma(k[t], w[t]))
        nz = s16[t] > 0
        y = k[t] * w[t][None]                                  # [N, H, D]
        for h in range(H):
            src = pair_source_channels(perm[beta, h], D)
            u[t, nz, h, :] = y[nz, h][:, src] / s16[t, nz, None]
    return u, s16


def tasq_inverse(u_hat: np.ndarray, w_h: np.ndarray, perm_h: np.ndarray, sigma16: np.ndarray) -> np.ndarray:
    """Key rebuilt from u space: k_hat[:, src[c]] = sigma * u_hat[:, c] / w[src[c]].

    u_hat [N, D] of one head and step, w_h [D], perm_h [D/2], sigma16 [N].
    """
    u_hat = np.asarray(u_hat, dtype=np.float64)
    N, D = u_hat.shape
    src = pair_source_channels(perm_h, D)
    w_h = np.asarray(w_h, dtype=np.float64)
    k = np.empty((N, D))
    k[:, src] = np.asarray(sigma16, dtype=np.float64)[:, None] * u_hat / w_h[src][None, :]
    return k


def decode_attention_tasq(q: np.ndarray, cache_block: np.ndarray, block_table_row: np.ndarray,
                          n: int, cb_block: np.ndarray, t: int, Tc: int, c: int, bits: int,
                          base: float, w_t: np.ndarray, perm_b: np.ndarray, sigma_pos: np.ndarray,
                          sm_scale: float | None = None):
    """Quantised decode attention at loop step t (1-based) with TaSQ-coded keys.

    As loopvq_ref.decode_attention, except that the key codes index u-space
    entries: the key of position j is tasq_inverse(rebuilt u, w_t[h],
    perm_b[h], sigma_pos[j]) before RoPE.  Values are coded as usual.
    w_t [H_kv, D] weights of step t, perm_b [H_kv, D/2] of block (t-1)//Tc,
    sigma_pos [n] fp16 scales of the request's positions at step t.
    Returns (o [H_q, D], lse [H_q]).
    """
    q = np.asarray(q, dtype=np.float64)
    H_q, D = q.shape
    H_kv = cache_block.shape[1]
    grp = H_q // H_kv
    m = (t - 1) % Tc
    sm_scale = 1.0 / np.sqrt(D) if sm_scale is None else sm_scale
    ng = D // c
    pos = np.arange(n)
    sig = np.asarray(sigma_pos, dtype=np.float64)[:n]
    o = np.zeros((H_q, D))
    lse = np.zeros(H_q)
    for h in range(H_kv):
        ki = slots_to_groups(unpack_rows(gather_rows(cache_block, block_table_row, n, h, 0), bits, ng))
        vi = slots_to_groups(unpack_rows(gather_rows(cache_block, block_table_row, n, h, 1), bits, ng))
        uhat = rebuild(ki, cb_block[h, 0], Tc, c, m)
        khat = tasq_inverse(uhat, w_t[h], perm_b[h], sig)
        vhat = rebuild(vi, cb_block[h, 1], Tc, c, m)
        krot = rope(khat, pos, base)
        for j in range(h * grp, (h + 1) * grp):
            o[j], lse[j] = attention(q[j], krot, vhat, sm_scale)
    return o, lse


def decode_attention_tasq_window(q: np.ndarray, cache_block: np.ndarray, block_table_row: np.ndarray,
                                 n: int, n_sink: int, win_start: int, k_bf: np.ndarray, v_bf: np.ndarray,
                                 cb_block: np.ndarray, t: int, Tc: int, c: int, bits: int, base: float,
                                 w_t: np.ndarray, perm_b: np.ndarray, sigma_pos: np.ndarray,
                                 sm_scale: float | None = None):
    """Decode attention over a cache mixing bf16 tokens and TaSQ-coded keys.

    As loopvq_ref.decode_attention_window [P1 section "System implementation":
    bf16 sink and recent window, codes elsewhere, one softmax over all tokens],
    except that the coded positions [n_sink, win_start) rebuild their keys as in
    decode_attention_tasq.  The bf16 tokens hold plain pre-RoPE keys (the
    transform applies only when a token is coded).  sigma_pos [n] is read only
    at coded positions.  Returns (o [H_q, D], lse [H_q]).
    """
    q = np.asarray(q, dtype=np.float64)
    H_q, D = q.shape
    H_kv = cache_block.shape[1]
    grp = H_q // H_kv
    assert 0 <= n_sink <= win_start <= n
    m = (t - 1) % Tc
    sm_scale = 1.0 / np.sqrt(D) if sm_scale is None else sm_scale
    ng = D // c
    qpos = np.arange(n_sink, win_start)
    bpos = np.concatenate([np.arange(n_sink), np.arange(win_start, n)]).astype(np.int64)
    k_bf = np.asarray(k_bf, dtype=np.float64)
    v_bf = np.asarray(v_bf, dtype=np.float64)
    sig = np.asarray(sigma_pos, dtype=np.float64)
    o = np.zeros((H_q, D))
    lse = np.zeros(H_q)
    for h in range(H_kv):
        k = np.empty((n, D))
        v = np.empty((n, D))
        ki = slots_to_groups(unpack_rows(gather_rows_at(cache_block, block_table_row, qpos, h, 0), bits, ng))
        vi = slots_to_groups(unpack_rows(gather_rows_at(cache_block, block_table_row, qpos, h, 1), bits, ng))
        k[qpos] = tasq_inverse(rebuild(ki, cb_block[h, 0], Tc, c, m), w_t[h], perm_b[h], sig[qpos])
        v[qpos] = rebuild(vi, cb_block[h, 1], Tc, c, m)
        k[bpos] = k_bf[bpos, h]
        v[bpos] = v_bf[bpos, h]
        krot = rope(k, np.arange(n), base)
        for j in range(h * grp, (h + 1) * grp):
            o[j], lse[j] = attention(q[j], krot, v, sm_scale)
    return o, lse


# --------------------------------------------------------------------------
# plain k-means and the two groupings of Fig. 2c  [P1 section "Redundancy
#   along the loop axis", Fig. 2c; P2 restatement of Fig. 2c]
# --------------------------------------------------------------------------
def kmeans_assign(z: np.ndarray, centers: np.ndarray) -> np.ndarray:
    """Index of the nearest centre of every row (squared L2, lowest index on ties)."""
    z = np.asarray(z, dtype=np.float64)
    C = np.asarray(centers, dtype=np.float64)
    d = (z * z).sum(1)[:, None] - 2.0 * (z @ C.T) + (C * C).sum(1)[None, :]
    return np.argmin(d, axis=1)


def kmeans_update(z: np.ndarray, idx: np.ndarray, centers: np.ndarray) -> np.ndarray:
    """Each centre moves to the mean of the rows assigned to it; a centre with
    no rows stays where it is."""
    z = np.asarray(z, dtype=np.float64)
    K = centers.shape[0]
    sums = np.zeros((K, z.shape[1]))
    np.add.at(sums, idx, z)
    cnt = np.bincount(idx, minlength=K)
    new = np.array(centers, dtype=np.float64, copy=True)
    nz = cnt > 0
    new[nz] = sums[nz] / cnt[nz, None]
    return new


def kmeans(z: np.ndarray, init: np.ndarray, iters: int):
    """Lloyd's algorithm: `iters` rounds of assignment then update, from the
    given initial centres.  Returns (centres, final assignment)."""
    C = np.asarray(init, dtype=np.float64)
    for _ in range(iters):
        C = kmeans_update(z, kmeans_assign(z, C), C)
    return C, kmeans_assign(z, C)


def nmse(z: np.ndarray, z_hat: np.ndarray) -> float:
    """Normalised reconstruction error sum ||z - z_hat||^2 / sum ||z||^2."""
    z = np.asarray(z, dtype=np.float64)
    e = z - np.asarray(z_hat, dtype=np.float64)
    return float((e * e).sum() / (z * z).sum())


def grouped_vectors(x: np.ndarray, G: int, grouping: str) -> np.ndarray:
    """The vectors that share a code under one grouping of Fig. 2c.

    x [Tc, N, D]: the Tc loop steps of one block of one (head, K|V) cache.
    "loop":    G/Tc channels at each of the Tc steps, the coupled vectors of
               eq. (4) -> [N * D*Tc/G, G];
    "channel": G contiguous channels of one step, every step -> [Tc * N * D/G, G].
    """
    x = np.asarray(x, dtype=np.float64)
    Tc, N, D = x.shape
    if grouping == "loop":
        assert G % Tc == 0
        return coupled_vectors(x, Tc, G // Tc, 0).reshape(-1, G)
    if grouping == "channel":
        assert D % G == 0
        return x.reshape(Tc * N * (D // G), G)
    raise ValueError(grouping)
