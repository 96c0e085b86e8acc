"""Plain fp64 CPU oracle for LoopVQ encoding and quantised decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import or call this module.  It shares no
code with the HIP library (no kernels, headers, helpers, tables or constant
generators) and imports nothing from it; the library never imports this.

Sources ("the pages"):
  [P1] "LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers"
       (hub.valency.io/works/W_7srt5hed_v1) - the authority on the method.
  [P2] The jaehun.me summary post of the same paper (paper-2611-05304v1), which
       states eq. (2) in full and restates the coupled-vector layout.
P1's display equations were lost when the page was extracted; where this
module rebuilds one from the prose it says which sentence it follows.

Readings taken where the pages are silent:
  * channel group g covers the contiguous channels [g*c, (g+1)*c) at every loop
    step of the block (P1 section "Preliminaries", "Vector quantization of the KV cache": G
    contiguous channels; no permutation outside TaSQ);
  * one codebook per (layer, KV head, K|V, block), shared by all groups g;
  * indices are stored 0-based (entry e_{r+1} is code r);
  * ties in the nearest-entry rule go to the lowest index;
  * RoPE uses the rotate-half pairs {f, f + D/2} (P1 appendix "Grouping under
    loop coupling" keeps RoPE pairs {i, i + D/2} together) with
    theta_f = base^(-2f/D) and position = the token's 0-based index;
  * the decode query arrives already rotated at its own position, and the
    softmax scale defaults to 1/sqrt(D).

Parity pins: every function below is pinned by a CPU test against something
other than itself (closed forms, hand-worked fixtures under tests/golden/,
exact rational brute force, library routines, invariants); see
tests/test_oracle_*.py.  None is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# relative width of the near-tie band for the nearest-entry rule
NEAR_TIE_REL = 1e-6


# --------------------------------------------------------------------------
# coupled vectors  [P1 section "Loop-axis vector quantization", eq. (4);
#                   P2 section 3.1: coordinate i*Tc + m of the coupled vector]
# --------------------------------------------------------------------------
def coupled_vectors(x: np.ndarray, Tc: int, c: int, beta: int) -> np.ndarray:
    """Coupled vectors of one (layer, head, K|V) cache.

    x: [T, N, D], the loop steps of one cache stream.  Block `beta` holds the
    loop steps beta*Tc + m (+1 in the paper's 1-based numbering), m < Tc.  A
    code covers c channels at each of those Tc steps; the coupled vector of
    token j and channel group g is

        z[j, g, i*Tc + m] = x[beta*Tc + m, j, g*c + i],   i < c, m < Tc.

    Returns float64 [N, D // c, c * Tc].
    """
    x = np.asarray(x, dtype=np.float64)
    T, N, D = x.shape
    assert T % Tc == 0 and D % c == 0 and 0 <= beta < T // Tc
    z = np.empty((N, D // c, c * Tc), dtype=np.float64)
    for m in range(Tc):
        step = x[beta * Tc + m]                 # [N, D]
        for i in range(c):
            z[:, :, i * Tc + m] = step[:, i::c]  # channels g*c + i, all g
    return z


# --------------------------------------------------------------------------
# nearest-entry encoding  [P1 section "Preliminaries", eq. (2); P2 "Terms to know first":
#                          a(z) = argmin_r ||z - e_r||^2]
# --------------------------------------------------------------------------
@dataclass
class NearestResult:
    idx: np.ndarray      # int64 [n]   lowest index achieving the minimum distance
    d1: np.ndarray       # float64 [n] smallest squared distance
    d2: np.ndarray       # float64 [n] second smallest squared distance (inf if K == 1)
    band: np.ndarray     # float64 [n] near-tie band NEAR_TIE_REL*(||z||^2 + ||e_idx||^2)

    @property
    def near_tie(self) -> np.ndarray:
        return (self.d2 - self.d1) < self.band


def squared_distances(z: np.ndarray, E: np.ndarray) -> np.ndarray:
    """Direct-difference squared distances sum_u (z_u - e_r[u])^2, float64 [n, K]."""
    z = np.asarray(z, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    diff = z[:, None, :] - E[None, :, :]
    return np.einsum("nkg,nkg->nk", diff, diff)


def nearest_entry(z: np.ndarray, E: np.ndarray, method: str = "direct",
                  chunk: int = 4096) -> NearestResult:
    """Nearest codebook entry of every row of z (eq. (2)).

    method="direct" evaluates every distance by direct differences.
    method="gemm" evaluates ||e||^2 - 2 z.e in fp64 with BLAS (the same
    minimiser up to fp64 rounding) and re-evaluates by direct differences every
    row whose two smallest values lie within 1e-10 of the distance scale, so
    the returned index equals the direct method's.
    """
    z = np.asarray(z, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    n, G = z.shape
    K = E.shape[0]
    idx = np.empty(n, dtype=np.int64)
    d1 = np.empty(n)
    d2 = np.full(n, np.inf)
    esq = (E * E).sum(1)
    for s in range(0, n, chunk):
        zs = z[s:s + chunk]
        if method == "direct":
            d = squared_distances(zs, E)
        elif method == "gemm":
            zsq = (zs * zs).sum(1)
            d = zsq[:, None] - 2.0 * (zs @ E.T) + esq[None, :]
            part = np.partition(d, 1, axis=1)[:, :2] if K > 1 else d[:, :1]
            scale = zsq + esq.max()
            redo = (part[:, 1] - part[:, 0] < 1e-10 * scale) if K > 1 else np.zeros(len(zs), bool)
            if redo.any():
                d[redo] = squared_distances(zs[redo], E)
        else:
            raise ValueError(method)
        a = np.argmin(d, axis=1)  # first occurrence: lowest index among exact ties
        idx[s:s + chunk] = a
        d1[s:s + chunk] = d[np.arange(len(zs)), a]
        if K > 1:
            d2[s:s + chunk] = np.partition(d, 1, axis=1)[:, 1]
        if method == "gemm":
            # report exact (direct-difference) d1 for the chosen entry
            diff = zs - E[a]
            d1[s:s + chunk] = (diff * diff).sum(1)
    band = NEAR_TIE_REL * ((z * z).sum(1) + esq[idx])
    return NearestResult(idx, d1, d2, band)


def accepts(z: np.ndarray, E: np.ndarray, res: NearestResult, idx_other: np.ndarray) -> np.ndarray:
    """True where idx_other equals the oracle's index or lies in its near-tied set."""
    idx_other = np.asarray(idx_other, dtype=np.int64)
    same = idx_other == res.idx
    if same.all():
        return same
    z = np.asarray(z, dtype=np.float64)
    diff = z - np.asarray(E, dtype=np.float64)[idx_other]
    d_other = (diff * diff).sum(1)
    return same | ((d_other - res.d1) < res.band)


def encode_stream(x: np.ndarray, E: np.ndarray, Tc: int, c: int, beta: int,
                  method: str = "direct") -> tuple:
    """Encode block `beta` of one cache stream x [T, N, D].

    E is either one codebook [K, c*Tc] shared by every channel group, or one
    codebook per group [D // c, K, c*Tc] (P1 section "Loop-axis vector
    quantization" writes the codebook of a code as B_{beta,l,h,g}: group g of
    token j is then coded with E[g]).
    Returns (idx [N, D // c], NearestResult over the N*(D//c) coupled vectors
    in (token, group) order).
    """
    z = coupled_vectors(x, Tc, c, beta)
    N, ng, G = z.shape
    E = np.asarray(E)
    if E.ndim == 2:
        res = nearest_entry(z.reshape(N * ng, G), E, method=method)
        return res.idx.reshape(N, ng), res
    assert E.shape[0] == ng
    parts = [nearest_entry(z[:, g, :], E[g], method=method) for g in range(ng)]
    stack = lambda f: np.stack([getattr(r, f) for r in parts], axis=1).reshape(N * ng)
    res = NearestResult(stack("idx"), stack("d1"), stack("d2"), stack("band"))
    return res.idx.reshape(N, ng), res


# --------------------------------------------------------------------------
# index rows  [P1 section "System implementation", cache layout: a quantised
#              page stores one index row per block; b bits per code]
# --------------------------------------------------------------------------
def row_group_order(n_groups: int) -> np.ndarray:
    """Group held by each slot of an index row.

    The row stores the codes in "RoPE-pair interleaved" order: with h = n/2
    and q = n/8, slot block i (i < 4) holds the q groups i*q .. i*q+q-1
    followed by their RoPE partners h + i*q .. h + i*q+q-1 (RoPE rotates
    channel f together with channel f + D/2, i.e. group g with group g + h).
    The pages fix no byte order inside a row; this is the library's layout.
    """
    assert n_groups % 8 == 0
    h, q = n_groups // 2, n_groups // 8
    order = []
    for i in range(4):
        order += list(range(i * q, i * q + q))
        order += list(range(h + i * q, h + i * q + q))
    return np.array(order, dtype=np.int64)


def groups_to_slots(idx: np.ndarray) -> np.ndarray:
    """Codes [N, n_groups] in group order -> the same codes in row slot order."""
    idx = np.asarray(idx)
    return idx[:, row_group_order(idx.shape[1])]


def slots_to_groups(slots: np.ndarray) -> np.ndarray:
    slots = np.asarray(slots)
    out = np.empty_like(slots)
    out[:, row_group_order(slots.shape[1])] = slots
    return out


def pack_rows(idx: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [N, n_slots] (already in slot order) into bytes [N, n_slots*bits/8].

    8-bit: one byte per slot.  4-bit: two slots per byte, the even slot in
    the low nibble.
    """
    idx = np.asarray(idx, dtype=np.int64)
    assert idx.min(initial=0) >= 0 and idx.max(initial=0) < (1 << bits)
    if bits == 8:
        return idx.astype(np.uint8)
    if bits == 4:
        assert idx.shape[1] % 2 == 0
        return (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)
    raise ValueError(bits)


def unpack_rows(rows: np.ndarray, bits: int, n_groups: int) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    if bits == 8:
        return rows[:, :n_groups].astype(np.int64)
    if bits == 4:
        out = np.empty((rows.shape[0], n_groups), dtype=np.int64)
        out[:, 0::2] = rows & 0xF
        out[:, 1::2] = rows >> 4
        return out
    raise ValueError(bits)


def scatter_rows(cache: np.ndarray, rows: np.ndarray, slots: np.ndarray, h: int, kv: int) -> None:
    """Write rows [n, R] into a paged cache [num_pages, H, 2, P, R] at physical slots."""
    P = cache.shape[3]
    slots = np.asarray(slots, dtype=np.int64)
    cache[slots // P, h, kv, slots % P, :] = rows


def gather_rows(cache: np.ndarray, block_table_row: np.ndarray, n: int, h: int, kv: int) -> np.ndarray:
    """Rows [n, R] of the first n logical tokens of one request."""
    P = cache.shape[3]
    p = np.arange(n)
    pages = np.asarray(block_table_row, dtype=np.int64)[p // P]
    return cache[pages, h, kv, p % P, :]


# --------------------------------------------------------------------------
# loop slices and reconstruction  [P1 section "Loop-axis vector quantization", eq. (5); section
#   "System implementation": loop step beta*Tc + m + 1 reads coordinates
#   [e]_{i*Tc + m}, i < c, of the chosen entry]
# --------------------------------------------------------------------------
def loop_slice(E: np.ndarray, Tc: int, c: int, m: int) -> np.ndarray:
    """B_t: coordinates i*Tc + m (i < c) of every entry, float64 [K, c]."""
    E = np.asarray(E, dtype=np.float64)
    return E[:, [i * Tc + m for i in range(c)]]


def rebuild(idx: np.ndarray, E: np.ndarray, Tc: int, c: int, m: int) -> np.ndarray:
    """Reconstruct one loop step: xhat[j, g*c + i] = e_{idx[j, g]}[i*Tc + m].

    E is a shared codebook [K, c*Tc] or one codebook per group [D // c, K, c*Tc]
    (group g then reads entry idx[j, g] of E[g]).
    """
    idx = np.asarray(idx, dtype=np.int64)
    N, ng = idx.shape
    E = np.asarray(E)
    if E.ndim == 2:
        return loop_slice(E, Tc, c, m)[idx].reshape(N, ng * c)
    out = np.empty((N, ng * c))
    for g in range(ng):
        out[:, g * c:(g + 1) * c] = loop_slice(E[g], Tc, c, m)[idx[:, g]]
    return out


# --------------------------------------------------------------------------
# RoPE  [P1 section "Preliminaries" and appendix "Optimizing pre-RoPE vector
#        quantization serving efficiency": keys are quantised before RoPE, which the
#        attention applies to the reconstructed key at the token's position]
# --------------------------------------------------------------------------
def rope_frequencies(D: int, base: float) -> np.ndarray:
    f = np.arange(D // 2, dtype=np.float64)
    return base ** (-2.0 * f / D)


def rope_cos_sin(pos: np.ndarray, D: int, base: float):
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_frequencies(D, base)[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE of rows x [N, D] at positions pos [N]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[1]
    cs, sn = rope_cos_sin(pos, D, base)
    a, b = x[:, :D // 2], x[:, D // 2:]
    return np.concatenate([a * cs - b * sn, b * cs + a * sn], axis=1)


def rope_table(max_pos: int, D: int, base: float) -> np.ndarray:
    """[max_pos, D] float64: cos(p*theta_f) in columns f, sin in columns D/2 + f."""
    cs, sn = rope_cos_sin(np.arange(max_pos), D, base)
    return np.concatenate([cs, sn], axis=1)


# --------------------------------------------------------------------------
# attention  [P1 section "System implementation": splitting the tokens and
#   merging the partial results by log-sum-exp changes nothing in the result,
#   so the reference is plain dense softmax attention over all tokens]
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """o = softmax(sm_scale * k @ q) @ v and lse = log sum exp(sm_scale * k @ q).

    With no keys the softmax is empty; the output is then taken to be zero and
    the lse -inf (the sum of no exponentials is 0).
    """
    q = np.asarray(q, dtype=np.float64)
    if np.asarray(k).shape[0] == 0:
        return np.zeros(np.asarray(v).shape[1]), -np.inf
    s = sm_scale * (np.asarray(k, dtype=np.float64) @ q)
    mx = s.max()
    w = np.exp(s - mx)
    l = w.sum()
    o = (w @ np.asarray(v, dtype=np.float64)) / l
    return o, mx + np.log(l)


def decode_attention(q: np.ndarray, cache_block: np.ndarray, block_table_row: np.ndarray,
                     n: int, cb_block: np.ndarray, t: int, Tc: int, c: int, bits: int,
                     base: float, sm_scale: float | None = None):
    """Quantised decode attention of one request at loop step t (1-based).

    q: [H_q, D] queries (already rotated at their own position).
    cache_block: [num_pages, H_kv, 2, P, R] index cache of block (t-1)//Tc.
    cb_block: [H_kv, 2, K, c*Tc] codebooks of that block, or [H_kv, 2, D//c, K,
    c*Tc] with one codebook per channel group.
    Query head j reads KV head j // (H_q / H_kv).
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
    o = np.zeros((H_q, D))
    lse = np.zeros(H_q)
    for h in range(H_kv):
        ki = slots_to_groups(unpack_rows(gather_rows(cache_block, block_table_row, n, h, 0), bits, ng))
        vi = slots_to_groups(unpack_rows(gather_rows(cache_block, block_table_row, n, h, 1), bits, ng))
        khat = rebuild(ki, cb_block[h, 0], Tc, c, m)
        vhat = rebuild(vi, cb_block[h, 1], Tc, c, m)
        krot = rope(khat, pos, base)
        for j in range(h * grp, (h + 1) * grp):
            o[j], lse[j] = attention(q[j], krot, vhat, sm_scale)
    return o, lse


def gather_rows_at(cache: np.ndarray, block_table_row: np.ndarray, pos: np.ndarray, h: int,
                   kv: int) -> np.ndarray:
    """Rows [len(pos), R] of the logical tokens at positions pos of one request."""
    P = cache.shape[3]
    p = np.asarray(pos, dtype=np.int64)
    pages = np.asarray(block_table_row, dtype=np.int64)[p // P]
    return cache[pages, h, kv, p % P, :]


# --------------------------------------------------------------------------
# bf16 sink and recent window  [P1 section "System implementation": a
#   request keeps its n_s leading tokens and its n_r latest tokens unquantised
#   (bf16), every other token as codes; the bf16 part and the coded part are
#   attended separately at loop step t and their partials joined by
#   log-sum-exp, so the result is a single softmax over all cached tokens]
# --------------------------------------------------------------------------
def decode_attention_window(q: np.ndarray, cache_block: np.ndarray, block_table_row: np.ndarray,
                            n: int, n_sink: int, win_start: int, k_bf: np.ndarray, v_bf: np.ndarray,
                            cb_block: np.ndarray, t: int, Tc: int, c: int, bits: int, base: float,
                            sm_scale: float | None = None):
    """Decode attention of one request whose cache mixes bf16 tokens and codes.

    Positions [0, n_sink) (the sink) and [win_start, n) (the recent window)
    keep their pre-RoPE keys and values in bf16: k_bf, v_bf [n, H_kv, D]
    (float64 holding the bf16 values; only the rows of those positions are
    read).  Positions [n_sink, win_start) are codes in cache_block, looked up
    through block_table_row exactly as in decode_attention.  Every key is
    rotated at its own position and one softmax runs over all n tokens.
    Returns (o [H_q, D], lse [H_q]).
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
    o = np.zeros((H_q, D))
    lse = np.zeros(H_q)
    for h in range(H_kv):
        k = np.empty((n, D))
        v = np.empty((n, D))
        ki = slots_to_groups(unpack_rows(gather_rows_at(cache_block, block_table_row, qpos, h, 0), bits, ng))
        vi = slots_to_groups(unpack_rows(gather_rows_at(cache_block, block_table_row, qpos, h, 1), bits, ng))
        k[qpos] = rebuild(ki, cb_block[h, 0], Tc, c, m)
        v[qpos] = rebuild(vi, cb_block[h, 1], Tc, c, m)
        k[bpos] = k_bf[bpos, h]
        v[bpos] = v_bf[bpos, h]
        krot = rope(k, np.arange(n), base)
        for j in range(h * grp, (h + 1) * grp):
            o[j], lse[j] = attention(q[j], krot, v, sm_scale)
    return o, lse


def build_index_cache(xk: np.ndarray, xv: np.ndarray, cb: np.ndarray, Tc: int, c: int,
                      bits: int, slots: np.ndarray, num_pages: int, page_size: int,
                      method: str = "direct"):
    """Encode caches xk, xv [T, n_tok, H_kv, D] into paged index caches.

    Returns (caches [n_blocks, num_pages, H_kv, 2, P, R] uint8, near-tie count,
    dict (beta, h, kv) -> NearestResult).
    """
    T, n_tok, H, D = xk.shape
    nb = T // Tc
    R = (D // c) * bits // 8
    caches = np.zeros((nb, num_pages, H, 2, page_size, R), dtype=np.uint8)
    results = {}
    ties = 0
    for beta in range(nb):
        for h in range(H):
            for kv, x in enumerate((xk, xv)):
                idx, res = encode_stream(x[:, :, h, :], cb[beta, h, kv], Tc, c, beta, method)
                results[(beta, h, kv)] = res
                ties += int(res.near_tie.sum())
                scatter_rows(caches[beta], pack_rows(groups_to_slots(idx), bits), slots, h, kv)
    return caches, ties, results


def bits_per_element(bits: int, G: int) -> float:
    """Storage cost of one code of b bits covering G elements [P1 section "Preliminaries"]."""
    return bits / G
