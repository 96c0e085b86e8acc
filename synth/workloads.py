"""Seeded synthetic workloads standing in for the looped-model KV caches.

The LoopVQ paper (hub.valency.io/works/W_7srt5hed_v1, section "Redundancy along
the loop axis") reports that the pre-RoPE keys and values of one layer are
strongly correlated across loop steps (adjacent-step correlation rising from
about 0.69 to 0.94).  The generators here reproduce that structure with a
first-order recurrence along the loop axis,

    x^(1) = eps_1,   x^(t) = rho_t * x^(t-1) + sqrt(1 - rho_t^2) * eps_t,

with eps i.i.d. standard normal over (token, head, channel, step), optionally
multiplied by a per-(head, channel) lognormal scale that is shared by every
token and loop step, and then rounded once to the storage precision.

Nothing here computes any part of the method (no coupling arithmetic for the
path under test, no distances, no attention): it draws inputs.  The one place
that touches the coupled-vector layout is `make_codebooks`, which builds the
codebook *inputs* by sampling calibration vectors; both the oracle and the GPU
path then receive the identical fp16 codebook.

Seeds: the data seed of a configuration is its index; calibration draws use
seed+1000, queries seed+2000 (+t for a per-loop-step query), page tables and
ragged lengths seed+3000, and the per-channel scales (a property of the
synthetic "model", shared by data and calibration) seed+4000.  All draws use
NumPy's PCG64 `default_rng`.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    index: int
    T: int                 # loop steps
    Tc: int                # loop steps per block (one index serves Tc steps)
    H_kv: int
    H_q: int
    D: int
    c: int                 # channels per loop step covered by one code
    bits: int              # index bits (4 or 8)
    x_dtype: str           # "f32" | "bf16"  (encoder input / cache data)
    io_dtype: str          # "f32" | "bf16"  (decode query and output)
    page_size: int
    batch: int             # decode batch
    seq_len: Optional[int]             # fixed decode context, or None if ragged
    ragged: Optional[Tuple[int, int]]  # inclusive bounds of ragged lengths
    rhos: Tuple[float, ...]            # rho_t for t = 2..T
    scale_sigma: float                 # lognormal sigma of per-channel scales (0: none)
    encode_batch: int                  # requests in the encode measurement
    encode_tokens: int                 # tokens per request in the encode measurement
    n_calib: int = 1024
    base: float = 10000.0

    @property
    def G(self) -> int:
        return self.c * self.Tc

    @property
    def K(self) -> int:
        return 1 << self.bits

    @property
    def n_blocks(self) -> int:
        return self.T // self.Tc

    @property
    def n_groups(self) -> int:
        return self.D // self.c

    @property
    def row_bytes(self) -> int:
        return self.n_groups * self.bits // 8

    @property
    def group_size(self) -> int:
        return self.H_q // self.H_kv

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _linear_rhos(T: int, lo: float, hi: float) -> Tuple[float, ...]:
    # rho_t for t = 2..T rising linearly from lo to hi
    return tuple(lo + (hi - lo) * (t - 2) / (T - 2) for t in range(2, T + 1))


CONFIGS = (
    # tiny CPU-checkable case: fp32 data, 4-bit codes, 0.5 bit/element
    Config("tiny", 0, T=4, Tc=4, H_kv=1, H_q=1, D=64, c=2, bits=4,
           x_dtype="f32", io_dtype="f32", page_size=64, batch=1, seq_len=256,
           ragged=None, rhos=(0.7, 0.8, 0.9), scale_sigma=0.0,
           encode_batch=1, encode_tokens=256),
    # one layer of a 1.4B looped model, 0.5 bit/element
    Config("layer1p4b", 1, T=4, Tc=4, H_kv=16, H_q=16, D=128, c=4, bits=8,
           x_dtype="bf16", io_dtype="bf16", page_size=64, batch=8, seq_len=4096,
           ragged=None, rhos=(0.7, 0.8, 0.9), scale_sigma=0.5,
           encode_batch=8, encode_tokens=4096),
    # long-context decode: the same layer at 32K context, batch 16
    Config("longctx32k", 2, T=4, Tc=4, H_kv=16, H_q=16, D=128, c=4, bits=8,
           x_dtype="bf16", io_dtype="bf16", page_size=64, batch=16, seq_len=32768,
           ragged=None, rhos=(0.7, 0.8, 0.9), scale_sigma=0.5,
           encode_batch=16, encode_tokens=32768),
    # 0.25 bit/element, GQA group 4, ragged batch of 64
    Config("gqa_ragged", 3, T=4, Tc=4, H_kv=8, H_q=32, D=128, c=8, bits=8,
           x_dtype="bf16", io_dtype="bf16", page_size=64, batch=64, seq_len=None,
           ragged=(1024, 16384), rhos=(0.7, 0.8, 0.9), scale_sigma=0.5,
           encode_batch=1, encode_tokens=4096),
    # deep-loop model: 32 loop steps in 8 blocks of 4
    Config("deeploop", 4, T=32, Tc=4, H_kv=16, H_q=16, D=128, c=4, bits=8,
           x_dtype="bf16", io_dtype="bf16", page_size=64, batch=4, seq_len=16384,
           ragged=None, rhos=_linear_rhos(32, 0.7, 0.95), scale_sigma=0.5,
           encode_batch=1, encode_tokens=4096),
)


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name or f"C{c.index}" == name:
            return c
    raise KeyError(name)


# --------------------------------------------------------------------------
# storage-precision rounding (input preparation)
# --------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round_to_f16(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------
# data generators
# --------------------------------------------------------------------------
def loop_correlated(rng: np.random.Generator, T: int, shape, rhos) -> np.ndarray:
    """float32 array [T, *shape] following the loop-axis recurrence."""
    assert len(rhos) == T - 1
    out = np.empty((T,) + tuple(shape), dtype=np.float32)
    out[0] = rng.standard_normal(shape, dtype=np.float32)
    for t in range(1, T):
        r = np.float32(rhos[t - 1])
        out[t] = r * out[t - 1] + np.float32(np.sqrt(1.0 - float(r) ** 2)) * \
            rng.standard_normal(shape, dtype=np.float32)
    return out


def channel_scales(cfg: Config) -> np.ndarray:
    """Per-(K|V, head, channel) lognormal(0, sigma) scales, float32 [2, H_kv, D]."""
    if cfg.scale_sigma == 0.0:
        return np.ones((2, cfg.H_kv, cfg.D), dtype=np.float32)
    rng = np.random.default_rng(cfg.index + 4000)
    return np.exp(cfg.scale_sigma * rng.standard_normal((2, cfg.H_kv, cfg.D))).astype(np.float32)


def _store(cfg: Config, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if cfg.x_dtype == "bf16" else np.asarray(x, dtype=np.float32)


def make_kv(cfg: Config, n_tok: int, seed: Optional[int] = None, heads=None):
    """Pre-RoPE keys and values, float32 holding storage-precision values.

    Returns (xk, xv), each [T, n_tok, H, D] for the selected heads (all by default).
    Keys are drawn first, then values, from one PCG64 stream.
    """
    seed = cfg.index if seed is None else seed
    heads = list(range(cfg.H_kv)) if heads is None else list(heads)
    rng = np.random.default_rng(seed)
    sc = channel_scales(cfg)
    out = []
    for kv in range(2):
        x = loop_correlated(rng, cfg.T, (n_tok, cfg.H_kv, cfg.D), cfg.rhos)
        x = x[:, :, heads, :] * sc[kv, heads, :][None, None, :, :]
        out.append(_store(cfg, x))
    return out[0], out[1]


def make_codebooks(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    """fp16 codebooks [n_blocks, H_kv, 2, K, G], entry coordinate u = i*Tc + m.

    For each (block, head, K|V) the entries are K distinct coupled vectors drawn
    uniformly without replacement from a separate calibration set of
    `cfg.n_calib` tokens (same generator and channel scales, other seed).
    """
    seed = (cfg.index if seed is None else seed) + 1000
    rng = np.random.default_rng(seed)
    xk, xv = make_kv(cfg, cfg.n_calib, seed=seed)
    cb = np.empty((cfg.n_blocks, cfg.H_kv, 2, cfg.K, cfg.G), dtype=np.float16)
    n_vec = cfg.n_calib * cfg.n_groups
    ii = np.arange(cfg.c)
    mm = np.arange(cfg.Tc)
    for beta in range(cfg.n_blocks):
        for h in range(cfg.H_kv):
            for kv, x in enumerate((xk, xv)):
                while True:
                    pick = rng.choice(n_vec, size=cfg.K, replace=False)
                    tok, grp = pick // cfg.n_groups, pick % cfg.n_groups
                    # entry[r, i*Tc + m] = x[beta*Tc + m, tok_r, h, grp_r*c + i]
                    steps = beta * cfg.Tc + mm[None, None, :]
                    chans = grp[:, None, None] * cfg.c + ii[None, :, None]
                    e = x[steps, tok[:, None, None], h, chans]       # [K, c, Tc]
                    e = round_to_f16(e.reshape(cfg.K, cfg.G))
                    if len(np.unique(e.view(np.uint16).reshape(cfg.K, -1), axis=0)) == cfg.K:
                        break
                cb[beta, h, kv] = e
    return cb


def make_codebooks_per_group(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    """fp16 codebooks, one per channel group: [n_blocks, H_kv, 2, D // c, K, G].

    The entries of group g's codebook are K distinct coupled vectors of group g
    drawn without replacement from the calibration tokens (same generator and
    channel scales as make_codebooks, seed + 1000 + 500).
    """
    seed = (cfg.index if seed is None else seed) + 1500
    rng = np.random.default_rng(seed)
    xk, xv = make_kv(cfg, cfg.n_calib, seed=seed)
    ng = cfg.n_groups
    cb = np.empty((cfg.n_blocks, cfg.H_kv, 2, ng, cfg.K, cfg.G), dtype=np.float16)
    ii = np.arange(cfg.c)
    mm = np.arange(cfg.Tc)
    for beta in range(cfg.n_blocks):
        steps = beta * cfg.Tc + mm[None, None, :]
        for h in range(cfg.H_kv):
            for kv, x in enumerate((xk, xv)):
                for g in range(ng):
                    while True:
                        tok = rng.choice(cfg.n_calib, size=cfg.K, replace=False)
                        chans = g * cfg.c + ii[None, :, None]
                        e = round_to_f16(x[steps, tok[:, None, None], h, chans].reshape(cfg.K, cfg.G))
                        if len(np.unique(e.view(np.uint16).reshape(cfg.K, -1), axis=0)) == cfg.K:
                            break
                    cb[beta, h, kv, g] = e
    return cb


def make_queries(cfg: Config, batch: int, seed: Optional[int] = None, t: int = 0) -> np.ndarray:
    """Decode queries [batch, H_q, D] ~ N(0, 1), already rotated at their own position."""
    seed = (cfg.index if seed is None else seed) + 2000 + t
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, cfg.H_q, cfg.D), dtype=np.float32)
    return round_to_bf16(q) if cfg.io_dtype == "bf16" else q


def make_seq_lens(cfg: Config, batch: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    batch = cfg.batch if batch is None else batch
    if cfg.ragged is None:
        return np.full(batch, cfg.seq_len, dtype=np.int32)
    seed = (cfg.index if seed is None else seed) + 3000
    rng = np.random.default_rng(seed)
    lo, hi = cfg.ragged
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def make_block_table(cfg: Config, seq_lens: np.ndarray, seed: Optional[int] = None,
                     extra_pages: int = 0):
    """Random page assignment.

    The physical pages are a random permutation of sum_b ceil(N_b / P) ids (plus
    `extra_pages` unused ones); request b owns the next ceil(N_b / P) of them.
    Returns (block_table [B, max_pages] int32 padded with 0, num_pages).
    """
    seed = (cfg.index if seed is None else seed) + 3000 + 1
    rng = np.random.default_rng(seed)
    P = cfg.page_size
    n_pages = [(int(n) + P - 1) // P for n in seq_lens]
    total = int(sum(n_pages)) + extra_pages
    perm = rng.permutation(total).astype(np.int32)
    max_pages = max(1, max(n_pages) if n_pages else 1)
    bt = np.zeros((len(seq_lens), max_pages), dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, total


def slot_mapping_for(block_table: np.ndarray, b: int, n_tok: int, page_size: int,
                     start: int = 0) -> np.ndarray:
    """Physical slot (page * P + offset) of tokens start..start+n_tok-1 of request b."""
    p = np.arange(start, start + n_tok)
    return (block_table[b, p // page_size].astype(np.int64) * page_size + p % page_size).astype(np.int32)


def random_index_cache(cfg: Config, num_pages: int, seed: int) -> np.ndarray:
    """Uniform random index bytes [num_pages, H_kv, 2, P, R] (every byte value is a valid code)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(num_pages, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes),
                        dtype=np.uint8)


def make_kv_torch(cfg: Config, n_tok: int, seed: int, device="cuda", dtype=None):
    """The same loop-axis recurrence drawn with torch's generator on `device`.

    For workloads too large to draw on the host (the bench's 32K-context
    batch).  Uses torch's Philox stream, so values differ from `make_kv` for
    the same seed; the statistics (rho_t, channel scales, storage rounding)
    are the same.  Returns (xk, xv), each [T, n_tok, H_kv, D].
    """
    import torch
    dtype = dtype or (torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    sc = torch.from_numpy(channel_scales(cfg)).to(device)
    out = []
    for kv in range(2):
        x = torch.empty((cfg.T, n_tok, cfg.H_kv, cfg.D), dtype=dtype, device=device)
        prev = torch.randn((n_tok, cfg.H_kv, cfg.D), generator=g, device=device, dtype=torch.float32)
        x[0] = (prev * sc[kv]).to(dtype)
        for t in range(1, cfg.T):
            r = float(cfg.rhos[t - 1])
            eps = torch.randn((n_tok, cfg.H_kv, cfg.D), generator=g, device=device, dtype=torch.float32)
            prev = r * prev + (1.0 - r * r) ** 0.5 * eps
            x[t] = (prev * sc[kv]).to(dtype)
        out.append(x)
    return out[0], out[1]


# --------------------------------------------------------------------------
# bf16 sink and recent window (placement only)
# --------------------------------------------------------------------------
def make_window(cfg: Config, seq_lens: np.ndarray, n_sink: int, n_recent: int,
                seed: Optional[int] = None):
    """Sink / recent-window split of each request and a random bf16 page assignment.

    Request b keeps positions [0, n_sink) and [win_start, seq_len) in bf16
    pages of 8 tokens; win_start is the largest multiple of 8 that leaves at
    least n_recent tokens in the window (so it holds n_recent to n_recent + 7
    tokens), and never below the sink.  Bf16 token u of a request (sink first,
    then window) sits in page page_table[b, u // 8], slot u % 8; the physical
    pages are a random permutation.
    Returns (n_sink [B] int32, win_start [B] int32, page_table [B, max_pages]
    int32, num_pages).
    """
    seed = (cfg.index if seed is None else seed) + 3000 + 2
    rng = np.random.default_rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int64)
    ns = np.minimum(n_sink, lens)
    ws = np.clip(((lens - n_recent) // 8) * 8, ns, lens)
    nbf = ns + lens - ws
    n_pages = (nbf + 7) // 8
    total = int(n_pages.sum())
    perm = rng.permutation(max(total, 1)).astype(np.int32)
    pt = np.zeros((len(lens), max(1, int(n_pages.max(initial=0)))), dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        pt[b, :n] = perm[off:off + n]
        off += int(n)
    return ns.astype(np.int32), ws.astype(np.int32), pt, max(total, 1)


def window_positions(n_sink: int, win_start: int, seq_len: int) -> np.ndarray:
    """Positions of a request's bf16 tokens u = 0, 1, ... (sink, then window)."""
    return np.concatenate([np.arange(n_sink), np.arange(win_start, seq_len)]).astype(np.int64)


def fill_window_pages(num_pages: int, page_table: np.ndarray, n_sink: np.ndarray, win_start: np.ndarray,
                      seq_lens: np.ndarray, k_of, v_of, H: int, D: int) -> np.ndarray:
    """bf16 pages [num_pages, H, 2, 8, D] (float32 holding bf16 values).

    k_of(b, pos) and v_of(b, pos) return the [len(pos), H, D] pre-RoPE keys and
    values of request b at the given positions (already bf16 values).
    """
    pages = np.zeros((num_pages, H, 2, 8, D), dtype=np.float32)
    for b in range(len(seq_lens)):
        pos = window_positions(int(n_sink[b]), int(win_start[b]), int(seq_lens[b]))
        if len(pos) == 0:
            continue
        u = np.arange(len(pos))
        pg = page_table[b, u // 8]
        pages[pg, :, 0, u % 8, :] = k_of(b, pos)
        pages[pg, :, 1, u % 8, :] = v_of(b, pos)
    return pages


# --------------------------------------------------------------------------
# TaSQ inputs (synthetic stand-ins for calibrated ones)
# --------------------------------------------------------------------------
def make_tasq(cfg: Config, seed: Optional[int] = None):
    """Synthetic TaSQ parameters of one layer.

    w    [T, H_kv, D] float32 channel weights, lognormal(0, 0.4): TaSQ sets
         w_i^2 proportional to the second moment of the queries on channel i,
         which needs a model; any positive weights exercise the same path.
    perm [T // Tc, H_kv, D/2] int32: one uniformly random pair permutation per
         (block, head), standing in for the covariance-based grouping.
    Seed: config index + 5000.
    """
    seed = (cfg.index if seed is None else seed) + 5000
    rng = np.random.default_rng(seed)
    w = np.exp(0.4 * rng.standard_normal((cfg.T, cfg.H_kv, cfg.D))).astype(np.float32)
    perm = np.stack([np.stack([rng.permutation(cfg.D // 2) for _ in range(cfg.H_kv)])
                     for _ in range(cfg.n_blocks)]).astype(np.int32)
    return w, perm


def make_sigma(n: int, seed: int) -> np.ndarray:
    """Positive fp16 per-token scales (lognormal(0, 0.3)), float16 [n]."""
    rng = np.random.default_rng(seed)
    return np.exp(0.3 * rng.standard_normal(n)).astype(np.float16)


def codebooks_from_vectors(cfg: Config, xk: np.ndarray, xv: np.ndarray, seed: int) -> np.ndarray:
    """fp16 codebooks [n_blocks, H_kv, 2, K, G] of K distinct coupled vectors
    sampled without replacement from the given per-step arrays xk, xv
    [T, n, H_kv, D] (the same sampling rule as make_codebooks, on any data,
    for example keys already mapped to another coordinate system)."""
    rng = np.random.default_rng(seed)
    n = xk.shape[1]
    cb = np.empty((cfg.n_blocks, cfg.H_kv, 2, cfg.K, cfg.G), dtype=np.float16)
    n_vec = n * cfg.n_groups
    ii = np.arange(cfg.c)
    mm = np.arange(cfg.Tc)
    for beta in range(cfg.n_blocks):
        for h in range(cfg.H_kv):
            for kv, x in enumerate((xk, xv)):
                while True:
                    pick = rng.choice(n_vec, size=cfg.K, replace=False)
                    tok, grp = pick // cfg.n_groups, pick % cfg.n_groups
                    steps = beta * cfg.Tc + mm[None, None, :]
                    chans = grp[:, None, None] * cfg.c + ii[None, :, None]
                    e = round_to_f16(np.asarray(x)[steps, tok[:, None, None], h, chans].reshape(cfg.K, cfg.G))
                    if len(np.unique(e.view(np.uint16).reshape(cfg.K, -1), axis=0)) == cfg.K:
                        break
                cb[beta, h, kv] = e
    return cb
