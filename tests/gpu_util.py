"""Helpers of the GPU parity tests: marshal synthetic inputs to the HIP library
and compute the oracle's answer on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_loopvq_amd as lv
import oracle
import synth

TOL = 2e-3


def dims_for(cfg: synth.Config, **over) -> "lv.loopvq_dims":
    kw = dict(D=cfg.D, c=cfg.c, Tc=cfg.Tc, T=cfg.T, bits=cfg.bits, H_kv=cfg.H_kv, H_q=cfg.H_q,
              page_size=cfg.page_size, x_dtype=cfg.x_dtype, io_dtype=cfg.io_dtype)
    kw.update(over)
    return lv.loopvq_dims.make(**kw)


def to_dev(a: np.ndarray, dtype: torch.dtype | None = None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def io_tensor(cfg, a):
    return to_dev(np.asarray(a, dtype=np.float32), torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32)


def x_tensor(cfg, a):
    return to_dev(np.asarray(a, dtype=np.float32), torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32)


def bound(ref: np.ndarray, io_dtype: str) -> np.ndarray:
    """2e-3, plus half a bf16 ulp of the reference when the output is bf16."""
    if io_dtype != "bf16":
        return np.full(ref.shape, TOL)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
    return TOL + 0.5 * 2.0 ** (e - 7)


class GpuLayer:
    """Device copies of one layer's codebooks, slices and RoPE table."""

    def __init__(self, cfg, cb: np.ndarray, max_pos: int, dims=None):
        self.cfg = cfg
        self.dims = dims if dims is not None else dims_for(cfg)
        self.cb = to_dev(cb)
        self.slices, self.hsq = lv.loopvq_build_codebook_slices(self.dims, self.cb)
        self.max_pos = max_pos
        self.rope = lv.loopvq_rope_table(max_pos, cfg.D, cfg.base).cuda()

    def decode(self, t, q, cache_block, block_table, seq_lens, max_seq_len=None, sm_scale=0.0,
               want_lse=True, max_pos=None):
        q_d = q if isinstance(q, torch.Tensor) else io_tensor(self.cfg, q)
        cache_d = cache_block if isinstance(cache_block, torch.Tensor) else to_dev(cache_block)
        bt = to_dev(np.asarray(block_table, dtype=np.int32))
        lens = to_dev(np.asarray(seq_lens, dtype=np.int32))
        msl = int(np.max(seq_lens)) if max_seq_len is None else max_seq_len
        lse = torch.empty((q_d.shape[0], self.cfg.H_q), dtype=torch.float32, device="cuda") if want_lse else None
        out, lse = lv.loopvq_decode_attn(self.dims, t, q_d, cache_d, self.slices, self.rope, bt, lens, msl,
                                         sm_scale=sm_scale, lse=lse,
                                         max_pos=self.max_pos if max_pos is None else max_pos)
        torch.cuda.synchronize()
        return (out.float().cpu().numpy().astype(np.float64),
                None if lse is None else lse.cpu().numpy().astype(np.float64))


    def decode_window(self, t, q, cache_block, block_table, seq_lens, kv_pages, page_table, n_sink, win_start,
                      max_seq_len=None, want_lse=True):
        q_d = q if isinstance(q, torch.Tensor) else io_tensor(self.cfg, q)
        cache_d = cache_block if isinstance(cache_block, torch.Tensor) else to_dev(cache_block)
        kv_d = kv_pages if isinstance(kv_pages, torch.Tensor) else to_dev(np.asarray(kv_pages, np.float32),
                                                                          torch.bfloat16)
        msl = int(np.max(seq_lens)) if max_seq_len is None else max_seq_len
        lse = torch.empty((q_d.shape[0], self.cfg.H_q), dtype=torch.float32, device="cuda") if want_lse else None
        i32 = lambda a: to_dev(np.asarray(a, dtype=np.int32))
        out, lse = lv.loopvq_decode_attn_window(self.dims, t, q_d, cache_d, self.slices, self.rope,
                                                i32(block_table), i32(seq_lens), msl, kv_d, i32(page_table),
                                                i32(n_sink), i32(win_start), lse=lse, max_pos=self.max_pos)
        torch.cuda.synchronize()
        return (out.float().cpu().numpy().astype(np.float64),
                None if lse is None else lse.cpu().numpy().astype(np.float64))


    def decode_tasq(self, t, q, cache_block, block_table, seq_lens, w, perm, sigma, window=None,
                    max_seq_len=None, want_lse=True):
        """TaSQ-coded keys: w [T][H_kv][D], perm [T/Tc][H_kv][D/2], sigma [T][n_slots] fp16 (numpy or
        device tensors); window = (kv_pages, page_table, n_sink, win_start) or None."""
        q_d = q if isinstance(q, torch.Tensor) else io_tensor(self.cfg, q)
        cache_d = cache_block if isinstance(cache_block, torch.Tensor) else to_dev(cache_block)
        i32 = lambda a: a if isinstance(a, torch.Tensor) else to_dev(np.asarray(a, dtype=np.int32))
        w_d = w if isinstance(w, torch.Tensor) else to_dev(np.asarray(w, np.float32))
        sig_d = sigma if isinstance(sigma, torch.Tensor) else to_dev(np.asarray(sigma, np.float16))
        msl = int(np.max(seq_lens)) if max_seq_len is None else max_seq_len
        lse = torch.empty((q_d.shape[0], self.cfg.H_q), dtype=torch.float32, device="cuda") if want_lse else None
        win = None
        if window is not None:
            kvp, pt, ns, ws = window
            kv_d = kvp if isinstance(kvp, torch.Tensor) else to_dev(np.asarray(kvp, np.float32), torch.bfloat16)
            win = (kv_d, i32(pt), i32(ns), i32(ws))
        out, lse = lv.loopvq_decode_attn_tasq(self.dims, t, q_d, cache_d, self.slices, self.rope, i32(block_table),
                                              i32(seq_lens), msl, w_d, i32(perm), sig_d, window=win, lse=lse,
                                              max_pos=self.max_pos)
        torch.cuda.synchronize()
        return (out.float().cpu().numpy().astype(np.float64),
                None if lse is None else lse.cpu().numpy().astype(np.float64))


def ref_decode_window(cfg, t, q, cache_block, block_table, seq_lens, cb, n_sink, win_start, kv_of,
                      requests=None, heads=None):
    """Oracle output with bf16 sink/window tokens; kv_of(b, h) -> (k [n, D], v [n, D]) bf16 values of
    request b's positions (only the bf16 positions are read)."""
    grp = cfg.H_q // cfg.H_kv
    beta = (t - 1) // cfg.Tc
    requests = range(len(seq_lens)) if requests is None else requests
    heads = range(cfg.H_kv) if heads is None else heads
    res = {}
    for b in requests:
        for h in heads:
            rows = slice(h * grp, (h + 1) * grp)
            k, v = kv_of(b, h)
            o, lse = oracle.decode_attention_window(np.asarray(q[b], np.float64)[rows], cache_block[:, h:h + 1],
                                                    block_table[b], int(seq_lens[b]), int(n_sink[b]),
                                                    int(win_start[b]), k[:, None, :], v[:, None, :],
                                                    cb[beta, h:h + 1], t, cfg.Tc, cfg.c, cfg.bits, cfg.base)
            res[(b, h)] = (o, lse)
    return res


def ref_decode(cfg, t, q, cache_block, block_table, seq_lens, cb, requests=None, heads=None, sm_scale=None):
    """Oracle output for the selected requests and KV heads (query rows of those heads)."""
    grp = cfg.H_q // cfg.H_kv
    beta = (t - 1) // cfg.Tc
    requests = range(len(seq_lens)) if requests is None else requests
    heads = range(cfg.H_kv) if heads is None else heads
    res = {}
    for b in requests:
        for h in heads:
            rows = slice(h * grp, (h + 1) * grp)
            o, lse = oracle.decode_attention(np.asarray(q[b], np.float64)[rows], cache_block[:, h:h + 1],
                                             block_table[b], int(seq_lens[b]), cb[beta, h:h + 1], t,
                                             cfg.Tc, cfg.c, cfg.bits, cfg.base, sm_scale)
            res[(b, h)] = (o, lse)
    return res


def compare(cfg, got_o, got_lse, ref, seq_lens):
    """Max abs error and worst bound ratio over the compared (request, head) pairs."""
    grp = cfg.H_q // cfg.H_kv
    worst = 0.0
    worst_ratio = 0.0
    for (b, h), (o, lse) in ref.items():
        rows = slice(h * grp, (h + 1) * grp)
        if seq_lens[b] == 0:
            assert np.all(got_o[b, rows] == 0.0)
            if got_lse is not None:
                assert np.all(np.isneginf(got_lse[b, rows]))
            continue
        err = np.abs(got_o[b, rows] - o)
        worst = max(worst, float(err.max()))
        worst_ratio = max(worst_ratio, float((err / bound(o, cfg.io_dtype)).max()))
        if got_lse is not None:
            assert np.allclose(got_lse[b, rows], lse, rtol=0, atol=1e-4), (b, h, got_lse[b, rows], lse)
    return worst, worst_ratio


def make_cache_from_data(cfg, xk, xv, cb, lens, block_table, num_pages, method="gemm"):
    """Oracle-built paged index caches of all blocks for the given requests."""
    nb = cfg.n_blocks
    caches = np.zeros((nb, num_pages, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=np.uint8)
    off = 0
    ties = 0
    for b, n in enumerate(lens):
        if n == 0:
            continue
        slots = synth.slot_mapping_for(block_table, b, int(n), cfg.page_size)
        c, t, _ = oracle.build_index_cache(xk[:, off:off + n], xv[:, off:off + n], cb, cfg.Tc, cfg.c, cfg.bits,
                                           slots, num_pages, cfg.page_size, method=method)
        caches |= c
        ties += t
        off += int(n)
    return caches, ties


def check_codes(cfg, got_cache, xk, xv, cb, slots, heads=None, blocks=None, method="gemm"):
    """Compare GPU rows with the oracle's nearest entries; returns (near-tie count, mismatches)."""
    P = cfg.page_size
    heads = range(cfg.H_kv) if heads is None else heads
    blocks = range(cfg.n_blocks) if blocks is None else blocks
    ties = bad = 0
    slots = np.asarray(slots, np.int64)
    for beta in blocks:
        for h in heads:
            for kv, x in enumerate((xk, xv)):
                rows = got_cache[beta][slots // P, h, kv, slots % P, :]
                got = oracle.slots_to_groups(oracle.unpack_rows(rows, cfg.bits, cfg.n_groups)).reshape(-1)
                z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, beta).reshape(-1, cfg.G)
                E = cb[beta, h, kv].astype(np.float64)
                res = oracle.nearest_entry(z, E, method=method)
                ties += int(res.near_tie.sum())
                ok = oracle.accepts(z, E, res, got)
                bad += int((~ok).sum())
    return ties, bad


def sigma_at_positions(sigma_t, block_table_row, n, page_size):
    """sigma of loop step t at positions 0..n-1 of one request (slot-indexed array -> by position)."""
    pos = np.arange(n)
    slots = np.asarray(block_table_row, np.int64)[pos // page_size] * page_size + pos % page_size
    return np.asarray(sigma_t, np.float64)[slots]


def ref_decode_tasq(cfg, t, q, cache_block, block_table, seq_lens, cb, w, perm, sigma, requests=None,
                    heads=None, window=None):
    """Oracle output with TaSQ-coded keys.  sigma [T][n_slots] (fp16 values); window = (n_sink,
    win_start, kv_of) adds the bf16 sink and recent window (kv_of(b, h) -> (k [n, D], v [n, D]))."""
    tq = oracle.tasq_ref
    grp = cfg.H_q // cfg.H_kv
    beta = (t - 1) // cfg.Tc
    requests = range(len(seq_lens)) if requests is None else requests
    heads = range(cfg.H_kv) if heads is None else heads
    res = {}
    for b in requests:
        n = int(seq_lens[b])
        sig = sigma_at_positions(sigma[t - 1], block_table[b], n, cfg.page_size)
        for h in heads:
            rows = slice(h * grp, (h + 1) * grp)
            qb = np.asarray(q[b], np.float64)[rows]
            args = (cb[beta, h:h + 1], t, cfg.Tc, cfg.c, cfg.bits, cfg.base, w[t - 1, h:h + 1],
                    perm[beta, h:h + 1], sig)
            if window is None:
                o, lse = tq.decode_attention_tasq(qb, cache_block[:, h:h + 1], block_table[b], n, *args)
            else:
                ns, ws, kv_of = window
                k, v = kv_of(b, h)
                o, lse = tq.decode_attention_tasq_window(qb, cache_block[:, h:h + 1], block_table[b], n,
                                                         int(ns[b]), int(ws[b]), k[:, None, :], v[:, None, :],
                                                         *args)
            res[(b, h)] = (o, lse)
    return res
