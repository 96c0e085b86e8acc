#!/usr/bin/env python3
"""Throughput of LoopVQ decode attention (32K context) and of the encoder on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--copy-probe] [--skip-encode] [--leg NAME]

One step = one quantised decode-attention call (split-K kernel + combine) of
the long-context workload at one loop step, for all KV and query heads of a
batch of 16 requests with 32768 cached tokens each; the loop step cycles
t = 1..4 from step to step.  The cache it reads was built beforehand by the
GPU encoder from synthetic loop-correlated keys and values.  Beside the
headline the line reports: the same batch with a 64-token bf16 sink and a
256-token bf16 recent window ("window"), the decode-time coding of one 8-token
window page per request ("page_encode"), the split pass with one codebook per
channel group ("per_group"), TaSQ-coded keys on the same batch and the TaSQ
transform + coding of the prefill ("tasq"), the encoder on the prefill of the
1.4B-layer workload (8 x 4096 tokens, "encode"), one k-means Lloyd iteration
over that prefill's coupled vectors ("kmeans"), and under "legs" the decode
of the 1.4B-layer batch, of the GQA ragged batch and of the deep-loop batch
(every loop step), each warm and with the last-level cache flushed, and the
deep-loop prefill encode.  The fp64 oracle is timed on the host beside it: on
one core over a bounded sample, and on all cores (one request per worker
process) over the batch; the same leg checks a sample of the GPU's codes and
decode outputs against it and times the oracle's encoder.
Every timed region is preceded by its warm-up steps and by CLOCK_SETTLE_S of
untimed back-to-back calls.  Prints one JSON line (--leg: that leg only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
# LDS read peak: 256 CUs x 256 B/clk (CDNA4 doubles CDNA3's 128 B/clk LDS read
# rate; a b128 streaming probe measured 208 B/clk/CU) x 2.4 GHz
LDS_PEAK_GBS = 256 * 256 * 2.4
FLUSH_BYTES = 512 << 20        # written between flushed reps: twice the 256 MB last-level cache
METRIC = "decode-attn cached tokens/s (all heads, 1 loop step) @32K ctx; encode vecs/s"
DECODE_KERNEL = "decode_split_kernel"


def _source_sha(files=("decode_split.h", "decode.hip", "common.h", "kernels.h")) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "decode_attention_loopvq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


ENCODE_SOURCES = ("encode.hip", "common.h", "kernels.h")


def _traffic_from_profile(sha: str, name: str = "decode_split_longctx32k_pmc.json"):
    """HBM bytes per launch from committed PMC counters, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


CLOCK_SETTLE_S = 0.25


def settle(fn, torch, seconds: float = CLOCK_SETTLE_S):
    """Run fn(i) back to back for about `seconds` before a timed region.

    The GPU raises its clocks only after tens of milliseconds of continuous
    work; a leg whose warm-up steps last a millisecond or two would otherwise
    time its steps at a clock that is still ramping.  Untimed."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def build_cache(cfg, lv, dims, layer_cb, layer_hsq, lens, bt_np, num_pages, seed, torch, synth, near_tie=None):
    """Encode every request's synthetic K/V (all blocks) into a fresh paged cache on the GPU
    (near_tie: a device int32 counter the encoder adds its near-tie count to, or None)."""
    cache = torch.zeros((cfg.n_blocks, num_pages, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes),
                        dtype=torch.uint8, device="cuda")
    for b, n in enumerate(lens):
        n = int(n)
        if n == 0:
            continue
        xk, xv = synth.make_kv_torch(cfg, n, seed * 1000 + b)
        slots = torch.from_numpy(synth.slot_mapping_for(bt_np, b, n, cfg.page_size)).cuda()
        lv.loopvq_encode(dims, xk, xv, layer_cb, layer_hsq, slots, cache, n_blocks=cfg.n_blocks,
                         block_stride_bytes=cache[0].numel(), near_tie_count=near_tie)
        del xk, xv
    torch.cuda.synchronize()
    return cache


def decode_bytes(cfg, lens):
    """Algorithmic bytes of one split launch: two index rows per (token, KV head), one RoPE-table
    row per position, one block-table entry per page; and the LDS bytes of the slice gathers
    (D/c entries of 2c bytes for K and for V per token and KV head)."""
    tokens = int(np.asarray(lens).sum())
    index_bytes = tokens * cfg.H_kv * 2 * cfg.row_bytes
    rope_bytes = int(np.max(lens)) * cfg.D * 4
    bt_bytes = sum((int(n) + cfg.page_size - 1) // cfg.page_size for n in lens) * 4
    lds = tokens * cfg.H_kv * 2 * cfg.D * 2
    return index_bytes + rope_bytes + bt_bytes, lds


def lds_roof(lds_bytes, ms):
    a = lds_bytes / (ms * 1e-3) / 1e9
    return {"achieved": round(a, 1), "peak": LDS_PEAK_GBS, "unit": "GB/s", "frac": round(a / LDS_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": lds_bytes,
            "what": "slice-entry gathers from LDS (2c bytes per code, K and V)"}


def bench_decode(args, torch, np, synth, lv):
    cfg = synth.config_by_name("longctx32k")
    lens = synth.make_seq_lens(cfg)
    B = len(lens)
    max_seq_len = int(lens.max())
    bt_np, num_pages = synth.make_block_table(cfg, lens)
    dims = lv.loopvq_dims.make(D=cfg.D, c=cfg.c, Tc=cfg.Tc, T=cfg.T, bits=cfg.bits, H_kv=cfg.H_kv,
                               H_q=cfg.H_q, page_size=cfg.page_size, x_dtype=cfg.x_dtype,
                               io_dtype=cfg.io_dtype)
    cb = torch.from_numpy(synth.make_codebooks(cfg)).cuda()
    slices, hsq = lv.loopvq_build_codebook_slices(dims, cb)
    near_tie = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = build_cache(cfg, lv, dims, cb, hsq, lens, bt_np, num_pages, cfg.index, torch, synth, near_tie)
    rope = lv.loopvq_rope_table(max_seq_len, cfg.D, cfg.base).cuda()
    bt = torch.from_numpy(bt_np).cuda()
    seq = torch.from_numpy(lens.astype(np.int32)).cuda()
    qs = [torch.from_numpy(synth.make_queries(cfg, B, t=t)).to(torch.bfloat16).cuda() for t in range(1, cfg.T + 1)]
    out = torch.empty((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, cfg.H_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(lv.loopvq_decode_workspace_bytes(dims, B, max_seq_len), dtype=torch.uint8, device="cuda")

    def step(i, ev=None):
        t = i % cfg.T + 1
        if ev is not None:
            ev[0].record()
        lv.loopvq_decode_split(dims, t, qs[t - 1], cache[0], slices, rope, bt, seq, max_seq_len, ws,
                               max_pos=max_seq_len)
        if ev is not None:
            ev[1].record()
        lv.loopvq_decode_combine(dims, B, seq, max_seq_len, ws, out, lse)

    for i in range(args.warmup):
        step(i)
    settle(step, torch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    split_ms = [a.elapsed_time(b) for a, b in evs]
    per_t = {}
    for i, ms in enumerate(split_ms):
        per_t.setdefault((args.warmup + i) % cfg.T + 1, []).append(ms)
    ms_per_step = ms_total / args.steps
    tokens = int(lens.sum())
    value = tokens / (ms_per_step * 1e-3)
    algo, lds_bytes = decode_bytes(cfg, lens)
    split_avg = float(np.mean(split_ms))
    # one call at t = 1 whose output the oracle checks on the host (cpu_baseline)
    out1 = torch.empty((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    lv.loopvq_decode_attn(dims, 1, qs[0], cache[0], slices, rope, bt, seq, max_seq_len, out=out1,
                          workspace=ws, max_pos=max_seq_len)
    torch.cuda.synchronize()
    achieved = algo / (split_avg * 1e-3) / 1e9
    sha = _source_sha()
    traffic = _traffic_from_profile(sha)
    res = dict(
        value=value, ms_per_step=ms_per_step, wall_s=t_wall, cfg=cfg, lens=lens, max_seq_len=max_seq_len,
        split_avg_ms=split_avg, combine_avg_ms=ms_per_step - split_avg,
        per_t_tokens_per_s={str(t): tokens / (np.mean(v) * 1e-3) for t, v in sorted(per_t.items())},
        roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                  "kernel": DECODE_KERNEL, "algorithmic_bytes_per_launch": algo,
                  "avg_launch_ms": round(split_avg, 5), "source_sha": sha,
                  "lds": lds_roof(lds_bytes, split_avg)},
        cache=cache, bt_np=bt_np, cb=cb, qs=qs, dims=dims, slices=slices, rope=rope, bt=bt, seq=seq,
        out1=out1.float().cpu().numpy(), near_ties=int(near_tie.item()),
        vectors=tokens * cfg.H_kv * 2 * cfg.n_groups * cfg.n_blocks,
    )
    return res


def bench_window(args, torch, np, synth, lv, dec, n_sink=64, n_recent=256):
    """The same 32K batch with a bf16 sink and recent window (whole call: coded split,
    bf16-window kernel, combine)."""
    cfg, dims, lens = dec["cfg"], dec["dims"], dec["lens"]
    B, max_seq_len = len(lens), dec["max_seq_len"]
    ns, ws, pt_np, n_wp = synth.make_window(cfg, lens, n_sink, n_recent)
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.index + 5000)
    kv = torch.randn((n_wp, cfg.H_kv, 2, 8, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    pt = torch.from_numpy(pt_np).cuda()
    ns_d = torch.from_numpy(ns).cuda()
    ws_d = torch.from_numpy(ws).cuda()
    out = torch.empty((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, cfg.H_q), dtype=torch.float32, device="cuda")
    wsp = torch.empty(lv.loopvq_decode_workspace_bytes(dims, B, max_seq_len), dtype=torch.uint8, device="cuda")

    def step(i):
        t = i % cfg.T + 1
        lv.loopvq_decode_attn_window(dims, t, dec["qs"][t - 1], dec["cache"][0], dec["slices"], dec["rope"],
                                     dec["bt"], dec["seq"], max_seq_len, kv, pt, ns_d, ws_d, out=out, lse=lse,
                                     workspace=wsp, max_pos=max_seq_len)
    for i in range(args.warmup):
        step(i)
    settle(step, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbf = int((ns + lens - ws).sum())
    return {"metric": "decode-attn cached tokens/s with a bf16 sink and recent window",
            "value": round(float(lens.sum()) / (ms * 1e-3), 1), "unit": "cached tokens/s",
            "ms_per_call": round(ms, 5),
            "workload": f"{cfg.name} batch, n_sink={n_sink}, window {n_recent}..{n_recent + 7} tokens: "
                        f"{nbf} bf16 tokens and {int(lens.sum()) - nbf} coded tokens per call",
            "bf16_bytes_per_call": nbf * cfg.H_kv * 2 * cfg.D * 2}


def bench_per_group(args, torch, np, synth, lv, dec):
    """The split pass of the same 32K batch with one codebook per channel group:
    the same index cache read through per-group slices."""
    cfg, lens = dec["cfg"], dec["lens"]
    B, max_seq_len = len(lens), dec["max_seq_len"]
    dims = lv.loopvq_dims.make(D=cfg.D, c=cfg.c, Tc=cfg.Tc, T=cfg.T, bits=cfg.bits, H_kv=cfg.H_kv,
                               H_q=cfg.H_q, page_size=cfg.page_size, x_dtype=cfg.x_dtype,
                               io_dtype=cfg.io_dtype, per_group=1)
    cb = torch.from_numpy(synth.make_codebooks_per_group(cfg)).cuda()
    slices, _ = lv.loopvq_build_codebook_slices(dims, cb)
    ws = torch.empty(lv.loopvq_decode_workspace_bytes(dims, B, max_seq_len), dtype=torch.uint8, device="cuda")

    def step(i):
        t = i % cfg.T + 1
        lv.loopvq_decode_split(dims, t, dec["qs"][t - 1], dec["cache"][0], slices, dec["rope"], dec["bt"],
                               dec["seq"], max_seq_len, ws, max_pos=max_seq_len)
    for i in range(args.warmup):
        step(i)
    settle(step, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"metric": "decode split with one codebook per channel group", "ms_per_call": round(ms, 5),
            "value": round(float(lens.sum()) / (ms * 1e-3), 1), "unit": "cached tokens/s (split pass only)",
            "workload": f"{cfg.name} batch, {cfg.n_groups} codebooks per (head, K|V): slices kept unreplicated "
                        "in LDS"}


def bench_tasq(args, torch, np, synth, lv, dec):
    """TaSQ-coded keys on the same 32K batch: the whole decode call (split pass with
    the weight-folded query, permuted RoPE rows and per-token sigma, then the
    combine), and the transform + coding of the 1.4B-layer prefill."""
    cfg, dims, lens = dec["cfg"], dec["dims"], dec["lens"]
    B, max_seq_len = len(lens), dec["max_seq_len"]
    w_np, perm_np = synth.make_tasq(cfg)
    w, perm = torch.from_numpy(w_np).cuda(), torch.from_numpy(perm_np).cuda()
    n_slots = dec["cache"].shape[1] * cfg.page_size
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.index + 7000)
    sigma = torch.exp(0.3 * torch.randn((cfg.T, n_slots), generator=g, device="cuda")).to(torch.float16)
    out = torch.empty((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, cfg.H_q), dtype=torch.float32, device="cuda")
    wsp = torch.empty(lv.loopvq_decode_workspace_bytes(dims, B, max_seq_len), dtype=torch.uint8, device="cuda")

    def step(i):
        t = i % cfg.T + 1
        lv.loopvq_decode_attn_tasq(dims, t, dec["qs"][t - 1], dec["cache"][0], dec["slices"], dec["rope"],
                                   dec["bt"], dec["seq"], max_seq_len, w, perm, sigma, out=out, lse=lse,
                                   workspace=wsp, max_pos=max_seq_len)
    for i in range(args.warmup):
        step(i)
    settle(step, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    res = {"metric": "decode-attn cached tokens/s with TaSQ-coded keys", "ms_per_call": round(ms, 5),
           "value": round(float(lens.sum()) / (ms * 1e-3), 1), "unit": "cached tokens/s",
           "workload": f"{cfg.name} batch, synthetic w and P, per-token fp16 sigma (2 bytes per token "
                       "and loop step beside the index rows)",
           "sigma_bytes_per_call": int(lens.sum()) * 2}
    if args.skip_encode:
        return res
    ecfg = synth.config_by_name("layer1p4b")
    n_tok = ecfg.encode_batch * ecfg.encode_tokens
    elens = np.full(ecfg.encode_batch, ecfg.encode_tokens)
    bt_np, num_pages = synth.make_block_table(ecfg, elens)
    slots = torch.from_numpy(np.concatenate([synth.slot_mapping_for(bt_np, b, int(n), ecfg.page_size)
                                             for b, n in enumerate(elens)])).cuda()
    edims = lv.loopvq_dims.make(D=ecfg.D, c=ecfg.c, Tc=ecfg.Tc, T=ecfg.T, bits=ecfg.bits, H_kv=ecfg.H_kv,
                                H_q=ecfg.H_q, page_size=ecfg.page_size, x_dtype=ecfg.x_dtype,
                                io_dtype=ecfg.io_dtype)
    cb = torch.from_numpy(synth.make_codebooks(ecfg)).cuda()
    _, hsq = lv.loopvq_build_codebook_slices(edims, cb)
    xk, xv = synth.make_kv_torch(ecfg, n_tok, 78)
    ew, eperm = (torch.from_numpy(a).cuda() for a in synth.make_tasq(ecfg))
    esig = torch.zeros((ecfg.T, num_pages * ecfg.page_size), dtype=torch.float16, device="cuda")
    cache = torch.zeros((num_pages, ecfg.H_kv, 2, ecfg.page_size, ecfg.row_bytes), dtype=torch.uint8,
                        device="cuda")
    ews = torch.empty(lv.loopvq_encode_tasq_workspace_bytes(edims, n_tok, ecfg.n_blocks), dtype=torch.uint8,
                      device="cuda")
    reps = max(3, args.steps // 4)
    for _ in range(2):
        lv.loopvq_encode_tasq(edims, xk, xv, ew, eperm, esig, cb, hsq, slots, cache, workspace=ews)
    settle(lambda i: lv.loopvq_encode_tasq(edims, xk, xv, ew, eperm, esig, cb, hsq, slots, cache, workspace=ews),
           torch)
    e0.record()
    for _ in range(reps):
        lv.loopvq_encode_tasq(edims, xk, xv, ew, eperm, esig, cb, hsq, slots, cache, workspace=ews)
    e1.record()
    torch.cuda.synchronize()
    ems = e0.elapsed_time(e1) / reps
    vecs = n_tok * ecfg.H_kv * 2 * ecfg.n_groups * ecfg.n_blocks
    res["encode"] = {"metric": "encode vecs/s with TaSQ-coded keys", "value": round(vecs / (ems * 1e-3), 1),
                     "unit": "coupled vectors/s", "ms_per_call": round(ems, 5),
                     "workload": f"{ecfg.name}: transform + coding of {ecfg.encode_batch} x {ecfg.encode_tokens} "
                                 "tokens (keys from fp32 u, values from bf16)"}
    del ews, xk, xv
    return res


def bench_kmeans(args, torch, np, synth, lv):
    """One Lloyd iteration of plain k-means over the coupled vectors of the 1.4B-layer
    prefill (8 x 4096 tokens, 16 KV heads, K and V): assignment by the encoder, then the
    codebook update."""
    cfg = synth.config_by_name("layer1p4b")
    n_tok = cfg.encode_batch * cfg.encode_tokens
    lens = np.full(cfg.encode_batch, cfg.encode_tokens)
    bt_np, num_pages = synth.make_block_table(cfg, lens)
    slots = torch.from_numpy(np.concatenate([synth.slot_mapping_for(bt_np, b, int(n), cfg.page_size)
                                             for b, n in enumerate(lens)])).cuda()
    dims = lv.loopvq_dims.make(D=cfg.D, c=cfg.c, Tc=cfg.Tc, T=cfg.T, bits=cfg.bits, H_kv=cfg.H_kv,
                               H_q=cfg.H_q, page_size=cfg.page_size, x_dtype=cfg.x_dtype,
                               io_dtype=cfg.io_dtype)
    cb = torch.from_numpy(synth.make_codebooks(cfg)).cuda()
    cb2 = torch.empty_like(cb)
    err = torch.zeros((cfg.n_blocks, cfg.H_kv, 2, 2), dtype=torch.float64, device="cuda")
    wsk = torch.empty(lv.loopvq_kmeans_workspace_bytes(dims, cfg.n_blocks), dtype=torch.uint8, device="cuda")
    xk, xv = synth.make_kv_torch(cfg, n_tok, 79)
    cache = torch.zeros((num_pages, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    _, hsq = lv.loopvq_build_codebook_slices(dims, cb)

    def iteration(src, dst):
        lv.loopvq_build_codebook_slices(dims, src, hsq=hsq, slices=slices_buf)
        lv.loopvq_encode(dims, xk, xv, src, hsq, slots, cache)
        lv.loopvq_kmeans_update(dims, xk, xv, slots, cache, src, cb_out=dst, err=err, workspace=wsk)
    slices_buf = torch.empty((cfg.T, cfg.H_kv, 2, cfg.K, cfg.c), dtype=torch.float16, device="cuda")
    iteration(cb, cb2)
    iteration(cb2, cb)
    settle(lambda i: iteration(cb if i % 2 == 0 else cb2, cb2 if i % 2 == 0 else cb), torch)
    reps = max(3, args.steps // 8)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eu0, eu1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        iteration(cb if i % 2 == 0 else cb2, cb2 if i % 2 == 0 else cb)
    e1.record()
    eu0.record()
    lv.loopvq_kmeans_update(dims, xk, xv, slots, cache, cb, cb_out=cb2, err=err, workspace=wsk)
    eu1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    vecs = n_tok * cfg.H_kv * 2 * cfg.n_groups * cfg.n_blocks
    e = err.cpu().numpy()
    del xk, xv
    return {"metric": "k-means Lloyd iterations/s", "value": round(1e3 / ms, 2), "unit": "iterations/s",
            "ms_per_iteration": round(ms, 4), "update_ms": round(eu0.elapsed_time(eu1), 4),
            "workload": f"{cfg.name}: {vecs} coupled vectors (8 x 4096 tokens, H_kv={cfg.H_kv}, K and V, G={cfg.G}), "
                        f"K={cfg.K}: slices + assignment (encoder) + codebook update",
            "nmse_after": round(float(e[..., 0].sum() / e[..., 1].sum()), 5)}


def bench_page_encode(args, torch, np, synth, lv, dec):
    """Decode-time page encoding at the 32K batch's shape: the oldest 8-token bf16
    window page of each of the 16 requests, coded for all loop steps at once."""
    cfg, dims = dec["cfg"], dec["dims"]
    B = len(dec["lens"])
    n_pool = 8 * B
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.index + 6000)
    pool = torch.randn((cfg.T, n_pool, cfg.H_kv, 2, 8, cfg.D), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(cfg.index + 6001)
    pages = rng.permutation(n_pool)[:B]
    src = torch.from_numpy((pages[:, None] * 8 + np.arange(8)[None, :]).reshape(-1).astype(np.int32)).cuda()
    cache = torch.zeros((B, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8, device="cuda")
    slots = torch.from_numpy((np.arange(B)[:, None] * cfg.page_size + np.arange(8)[None, :])
                             .reshape(-1).astype(np.int32)).cuda()
    _, hsq = lv.loopvq_build_codebook_slices(dims, dec["cb"])
    for _ in range(args.warmup):
        lv.loopvq_encode_pages(dims, pool, src, dec["cb"], hsq, slots, cache)
    settle(lambda i: lv.loopvq_encode_pages(dims, pool, src, dec["cb"], hsq, slots, cache), torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        lv.loopvq_encode_pages(dims, pool, src, dec["cb"], hsq, slots, cache)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"metric": "decode-time page encode latency", "value": round(ms * 1e3, 2), "unit": "us per call",
            "workload": f"{B} requests x 8 tokens, {cfg.T} loop steps ({cfg.n_blocks} block), H_kv={cfg.H_kv}, "
                        f"D={cfg.D}, c={cfg.c}, K={cfg.K}: {B * 8 * cfg.H_kv * 2 * cfg.n_groups} coupled vectors",
            "higher_is_better": False}


def bench_decode_config(args, torch, np, synth, lv, name):
    """Decode of another workload (split + combine), its cache built by the GPU encoder: warm
    (the cache may sit in the last-level cache between calls) and with that cache flushed
    (FLUSH_BYTES written between calls), per loop step, with HBM and LDS roofs of the split."""
    cfg = synth.config_by_name(name)
    lens = synth.make_seq_lens(cfg)
    B, msl = len(lens), int(lens.max())
    bt_np, num_pages = synth.make_block_table(cfg, lens)
    dims = lv.loopvq_dims.make(D=cfg.D, c=cfg.c, Tc=cfg.Tc, T=cfg.T, bits=cfg.bits, H_kv=cfg.H_kv,
                               H_q=cfg.H_q, page_size=cfg.page_size, x_dtype=cfg.x_dtype,
                               io_dtype=cfg.io_dtype)
    cb = torch.from_numpy(synth.make_codebooks(cfg)).cuda()
    slices, hsq = lv.loopvq_build_codebook_slices(dims, cb)
    cache = build_cache(cfg, lv, dims, cb, hsq, lens, bt_np, num_pages, cfg.index, torch, synth)
    rope = lv.loopvq_rope_table(msl, cfg.D, cfg.base).cuda()
    bt = torch.from_numpy(bt_np).cuda()
    seq = torch.from_numpy(lens.astype(np.int32)).cuda()
    ts = list(range(1, cfg.T + 1))
    qs = {t: torch.from_numpy(synth.make_queries(cfg, B, t=t)).to(torch.bfloat16).cuda() for t in ts}
    out = torch.empty((B, cfg.H_q, cfg.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lv.loopvq_decode_workspace_bytes(dims, B, msl), dtype=torch.uint8, device="cuda")
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def split(t):
        lv.loopvq_decode_split(dims, t, qs[t], cache[(t - 1) // cfg.Tc], slices, rope, bt, seq, msl, ws,
                               max_pos=msl)

    def combine():
        lv.loopvq_decode_combine(dims, B, seq, msl, ws, out)

    def timed(n_reps, flushed):
        """per-t lists of (split ms, whole-call ms), t cycling 1..T"""
        res = {t: [] for t in ts}
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_reps)]
        for i in range(n_reps):
            t = ts[i % len(ts)]
            if flushed:
                flush.fill_(i & 255)
            evs[i][0].record()
            split(t)
            evs[i][1].record()
            combine()
            evs[i][2].record()
        torch.cuda.synchronize()
        for i, (a, b, c) in enumerate(evs):
            res[ts[i % len(ts)]].append((a.elapsed_time(b), a.elapsed_time(c)))
        return res

    for i in range(args.warmup):
        split(ts[i % len(ts)])
        combine()
    settle(lambda i: (split(ts[i % len(ts)]), combine()), torch)
    reps = max(args.steps, 3 * len(ts))
    warm = timed(reps, False)
    cold = timed(max(args.steps // 2, 2 * len(ts)), True)
    tokens = int(lens.sum())
    algo, lds_bytes = decode_bytes(cfg, lens)

    def summary(r):
        sp = float(np.mean([x[0] for v in r.values() for x in v]))
        wh = float(np.mean([x[1] for v in r.values() for x in v]))
        a = algo / (sp * 1e-3) / 1e9
        return {"value": round(tokens / (wh * 1e-3), 1), "unit": "cached tokens/s", "ms_per_call": round(wh, 5),
                "split_ms": round(sp, 5),
                "roofline": {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(a / HBM_PEAK_GBS, 4), "kernel": DECODE_KERNEL,
                             "algorithmic_bytes_per_launch": algo, "avg_launch_ms": round(sp, 5),
                             "lds": lds_roof(lds_bytes, sp)},
                "per_loop_step_split_ms": {str(t): round(float(np.mean([x[0] for x in v])), 5)
                                           for t, v in r.items()}}
    out_d = {"metric": "decode-attn cached tokens/s (all heads, 1 loop step)",
             "workload": f"{cfg.name}: B={B}, tokens {tokens} ({int(lens.min())}..{msl} per request), "
                         f"H_kv={cfg.H_kv}, H_q={cfg.H_q}, D={cfg.D}, c={cfg.c}, Tc={cfg.Tc}, T={cfg.T}, "
                         f"K={cfg.K}, P={cfg.page_size}; cache from the GPU encoder, t cycling 1..{cfg.T}",
             "warm": summary(warm), "mall_flushed": summary(cold),
             "flush": f"{FLUSH_BYTES >> 20} MiB written between flushed calls (not timed)"}
    del cache, flush
    return out_d


def bench_encode_cfg(args, torch, np, synth, lv, name):
    """Prefill encode of a configuration's encode batch (all blocks), with an MFMA roofline."""
    cfg = synth.config_by_name(name)
    n_tok = cfg.encode_batch * cfg.encode_tokens
    lens = np.full(cfg.encode_batch, cfg.encode_tokens)
    bt_np, num_pages = synth.make_block_table(cfg, lens)
    slots = torch.from_numpy(np.concatenate([synth.slot_mapping_for(bt_np, b, int(n), cfg.page_size)
                                             for b, n in enumerate(lens)])).cuda()
    dims = lv.loopvq_dims.make(D=cfg.D, c=cfg.c, Tc=cfg.Tc, T=cfg.T, bits=cfg.bits, H_kv=cfg.H_kv,
                               H_q=cfg.H_q, page_size=cfg.page_size, x_dtype=cfg.x_dtype,
                               io_dtype=cfg.io_dtype)
    cb = torch.from_numpy(synth.make_codebooks(cfg)).cuda()
    _, hsq = lv.loopvq_build_codebook_slices(dims, cb)
    xk, xv = synth.make_kv_torch(cfg, n_tok, 77)
    cache = torch.zeros((cfg.n_blocks, num_pages, cfg.H_kv, 2, cfg.page_size, cfg.row_bytes), dtype=torch.uint8,
                        device="cuda")

    def enc(_=0):
        lv.loopvq_encode(dims, xk, xv, cb, hsq, slots, cache, n_blocks=cfg.n_blocks,
                         block_stride_bytes=cache[0].numel())
    reps = max(3, args.steps // 4)
    for _ in range(2):
        enc()
    settle(enc, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        enc()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    vecs = n_tok * cfg.H_kv * 2 * cfg.n_groups * cfg.n_blocks
    flops = vecs * 2 * cfg.G * cfg.K
    tflops = flops / (ms * 1e-3) / 1e12
    del xk, xv, cache
    return {"metric": "encode vecs/s", "value": round(vecs / (ms * 1e-3), 1), "unit": "coupled vectors/s",
            "ms_per_call": round(ms, 5),
            "workload": f"{cfg.name}: prefill encode of {cfg.encode_batch} x {cfg.encode_tokens} tokens, "
                        f"{cfg.n_blocks} block(s), H_kv={cfg.H_kv}, D={cfg.D}, c={cfg.c}, Tc={cfg.Tc}, K={cfg.K}",
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": (_traffic_from_profile(_source_sha(ENCODE_SOURCES), "encode_layer1p4b_pmc.json")
                                     if name == "layer1p4b" else None),
                         "kernel": "encode_kernel", "algorithmic_flops_per_launch": flops}}


def code_sample_check(np, synth, dec, n_tok: int = 96):
    """GPU codes of the bench's cache against the oracle's nearest entries on a sample: the first
    n_tok tokens of request 0, every head, K and V (the K/V drawn again from the same seed)."""
    import oracle  # test infrastructure: used only for this check
    import torch
    cfg = dec["cfg"]
    xk, xv = synth.make_kv_torch(cfg, int(dec["lens"][0]), cfg.index * 1000 + 0)
    xk = xk[:, :n_tok].float().cpu().numpy()
    xv = xv[:, :n_tok].float().cpu().numpy()
    slots = synth.slot_mapping_for(dec["bt_np"], 0, n_tok, cfg.page_size).astype(np.int64)
    cache = dec["cache"][0].cpu().numpy()
    cb = dec["cb"].cpu().numpy()
    P = cfg.page_size
    ties = bad = n = 0
    for h in range(cfg.H_kv):
        for kv, x in enumerate((xk, xv)):
            rows = cache[slots // P, h, kv, slots % P, :]
            got = oracle.slots_to_groups(oracle.unpack_rows(rows, cfg.bits, cfg.n_groups)).reshape(-1)
            z = oracle.coupled_vectors(x[:, :, h, :], cfg.Tc, cfg.c, 0).reshape(-1, cfg.G)
            E = cb[0, h, kv].astype(np.float64)
            res = oracle.nearest_entry(z, E, method="gemm")
            ties += int(res.near_tie.sum())
            bad += int((~oracle.accepts(z, E, res, got)).sum())
            n += len(z)
    del xk, xv
    torch.cuda.empty_cache()
    return {"vectors": n, "oracle_near_ties": ties, "mismatches_outside_band": bad,
            "sample": f"first {n_tok} tokens of request 0, all {cfg.H_kv} heads, K and V"}


def cpu_encode_baseline(np, synth, budget_s: float = 10.0):
    """The oracle's encoder (fp64, BLAS form with direct-difference rechecks) on a bounded sample of
    the 1.4B-layer prefill: on one core, and with BLAS on all host cores."""
    import oracle  # test infrastructure: used only for this reference timing
    from threadpoolctl import threadpool_limits
    cfg = synth.config_by_name("layer1p4b")
    xk, xv = synth.make_kv(cfg, 256, seed=cfg.index + 9000)
    cb = synth.make_codebooks(cfg)

    def run(limit):
        vecs = 0
        t0 = time.perf_counter()
        with threadpool_limits(limits=limit):
            while time.perf_counter() - t0 < budget_s:
                for h in range(cfg.H_kv):
                    for kv, x in enumerate((xk, xv)):
                        idx, _ = oracle.encode_stream(x[:, :, h, :], cb[0, h, kv], cfg.Tc, cfg.c, 0, method="gemm")
                        vecs += idx.size
                    if time.perf_counter() - t0 >= budget_s:
                        break
        return vecs, time.perf_counter() - t0
    v1, t1 = run(1)
    # all cores: one (head, K|V) stream per task over spawned workers, one BLAS thread each
    import concurrent.futures
    import multiprocessing
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(16, avail))
    tasks = [(x[:, :, h, :], cb[0, h, kv], cfg.Tc, cfg.c) for h in range(cfg.H_kv)
             for kv, x in enumerate((xk, xv))] * 8
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        list(ex.map(_oracle_worker_start, range(workers)))
        t0 = time.perf_counter()
        va = sum(ex.map(_oracle_encode_stream, tasks))
        ta = time.perf_counter() - t0
    return {"value": round(v1 / t1, 1), "unit": "coupled vectors/s", "cores": 1, "kind": "oracle",
            "sample": f"layer1p4b coupled vectors of 256 tokens, (head, K|V) streams in turn, {v1} vectors in "
                      f"{t1:.1f} s; fp64 BLAS form (nearest_entry method gemm), 1 BLAS thread",
            "all_cores": {"value": round(va / ta, 1), "unit": "coupled vectors/s", "cores": workers,
                          "kind": "oracle",
                          "sample": f"the same streams 8 times over, one stream per task on {workers} worker "
                                    f"processes (one BLAS thread each), {va} vectors in {ta:.1f} s"}}


def _oracle_encode_stream(task):
    """One (head, K|V) stream of the encode sample through the oracle's encoder."""
    import oracle
    from threadpoolctl import threadpool_limits
    x, E, Tc, c = task
    with threadpool_limits(limits=1):
        idx, _ = oracle.encode_stream(x, E, Tc, c, 0, method="gemm")
    return int(idx.size)


def cpu_baseline(np, synth, dec, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample of the same decode workload, one core."""
    import oracle  # test infrastructure: used only for this reference timing
    from threadpoolctl import threadpool_limits
    cfg = dec["cfg"]
    cache = dec["cache"][0].cpu().numpy()
    cb = dec["cb"].cpu().numpy()
    q = dec["qs"][0].float().cpu().numpy()
    lens = dec["lens"]
    model, nproc = _cpu_info()
    done_tokens = 0
    done_req = 0
    t0 = time.perf_counter()
    worst = worst_ratio = 0.0
    with threadpool_limits(limits=1):
        for b in range(len(lens)):
            o, _ = oracle.decode_attention(q[b], cache, dec["bt_np"][b], int(lens[b]), cb[0], 1, cfg.Tc, cfg.c,
                                           cfg.bits, cfg.base)
            err = np.abs(dec["out1"][b] - o)
            # bf16 output: 2e-3 plus half a bf16 ulp of the reference
            bound = 2e-3 + 0.5 * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(o), 1e-30))) - 7)
            worst = max(worst, float(err.max()))
            worst_ratio = max(worst_ratio, float((err / bound).max()))
            done_tokens += int(lens[b])
            done_req += 1
            if time.perf_counter() - t0 > budget_s:
                break
    el = time.perf_counter() - t0
    return {"value": done_tokens / el, "unit": "cached tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done_req} of {len(lens)} requests of the same 32K-context batch (all 16 KV heads, "
                      f"loop step 1), fp64 NumPy with BLAS limited to 1 thread, {el:.1f} s",
            "cpu_model": model, "host_cpus": nproc,
            "gpu_vs_oracle": {"requests": done_req, "max_abs_err": worst, "max_bound_ratio": round(worst_ratio, 3),
                              "bound": "2e-3 + half a bf16 ulp of the oracle output"}}


def _oracle_worker_start(_):
    """Warm a worker of the all-cores baseline (imports the oracle, one BLAS thread)."""
    import oracle  # noqa: F401  (test infrastructure: used only for this reference timing)
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    return os.getpid()


def _oracle_request(task):
    """One request of the decode workload through the oracle, on the request's own pages."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    q, pages, n, cb, Tc, c, bits, base = task
    with threadpool_limits(limits=1):
        oracle.decode_attention(q, pages, np.arange(pages.shape[0], dtype=np.int32), n, cb, 1, Tc, c, bits, base)
    return n


def cpu_baseline_all_cores(np, dec, max_workers: int = 16):
    """The same oracle over every request of the batch, one request per worker process
    (spawned, one BLAS thread each) on the host's cores; each task carries only its
    request's pages.  Worker start-up is excluded from the timing."""
    import concurrent.futures
    import multiprocessing
    cfg = dec["cfg"]
    cache = dec["cache"][0].cpu().numpy()
    cb = dec["cb"].cpu().numpy()[0]
    q = dec["qs"][0].float().cpu().numpy()
    lens, bt = dec["lens"], dec["bt_np"]
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    workers = max(1, min(max_workers, avail, len(lens)))
    tasks = []
    for b in range(len(lens)):
        n = int(lens[b])
        npg = (n + cfg.page_size - 1) // cfg.page_size
        tasks.append((q[b], np.ascontiguousarray(cache[bt[b][:npg]]), n, cb, cfg.Tc, cfg.c, cfg.bits, cfg.base))
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        list(ex.map(_oracle_worker_start, range(workers)))
        t0 = time.perf_counter()
        tokens = sum(ex.map(_oracle_request, tasks))
        el = time.perf_counter() - t0
    return {"value": tokens / el, "unit": "cached tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"all {len(lens)} requests of the same 32K-context batch (all 16 KV heads, loop "
                      f"step 1), one request per worker process, {el:.1f} s wall"}


# --leg names: (kind, workload)
LEGS = {"headline": ("headline", "longctx32k"),
        "decode_layer1p4b": ("decode", "layer1p4b"), "decode_gqa_ragged": ("decode", "gqa_ragged"),
        "decode_deeploop": ("decode", "deeploop"),
        "encode_layer1p4b": ("encode", "layer1p4b"), "encode_deeploop": ("encode", "deeploop")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-encode", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB copy kernel (reference for PMC byte counters)")
    ap.add_argument("--leg", choices=sorted(LEGS), default=None,
                    help="run one leg only and print its JSON (for profiler runs); not the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the decode path is not sharded "
              "across GPUs", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")

    import numpy as np
    import torch
    import synth
    import decode_attention_loopvq_amd as lv
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    lv.lib()  # fail loudly if the HIP library is missing

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.leg is not None:
        kind, name = LEGS[args.leg]
        if kind == "headline":
            r = bench_decode(args, torch, np, synth, lv)
            r = {k: r[k] for k in ("value", "ms_per_step", "split_avg_ms", "roofline")}
        elif kind == "decode":
            r = bench_decode_config(args, torch, np, synth, lv, name)
        else:
            r = bench_encode_cfg(args, torch, np, synth, lv, name)
        print(json.dumps({"leg": args.leg, **r}), flush=True)
        return

    dec = bench_decode(args, torch, np, synth, lv)
    win = bench_window(args, torch, np, synth, lv, dec)
    penc = bench_page_encode(args, torch, np, synth, lv, dec)
    pgr = bench_per_group(args, torch, np, synth, lv, dec)
    tqr = bench_tasq(args, torch, np, synth, lv, dec)
    legs = {}
    for leg in ("decode_layer1p4b", "decode_gqa_ragged", "decode_deeploop"):
        legs[leg] = bench_decode_config(args, torch, np, synth, lv, LEGS[leg][1])
        torch.cuda.empty_cache()
    enc = kms = None
    if not args.skip_encode:
        enc = bench_encode_cfg(args, torch, np, synth, lv, "layer1p4b")
        legs["encode_deeploop"] = bench_encode_cfg(args, torch, np, synth, lv, "deeploop")
        kms = bench_kmeans(args, torch, np, synth, lv)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, synth, dec)
        cpu["all_cores"] = cpu_baseline_all_cores(np, dec)
        cpu["gpu_vs_oracle"]["codes"] = code_sample_check(np, synth, dec)
        cpu["encode"] = cpu_encode_baseline(np, synth)
    cfg = dec["cfg"]
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 1),
        "unit": "cached tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 q/out; fp16 MFMA operands (codebooks, q, p); fp32 accumulate and RoPE",
        "data": "synthetic (loop-correlated Gaussian K/V encoded on the GPU; fp16 codebooks from a "
                "synthetic calibration set; bf16 queries)",
        "config": {"workload": f"{cfg.name}: decode attention, B={len(dec['lens'])}, N={dec['max_seq_len']}, "
                               f"H_kv=H_q={cfg.H_kv}, D={cfg.D}, c={cfg.c}, Tc={cfg.Tc}, K={cfg.K} (8-bit), "
                               f"P={cfg.page_size}, one loop step per call, t cycling 1..4",
                   "global_batch": len(dec["lens"]), "seq_len": dec["max_seq_len"], "parallelism": "none (1 GPU)"},
        "clock_settle_s_per_leg": CLOCK_SETTLE_S,
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_split_ms": round(dec["split_avg_ms"], 5),
        "decode_combine_ms": round(dec["combine_avg_ms"], 5),
        "per_loop_step_tokens_per_s": {k: round(v, 1) for k, v in dec["per_t_tokens_per_s"].items()},
        "window": win,
        "page_encode": penc,
        "per_group": pgr,
        "tasq": tqr,
        "encode": enc,
        "kmeans": kms,
        "legs": legs,
        "near_ties": {"gpu_count": dec["near_ties"], "vectors_encoded": dec["vectors"],
                      "what": "vectors of the timed cache whose two best distances lie within 1e-6*(||z||^2 + "
                              "||e||^2), counted by the encoder while it built that cache"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
