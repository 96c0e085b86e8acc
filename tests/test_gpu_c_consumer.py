"""Decode attention through the C ABI from a C program with no PyTorch in its
process: tests/c/decode_consumer.c is built with gcc against include/loopvq.h
and the HIP runtime, reads inputs this test writes (the 1.4B-layer shape, a
ragged batch of three requests, a cache of random codes), builds the slices
and the RoPE table itself, calls loopvq_decode_attn and writes out and lse,
which are checked against the fp64 oracle (2e-3 + half a bf16 ulp, lse 1e-4).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from gpu_util import compare, ref_decode

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_loopvq_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_decodes(tmp_path):
    exe = tmp_path / "decode_consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "decode_consumer.c"), "-o", str(exe),
           "-L", PKG, "-lloopvq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr

    cfg = synth.config_by_name("layer1p4b")
    lens = np.array([700, 1, 300], dtype=np.int32)
    B, t = len(lens), 2
    msl = int(lens.max())
    bt, npg = synth.make_block_table(cfg, lens)
    cache = synth.random_index_cache(cfg, npg, 91)
    cb = synth.make_codebooks(cfg)
    q = synth.make_queries(cfg, B, t=t)
    d = tmp_path / "io"
    d.mkdir()
    (d / "meta.txt").write_text(" ".join(str(v) for v in (
        cfg.D, cfg.c, cfg.Tc, cfg.T, cfg.bits, cfg.H_kv, cfg.H_q, cfg.page_size, B, t, msl, bt.shape[1], npg)))
    (d / "cb.bin").write_bytes(np.ascontiguousarray(cb, dtype=np.float16).tobytes())
    # q holds bf16 values: the top 16 bits of each fp32 are its bf16 code
    (d / "q.bin").write_bytes((np.ascontiguousarray(q, dtype=np.float32).view(np.uint32) >> 16)
                              .astype(np.uint16).tobytes())
    (d / "cache.bin").write_bytes(np.ascontiguousarray(cache[(t - 1) // cfg.Tc] if cache.ndim == 6 else cache,
                                                       dtype=np.uint8).tobytes())
    (d / "bt.bin").write_bytes(np.ascontiguousarray(bt, dtype=np.int32).tobytes())
    (d / "lens.bin").write_bytes(lens.tobytes())
    print("running the C decode program", flush=True)
    r = subprocess.run([str(exe), str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr

    out_bits = np.fromfile(d / "out.bin", dtype=np.uint16).astype(np.uint32) << 16
    o = out_bits.view(np.float32).reshape(B, cfg.H_q, cfg.D).astype(np.float64)
    lse = np.fromfile(d / "lse.bin", dtype=np.float32).reshape(B, cfg.H_q).astype(np.float64)
    ref = ref_decode(cfg, t, q, cache, bt, lens, cb)
    err, ratio = compare(cfg, o, lse, ref, lens)
    print(f"C program decode: max err {err:.2e} (bound ratio {ratio:.2f})", flush=True)
    assert ratio <= 1.0
