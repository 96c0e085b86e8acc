"""Build libloopvq.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m decode_attention_loopvq_amd.build [--debug]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libloopvq.so")
SOURCES = ["abi.hip", "decode.hip", "decode_pg.hip", "decode_tasq.hip", "encode.hip", "kmeans.hip", "tasq.hip", "window.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 math unpacked (no v_pk_*_f32 generated)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs (no AGPR copies around MFMAs)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]


# per-source flags: the encoder's argmax assumes finite scores (no NaN
# canonicalisation around v_max)
SOURCE_FLAGS = {"encode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature" not in l and "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if errs.strip() and verbose:
        print(errs)


def build(verbose: bool = True, extra=None) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    objs = [os.path.join(PKG, "_obj_" + src.replace(".hip", ".o")) for src in SOURCES]
    cmds = [[HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + (extra or []) + ["-c", os.path.join(CSRC, src), "-o", obj]
            for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    for o in objs:
        os.remove(o)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:])
