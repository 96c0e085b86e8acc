"""The C ABI from a plain C11 program: tests/c/abi_consumer.c is compiled with
gcc against include/loopvq.h (as C, not C++) and linked to libloopvq.so; it
exercises the host-side entry points and the argument checks that run before
any launch, so it needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_loopvq_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(PKG, "libloopvq.so")
    assert os.path.exists(lib), "build the library first (python -m decode_attention_loopvq_amd.build)"
    exe = tmp_path / "abi_consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", str(exe),
           "-L", PKG, "-lloopvq", f"-Wl,-rpath,{PKG}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.pathsep.join([PKG, os.path.join(ROCM, "lib"), env.get("LD_LIBRARY_PATH", "")])
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
