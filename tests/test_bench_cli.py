"""bench.py's command line on a host without a GPU: it measures one GPU only
and refuses more, and it fails loudly rather than timing anything on the CPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a run that did not happen


def test_no_gpu_no_number():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline", "--skip-encode")
    assert r.returncode == 1
    assert "needs an MI355X GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_zero_steps_is_refused():
    r = _run("--steps", "0")
    assert r.returncode == 2
    assert "--steps must be at least 1" in r.stderr
