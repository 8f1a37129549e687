"""bench.py's command-line contract, checked without a GPU: more than one
GPU is refused with a message and exit status 2, and so is a run on a host
without a GPU (the benchmark has no CPU fallback)."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="host has a GPU")
def test_no_gpu_no_fallback():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""
