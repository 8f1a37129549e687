"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests only).

The tolerances come from the accuracy the library promises: at most 1e-5
absolute error for fp32 data and 2e-2 for bf16 / fp16 data, both against the
float64 oracle fed with the same (already rounded) input values.  For 16-bit
data that budget covers the single rounding of the output (up to 2^-9 |out|
for bf16, |out| < 6 on these inputs) plus the 16-bit probabilities fed to the
P.V product (relative error 2^-9 per weight).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from vision_transformer_local_amd import na2d
from vision_transformer_local_amd.inputs import Problem, make_inputs

TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}


def note(msg: str):
    """Name the case on stderr before any GPU work, so a crash names it."""
    sys.stderr.write("[parity] %s\n" % msg)
    sys.stderr.flush()


def gpu_inputs(p: Problem, seed: int = 0):
    cpu = make_inputs(p, seed)
    return cpu, tuple(t.to("cuda") for t in cpu)


def run_path(path: str, p: Problem, g):
    q, k, v, rpb = g
    if path == "unfused":
        out = na2d.forward_unfused(q, k, v, rpb, p.kernel_size, p.dilation)
    else:
        out = na2d.forward(q, k, v, rpb, p.kernel_size, p.dilation, algo=path)
    torch.cuda.synchronize()
    return out


def sample_indices(p: Problem, max_queries: int, seed: int = 1):
    """All queries when small, else every query of the first and last plane
    (all borders and residue classes) plus a seeded random sample."""
    n = p.n_query_heads
    if n <= max_queries:
        return None
    hw = p.H * p.W
    rng = np.random.default_rng(seed)
    first = np.arange(hw)
    last = np.arange(n - hw, n)
    rand = rng.choice(n, size=max(0, max_queries - 2 * hw), replace=False)
    return np.unique(np.concatenate([first, last, rand]))


def compare(p: Problem, got: torch.Tensor, cpu_inputs, idx=None, tol=None):
    """Max |gpu - oracle| over the selected queries; asserts the tolerance."""
    q, k, v, rpb = cpu_inputs
    ref = oracle.forward(q, k, v, rpb, p.kernel_size, p.dilation, idx=idx)["out"]
    g = got.detach().to("cpu").to(torch.float64).numpy().reshape(-1, p.D)
    if idx is not None:
        g = g[idx]
    ref = ref.reshape(-1, p.D)
    err = float(np.abs(g - ref).max())
    t = TOL[p.dtype] if tol is None else tol
    assert np.isfinite(g).all(), "non-finite output"
    assert err <= t, "max abs error %.3g > %.3g for %s" % (err, t, p.describe())
    return err
