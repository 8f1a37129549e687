"""GPU parity of the forward pass's per-query log-sum-exp (na2d_forward_lse)
against the float64 oracle on the same seeded inputs, through the C ABI.

Every forward kernel family writes it: the general matrix-core kernel, the
row-streaming kernel (k = 3, 5, 7; at k = 7 maps more than 32 columns wide),
the whole-sub-grid kernel (maps of exactly k*d, k = 3, 5, 7, power-of-two d)
and the per-lane kernel (fp32).  out must stay bit-identical to na2d_forward's.

Tolerance: the fp32 scores carry at most 1e-5 absolute error on these inputs
(the bound the score test of the unfused path holds); lse is 1-Lipschitz in
the scores (max norm), and the fp32 exp2 / log2 of the weights' sum add a
relative 2^-22 each on a value below 10.  2e-5 (times the input scale when q
is scaled up) leaves a factor of about 2.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_transformer_local_amd import inputs as I
from vision_transformer_local_amd import na2d
from vision_transformer_local_amd.inputs import Problem

from parity_util import gpu_inputs, note, sample_indices

pytestmark = pytest.mark.gpu

LSE_TOL = 2e-5

KD = [(1, 1), (3, 1), (3, 2), (5, 1), (5, 2), (7, 1), (7, 2), (7, 3), (7, 8), (9, 1),
      (11, 1), (13, 1), (13, 2)]


def _shapes(ks, d):
    m = ks * d
    return [(m, m), (m + 5, m + 3), (m + 19 * d + 3, m + 37 * d + 1)]


SMALL = [(ks, d, H, W) for ks, d in KD for H, W in _shapes(ks, d)]


def _check(p, g, cpu, idx=None, scale=1.0):
    q, k, v, rpb = g
    out, lse = na2d.forward_lse(q, k, v, rpb, p.kernel_size, p.dilation)
    ref_out = na2d.forward(q, k, v, rpb, p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "out differs from na2d_forward"
    ref = oracle.forward(*cpu, p.kernel_size, p.dilation, idx=idx, lse=True)["lse"].reshape(-1)
    got = lse.cpu().numpy().astype(np.float64).reshape(-1)
    if idx is not None:
        got = got[idx]
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    assert err <= LSE_TOL * scale, "lse error %.3g for %s" % (err, p.describe())
    return err


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("ks,d,H,W", SMALL, ids=lambda x: str(x))
def test_lse_small_maps(ks, d, H, W, dtype):
    p = Problem(2, 2, H, W, 32, ks, d, dtype)
    note("lse %s" % p.describe())
    cpu, g = gpu_inputs(p, seed=ks * 100 + d * 10 + H % 7)
    _check(p, g, cpu)


@pytest.mark.parametrize("p", [Problem(2, 3, 23, 30, 32, 7, 2, "bf16"),
                               Problem(2, 2, 21, 21, 32, 7, 3, "f16"),
                               Problem(1, 2, 17, 19, 32, 5, 1, "f32")],
                         ids=lambda p: p.describe().replace(" ", "_"))
def test_lse_without_bias_table(p):
    note("lse no rpb %s" % p.describe())
    cpu, g = gpu_inputs(p, seed=9)
    cpu = cpu[:3] + (None,)
    g = g[:3] + (None,)
    _check(p, g, cpu)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lse_large_scores(dtype):
    """q scaled by 16 (exact in every dtype): scores reach the hundreds, far
    past exp's fp32 range without the maximum's shift."""
    p = Problem(2, 2, 30, 27, 32, 7, 2, dtype)
    note("lse large scores %s" % p.describe())
    cpu, g = gpu_inputs(p, seed=11)
    cpu = (cpu[0] * 16,) + cpu[1:]
    g = (g[0] * 16,) + g[1:]
    _check(p, g, cpu, scale=16.0)


@pytest.mark.parametrize("p", [I.NAT_TINY_S1, I.DINAT_S1_D8, I.DINAT_S2_D4, I.DETECTION[0]],
                         ids=lambda p: p.describe().replace(" ", "_"))
def test_lse_workloads_full_size(p):
    note("lse full size %s" % p.describe())
    cpu, g = gpu_inputs(p, seed=0)
    idx = sample_indices(p, max_queries=200_000)
    _check(p, g, cpu, idx=idx)


def test_lse_is_deterministic():
    p = Problem(3, 2, 40, 33, 32, 7, 1, "bf16")
    note("lse repeat %s" % p.describe())
    _, (q, k, v, rpb) = gpu_inputs(p, seed=12)
    a = na2d.forward_lse(q, k, v, rpb, 7, 1)
    b = na2d.forward_lse(q, k, v, rpb, 7, 1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
