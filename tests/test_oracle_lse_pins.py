"""Pins for the oracle's per-query log-sum-exp (the natural log of the
softmax denominator over a query's window; the softmax of the blog's
natten2dqkrpb -> softmax(dim=-1) -> natten2dav chain, DiNAT walk-through
blog, "What is DiNAT").  None of them re-types the oracle's loop:

  * q = 0 and no bias: every score is 0, so lse = ln(k*k) exactly;
  * q = 0 with a bias: the scores are the bias entries the window reaches --
    for an interior query the centred (k x k) block of the table, for the
    top-left corner query the bottom-right block (hand-indexed here, summed
    with math.fsum);
  * a constant bias c shifts every score, so lse shifts by exactly c and the
    output does not move (also far beyond exp's range, which only a
    max-shifted sum survives);
  * full-size window (k = H = W): NA is dense attention, so lse is torch's
    logsumexp over all H*W keys of the dense score matrix in float64;
  * consistency: exp(score - lse) reproduces the probabilities.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _problem(B, heads, H, W, D, ks, seed=0, bias_scale=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, heads, H, W, D))
    k = rng.standard_normal((B, heads, H, W, D))
    v = rng.standard_normal((B, heads, H, W, D))
    rpb = bias_scale * rng.standard_normal((heads, 2 * ks - 1, 2 * ks - 1))
    return q, k, v, rpb


@pytest.mark.parametrize("ks,d", [(1, 1), (3, 1), (5, 2), (7, 1), (13, 1)])
def test_equal_scores_give_log_of_window_size(ks, d):
    H, W = ks * d + 2, ks * d + 3
    _, k, v, _ = _problem(2, 2, H, W, 4, ks, seed=ks)
    zeros = np.zeros_like(k)
    r = oracle.forward(zeros, k, v, None, ks, d, lse=True)
    np.testing.assert_allclose(r["lse"], math.log(ks * ks), atol=1e-14, rtol=0)


@pytest.mark.parametrize("ks", [3, 5, 7])
def test_zero_query_lse_is_the_bias_block_logsumexp(ks):
    """Interior query: the window is centred, offsets -k/2..k/2 on both axes,
    i.e. table rows and columns k/2 .. k/2 + k - 1.  Corner query (0, 0): the
    window starts at the query, offsets 0..k-1, i.e. rows and columns
    k-1 .. 2k-2."""
    H = W = 3 * ks
    heads = 2
    _, k, v, rpb = _problem(1, heads, H, W, 4, ks, seed=10 + ks, bias_scale=2.0)
    zeros = np.zeros_like(k)
    r = oracle.forward(zeros, k, v, rpb, ks, 1, lse=True)["lse"]
    c = H // 2
    for h in range(heads):
        centre = rpb[h, ks // 2:ks // 2 + ks, ks // 2:ks // 2 + ks]
        corner = rpb[h, ks - 1:2 * ks - 1, ks - 1:2 * ks - 1]
        want_c = math.log(math.fsum(math.exp(x) for x in centre.ravel()))
        want_0 = math.log(math.fsum(math.exp(x) for x in corner.ravel()))
        assert abs(r[0, h, c, c] - want_c) <= 1e-13
        assert abs(r[0, h, 0, 0] - want_0) <= 1e-13


@pytest.mark.parametrize("shift", [3.25, -40.0, 1000.0, -1000.0])
def test_constant_bias_shifts_lse_and_leaves_output(shift):
    ks, d = 5, 2
    q, k, v, rpb = _problem(1, 2, 13, 12, 8, ks, seed=7)
    a = oracle.forward(q, k, v, rpb, ks, d, lse=True)
    b = oracle.forward(q, k, v, rpb + shift, ks, d, lse=True)
    assert np.isfinite(b["lse"]).all()
    np.testing.assert_allclose(b["lse"], a["lse"] + shift, atol=1e-12 * (1 + abs(shift)), rtol=0)
    np.testing.assert_allclose(b["out"], a["out"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("ks,D", [(3, 4), (7, 32), (13, 8)])
def test_full_window_lse_is_dense_logsumexp(ks, D):
    B, heads = 2, 2
    q, k, v, rpb = _problem(B, heads, ks, ks, D, ks, seed=20 + ks)
    got = oracle.forward(q, k, v, rpb, ks, 1, lse=True)["lse"]
    N = ks * ks
    qf = torch.from_numpy(q.reshape(B, heads, N, D))
    kf = torch.from_numpy(k.reshape(B, heads, N, D))
    ys, xs = np.divmod(np.arange(N), ks)
    dy = ys[None, :] - ys[:, None] + ks - 1  # key row - query row
    dx = xs[None, :] - xs[:, None] + ks - 1
    bias = torch.from_numpy(rpb[:, dy, dx])  # [heads, N (query), N (key)]
    dense = qf @ kf.transpose(-1, -2) * D ** -0.5 + bias[None]
    ref = torch.logsumexp(dense, dim=-1).numpy().reshape(B, heads, ks, ks)
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("ks,d", [(3, 1), (7, 2)])
def test_lse_recovers_probabilities(ks, d):
    q, k, v, rpb = _problem(2, 2, ks * d + 4, ks * d + 1, 8, ks, seed=30 + ks)
    r = oracle.forward(q, k, v, rpb, ks, d, scores=True, probs=True, lse=True)
    np.testing.assert_allclose(np.exp(r["scores"] - r["lse"][..., None]), r["probs"],
                               atol=1e-14, rtol=1e-12)


def test_sampled_lse_matches_full_run():
    q, k, v, rpb = _problem(2, 2, 12, 11, 8, 5, seed=4)
    full = oracle.forward(q, k, v, rpb, 5, 2, lse=True)["lse"].reshape(-1)
    idx = np.array([0, 5, 17, 100, 2 * 2 * 12 * 11 - 1])
    part = oracle.forward(q, k, v, rpb, 5, 2, idx=idx, lse=True)["lse"]
    np.testing.assert_array_equal(part, full[idx])
