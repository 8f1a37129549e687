"""Pins for the oracle's backward pass (gradients of sum(out * dout)).

None of these re-types the oracle's loops:
  * central finite differences of the oracle's own forward pass (float64),
    element by element, for q, k, v and the bias table;
  * at full size (window = image, NAT repository README, introduction) and
    per residue class for H = W = k*d, the operator is dense attention with a
    bias: torch autograd through a dense float64 formulation;
  * dilated NA is NA on each strided sub-grid (DiNAT walk-through blog, "What
    is DiNAT"), so the dilated gradients equal those of the sub-grid problems;
  * invariants: the softmax rows sum to one, so the bias gradient of every
    head sums to zero; k = 1 gives out = v, hence dv = dout and no other
    gradient.
"""
import numpy as np
import pytest
import torch

import oracle


def _problem(B, heads, H, W, D, ks, seed):
    rng = np.random.default_rng(seed)
    q, k, v, dout = (rng.standard_normal((B, heads, H, W, D)) for _ in range(4))
    rpb = 0.5 * rng.standard_normal((heads, 2 * ks - 1, 2 * ks - 1))
    return q, k, v, rpb, dout


def _loss(q, k, v, rpb, dout, ks, d):
    return float((oracle.forward(q, k, v, rpb, ks, d, threads=1)["out"] * dout).sum())


FD_CASES = [(1, 2, 6, 7, 3, 3, 1), (1, 1, 7, 8, 2, 3, 2), (1, 1, 5, 5, 2, 5, 1),
            (2, 1, 5, 6, 2, 1, 1)]


@pytest.mark.parametrize("B,heads,H,W,D,ks,d", FD_CASES)
def test_finite_differences(B, heads, H, W, D, ks, d):
    q, k, v, rpb, dout = _problem(B, heads, H, W, D, ks, seed=H * W + ks)
    g = oracle.backward(q, k, v, rpb, dout, ks, d, threads=1)
    eps = 1e-5
    for name, arr in (("dq", q), ("dk", k), ("dv", v), ("drpb", rpb)):
        num = np.empty_like(arr)
        flat, nflat = arr.reshape(-1), num.reshape(-1)
        for t in range(flat.size):
            keep = flat[t]
            flat[t] = keep + eps
            up = _loss(q, k, v, rpb, dout, ks, d)
            flat[t] = keep - eps
            dn = _loss(q, k, v, rpb, dout, ks, d)
            flat[t] = keep
            nflat[t] = (up - dn) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=0, atol=2e-7, err_msg=name)


def _dense_grads(q, k, v, rpb, dout, ks):
    """torch autograd of softmax(q k^T / sqrt(D) + bias) v on a k x k map,
    bias[i, n] = rpb[h, dy + k - 1, dx + k - 1] with (dy, dx) = key - query."""
    B, heads, H, W, D = q.shape
    assert H == W == ks
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, rpb)]
    tq, tk, tv, tr = t
    ys, xs = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    ys, xs = ys.reshape(-1), xs.reshape(-1)
    iy = torch.tensor(ys[None, :] - ys[:, None] + ks - 1)
    ix = torch.tensor(xs[None, :] - xs[:, None] + ks - 1)
    bias = tr[:, iy, ix]                                      # [heads, N, N]
    qq, kk, vv = (x.reshape(B, heads, H * W, D) for x in (tq, tk, tv))
    s = qq @ kk.transpose(-1, -2) / np.sqrt(D) + bias[None]
    out = torch.softmax(s, dim=-1) @ vv
    (out * torch.tensor(dout.reshape(B, heads, H * W, D))).sum().backward()
    return {"dq": tq.grad.numpy(), "dk": tk.grad.numpy(), "dv": tv.grad.numpy(),
            "drpb": tr.grad.numpy()}


@pytest.mark.parametrize("ks", [1, 3, 5, 7])
def test_full_window_equals_dense_attention_gradients(ks):
    q, k, v, rpb, dout = _problem(2, 3, ks, ks, 8, ks, seed=ks)
    g = oracle.backward(q, k, v, rpb, dout, ks, 1)
    ref = _dense_grads(q, k, v, rpb, dout, ks)
    for name in ("dq", "dk", "dv", "drpb"):
        np.testing.assert_allclose(g[name], ref[name], rtol=1e-10, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("ks,d", [(3, 2), (5, 3), (7, 2)])
def test_whole_class_maps_equal_dense_attention_per_class(ks, d):
    m = ks * d
    q, k, v, rpb, dout = _problem(1, 2, m, m, 4, ks, seed=ks * 10 + d)
    g = oracle.backward(q, k, v, rpb, dout, ks, d)
    drpb = np.zeros_like(rpb)
    for ry in range(d):
        for rx in range(d):
            sub = [x[:, :, ry::d, rx::d] for x in (q, k, v, dout)]
            ref = _dense_grads(sub[0], sub[1], sub[2], rpb, sub[3], ks)
            for name in ("dq", "dk", "dv"):
                np.testing.assert_allclose(g[name][:, :, ry::d, rx::d], ref[name], rtol=1e-10,
                                           atol=1e-11, err_msg=name)
            drpb += ref["drpb"]
    np.testing.assert_allclose(g["drpb"], drpb, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("H,W,ks,d", [(13, 11, 3, 2), (17, 23, 5, 3), (16, 16, 3, 4)])
def test_dilated_gradients_are_subgrid_gradients(H, W, ks, d):
    q, k, v, rpb, dout = _problem(1, 2, H, W, 4, ks, seed=H + W)
    g = oracle.backward(q, k, v, rpb, dout, ks, d)
    drpb = np.zeros_like(rpb)
    for ry in range(d):
        for rx in range(d):
            sub = [x[:, :, ry::d, rx::d] for x in (q, k, v, dout)]
            r = oracle.backward(sub[0], sub[1], sub[2], rpb, sub[3], ks, 1)
            for name in ("dq", "dk", "dv"):
                np.testing.assert_array_equal(g[name][:, :, ry::d, rx::d], r[name], err_msg=name)
            drpb += r["drpb"]
    np.testing.assert_allclose(g["drpb"], drpb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ks,d", [(3, 1), (7, 1), (5, 2)])
def test_bias_gradient_sums_to_zero_per_head(ks, d):
    q, k, v, rpb, dout = _problem(2, 3, 3 * ks * d, 2 * ks * d + 1, 8, ks, seed=3)
    g = oracle.backward(q, k, v, rpb, dout, ks, d)
    scale = np.abs(g["drpb"]).sum(axis=(1, 2))
    assert np.all(np.abs(g["drpb"].sum(axis=(1, 2))) <= 1e-12 * scale + 1e-12)


def test_kernel_size_one():
    q, k, v, rpb, dout = _problem(2, 2, 5, 6, 4, 1, seed=5)
    g = oracle.backward(q, k, v, rpb, dout, 1, 2)
    np.testing.assert_array_equal(g["dv"], dout)
    assert not g["dq"].any() and not g["dk"].any() and not g["drpb"].any()


def test_zero_bias_table_matches_none():
    q, k, v, rpb, dout = _problem(1, 2, 9, 10, 4, 3, seed=6)
    a = oracle.backward(q, k, v, None, dout, 3, 1)
    b = oracle.backward(q, k, v, np.zeros_like(rpb), dout, 3, 1)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])


def test_threads_do_not_change_the_result():
    q, k, v, rpb, dout = _problem(3, 2, 10, 9, 4, 3, seed=7)
    a = oracle.backward(q, k, v, rpb, dout, 3, 1, threads=1)
    b = oracle.backward(q, k, v, rpb, dout, 3, 1, threads=5)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(a[name], b[name])
    np.testing.assert_allclose(a["drpb"], b["drpb"], rtol=1e-13, atol=1e-14)


def test_rejects_invalid_problem():
    q, k, v, rpb, dout = _problem(1, 1, 5, 5, 2, 3, seed=8)
    with pytest.raises(ValueError):
        oracle.backward(q, k, v, rpb, dout, 3, 2)  # map smaller than k*d
