"""Pins for the oracle's padded forward (maps smaller than k*d, padded below
and to the right, attended, cropped back; DiNAT walk-through blog, layer
organisation).  Each pin is a closed form or an independent route, not the
oracle's own construction:
  * maps that need no padding: the plain forward, pads ignored;
  * one pixel, k = 3: the softmax over 1 real and 8 padded keys written out;
  * q = 0, zero bias: every window is a whole padded residue class, so out is
    the class mean of v with padded pixels counting pad_v (d = 1 and d = 4);
  * pad vectors = projection biases equals padding the features with zeros
    and projecting them (torch float64), i.e. the layer's maybe_pad.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_no_padding_needed_equals_forward():
    q, k, v = (_rand((2, 2, 9, 8, 4), s) for s in (1, 2, 3))
    rpb = 0.3 * _rand((2, 5, 5), 4)
    pk, pv = _rand((2, 4), 5), _rand((2, 4), 6)
    a = oracle.forward_padded(q, k, v, rpb, pk, pv, 3, 2)  # 9, 8 >= 3*2
    b = oracle.forward(q, k, v, rpb, 3, 2)["out"]
    np.testing.assert_array_equal(a, b)


def test_single_pixel_closed_form():
    D, heads = 4, 2
    q, k, v = (_rand((1, heads, 1, 1, D), s) for s in (7, 8, 9))
    rpb = 0.5 * _rand((heads, 5, 5), 10)
    pk, pv = _rand((heads, D), 11), _rand((heads, D), 12)
    got = oracle.forward_padded(q, k, v, rpb, pk, pv, 3, 1)
    for h in range(heads):
        qq = q[0, h, 0, 0]
        # window = the padded 3x3 map; key (a, c) - query (0, 0) = (a, c)
        logits, vals = [], []
        for a in range(3):
            for c in range(3):
                key, val = (k[0, h, 0, 0], v[0, h, 0, 0]) if (a, c) == (0, 0) else (pk[h], pv[h])
                logits.append(qq @ key / np.sqrt(D) + rpb[h, a + 2, c + 2])
                vals.append(val)
        w = np.exp(np.array(logits) - max(logits))
        ref = (w[:, None] * np.array(vals)).sum(0) / w.sum()
        np.testing.assert_allclose(got[0, h, 0, 0], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("H,W,ks,d", [(2, 3, 5, 1), (6, 6, 3, 4), (5, 2, 3, 3), (7, 3, 7, 1)])
def test_uniform_weights_give_padded_class_means(H, W, ks, d):
    B, heads, D = 1, 2, 3
    q = np.zeros((B, heads, H, W, D))
    k, v = _rand((B, heads, H, W, D), 13), _rand((B, heads, H, W, D), 14)
    pk, pv = _rand((heads, D), 15), _rand((heads, D), 16)
    got = oracle.forward_padded(q, k, v, None, pk, pv, ks, d)
    # H, W < k*d: the padded map is (k*d)^2 and each class exactly k x k, so
    # every window is its whole class
    assert H <= ks * d and W <= ks * d
    for i in range(H):
        for j in range(W):
            for h in range(heads):
                tot, n = np.zeros(D), 0
                for a in range(ks):
                    for c in range(ks):
                        r, s = i % d + a * d, j % d + c * d
                        tot += v[0, h, r, s] if (r < H and s < W) else pv[h]
                        n += 1
                np.testing.assert_allclose(got[0, h, i, j], tot / n, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("H,W", [(5, 4), (9, 4), (4, 11), (1, 1)])
def test_pad_vectors_are_the_projection_of_zero_features(H, W):
    B, C, heads, D, ks, d = 2, 6, 2, 3, 3, 2
    g = torch.Generator().manual_seed(17)
    x = torch.randn(B, H, W, C, generator=g, dtype=torch.float64)
    lin = torch.nn.Linear(C, 3 * heads * D, dtype=torch.float64)
    torch.nn.init.normal_(lin.weight, generator=g)
    torch.nn.init.normal_(lin.bias, generator=g)
    rpb = 0.2 * torch.randn(heads, 2 * ks - 1, 2 * ks - 1, generator=g, dtype=torch.float64)

    def split(t):  # [B, H', W', 3*heads*D] -> three [B, heads, H', W', D]
        t = t.unflatten(3, (3, heads, D)).permute(3, 0, 4, 1, 2, 5)
        return [u.detach().numpy() for u in t]

    # the layer: pad the features with zeros, project, attend, crop
    Hp, Wp = max(H, ks * d), max(W, ks * d)
    xp = torch.nn.functional.pad(x, (0, 0, 0, Wp - W, 0, Hp - H))
    qp, kp, vp = split(lin(xp))
    ref = oracle.forward(qp, kp, vp, rpb.numpy(), ks, d)["out"][:, :, :H, :W]
    # the operator: project the unpadded features, pad with the biases
    q, k, v = split(lin(x))
    bias = lin.bias.detach().numpy().reshape(3, heads, D)
    got = oracle.forward_padded(q, k, v, rpb.numpy(), bias[1], bias[2], ks, d)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_rejects_bad_pad_shape():
    q = _rand((1, 2, 3, 3, 4), 18)
    with pytest.raises(ValueError):
        oracle.forward_padded(q, q, q, None, np.zeros((2, 3)), None, 3, 2)
