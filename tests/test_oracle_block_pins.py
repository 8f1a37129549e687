"""Pins for the oracle's attention block (projections -> NA -> output
projection), each an independent route:
  * window = whole map (k = H = W, d = 1): torch float64 linear layers and
    scaled_dot_product_attention with the bias as an additive mask;
  * identity projections without bias: the block is the operator itself on
    q = k = v = x split into heads;
  * maps below k*d: padding the features with zeros, running the block on the
    padded map, and cropping (the layer's maybe_pad) gives the same result.
"""
import numpy as np
import pytest
import torch

import oracle


def _weights(C, heads, ks, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    w_qkv = torch.randn(3 * C, C, generator=g, dtype=torch.float64) / np.sqrt(C)
    b_qkv = torch.randn(3 * C, generator=g, dtype=torch.float64) if bias else None
    w_out = torch.randn(C, C, generator=g, dtype=torch.float64) / np.sqrt(C)
    b_out = torch.randn(C, generator=g, dtype=torch.float64) if bias else None
    rpb = 0.3 * torch.randn(heads, 2 * ks - 1, 2 * ks - 1, generator=g, dtype=torch.float64)
    return w_qkv, b_qkv, w_out, b_out, rpb


def _np(t):
    return None if t is None else t.numpy()


@pytest.mark.parametrize("ks,heads,D", [(3, 2, 4), (5, 1, 8), (7, 3, 2)])
def test_full_window_block_is_dense_attention(ks, heads, D):
    B, C = 2, heads * D
    g = torch.Generator().manual_seed(ks)
    x = torch.randn(B, ks, ks, C, generator=g, dtype=torch.float64)
    w_qkv, b_qkv, w_out, b_out, rpb = _weights(C, heads, ks, ks + 1)
    got = oracle.block_forward(x.numpy(), _np(w_qkv), _np(b_qkv), rpb.numpy(), _np(w_out),
                               _np(b_out), heads, ks, 1)
    qkv = torch.nn.functional.linear(x, w_qkv, b_qkv).reshape(B, ks * ks, 3, heads, D)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))     # [B, heads, N, D]
    ys, xs = np.meshgrid(np.arange(ks), np.arange(ks), indexing="ij")
    ys, xs = ys.reshape(-1), xs.reshape(-1)
    mask = rpb[:, torch.tensor(ys[None, :] - ys[:, None] + ks - 1),
               torch.tensor(xs[None, :] - xs[:, None] + ks - 1)]     # [heads, N, N]
    ctx = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None])
    ref = torch.nn.functional.linear(ctx.transpose(1, 2).reshape(B, ks, ks, C), w_out, b_out)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-11)


def test_identity_projections_give_the_operator():
    B, H, W, heads, D, ks, d = 2, 9, 11, 2, 4, 3, 2
    C = heads * D
    x = np.random.default_rng(3).standard_normal((B, H, W, C))
    rpb = 0.2 * np.random.default_rng(4).standard_normal((heads, 5, 5))
    eye = np.eye(C)
    got = oracle.block_forward(x, np.concatenate([eye, eye, eye]), None, rpb, eye, None, heads,
                               ks, d)
    xh = np.ascontiguousarray(x.reshape(B, H, W, heads, D).transpose(0, 3, 1, 2, 4))
    ref = oracle.forward(xh, xh, xh, rpb, ks, d)["out"].transpose(0, 2, 3, 1, 4).reshape(x.shape)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("H,W", [(4, 5), (2, 9), (1, 1)])
def test_small_maps_are_padded_features(H, W):
    B, heads, D, ks, d = 2, 2, 3, 3, 3
    C = heads * D
    x = np.random.default_rng(H * 10 + W).standard_normal((B, H, W, C))
    w_qkv, b_qkv, w_out, b_out, rpb = (_np(t) for t in _weights(C, heads, ks, 5))
    got = oracle.block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, heads, ks, d)
    Hp, Wp = max(H, ks * d), max(W, ks * d)
    xp = np.zeros((B, Hp, Wp, C))
    xp[:, :H, :W] = x
    ref = oracle.block_forward(xp, w_qkv, b_qkv, rpb, w_out, b_out, heads, ks, d)[:, :H, :W]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_rejects_bad_shapes():
    x = np.zeros((1, 4, 4, 6))
    w_qkv, b_qkv, w_out, b_out, rpb = (_np(t) for t in _weights(6, 2, 3, 6))
    with pytest.raises(ValueError):
        oracle.block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, 4, 3, 1)   # 6 % 4
    with pytest.raises(ValueError):
        oracle.block_forward(x, w_qkv[:6], b_qkv, rpb, w_out, b_out, 2, 3, 1)
