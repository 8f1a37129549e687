"""Pins for the CPU oracle: checks against facts fixed by the source pages and
by mathematics, none of which re-types the oracle's own loops.

  * hand-written window/bias tables (tests/golden/windows_1d.txt);
  * self-attention equivalence at full size (NAT repository README,
    introduction), against torch's scaled_dot_product_attention in float64;
  * dilated NA equals NA on each strided sub-grid (DiNAT walk-through blog,
    "What is DiNAT": dilation only changes which pixels are sampled);
  * translational equivariance of interior pixels (NAT model doc, Overview);
  * brute force on tiny maps with a different formulation (dense masked
    attention, window chosen by minimising the distance to the query);
  * special cases: k = 1, constant values, zero queries and bias.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "windows_1d.txt")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _problem(B, heads, H, W, D, ks, seed=0, bias_scale=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, heads, H, W, D))
    k = rng.standard_normal((B, heads, H, W, D))
    v = rng.standard_normal((B, heads, H, W, D))
    rpb = bias_scale * rng.standard_normal((heads, 2 * ks - 1, 2 * ks - 1))
    return q, k, v, rpb


# --------------------------------------------------------------------------
# golden tables


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, rest = line.split(":")
            L, ks, d, i = (int(x) for x in head.split())
            pix, bias = rest.split("|")
            rows.append((L, ks, d, i, [int(x) for x in pix.split()], [int(x) for x in bias.split()]))
    return rows


GOLDEN_ROWS = _golden_rows()


def test_golden_file_is_not_empty():
    assert len(GOLDEN_ROWS) >= 30


@pytest.mark.parametrize("row", GOLDEN_ROWS, ids=lambda r: "L%d-k%d-d%d-i%d" % r[:4])
def test_golden_windows_and_bias_index(row):
    L, ks, d, i, pix, bias = row
    D = 2
    shape = (1, 1, L, L, D)
    zeros = np.zeros(shape)
    side = 2 * ks - 1
    # a bias table whose entries name their own (row, col) position
    rpb = (1000.0 * np.arange(side)[:, None] + np.arange(side)[None, :])[None]
    # query (i, i): rows and columns of the window follow the same rule
    idx = np.array([i * L + i])
    r = oracle.forward(zeros, zeros, zeros, rpb, ks, d, idx=idx, scores=True, neighbours=True)
    nb = r["neighbours"][0].reshape(ks, ks)
    assert [int(x) // L for x in nb[:, 0]] == pix  # window rows
    assert [int(x) % L for x in nb[0, :]] == pix  # window columns
    s = r["scores"][0].reshape(ks, ks)
    expect = 1000.0 * np.array(bias)[:, None] + np.array(bias)[None, :]
    np.testing.assert_array_equal(s, expect)


# --------------------------------------------------------------------------
# self-attention equivalence


def _sdpa_with_bias(qf, kf, vf, bias):
    """Dense attention by the library routine: qf,kf,vf [B,h,N,D], bias [h,N,N]."""
    D = qf.shape[-1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    o = torch.nn.functional.scaled_dot_product_attention(
        t(qf), t(kf), t(vf), attn_mask=t(bias)[None], scale=D ** -0.5)
    return o.numpy()


def _dense_bias(rpb, side_len, ks):
    """Bias matrix for a side_len x side_len map, indexed by key-minus-query offset."""
    heads = rpb.shape[0]
    N = side_len * side_len
    ys, xs = np.divmod(np.arange(N), side_len)
    dy = ys[None, :] - ys[:, None] + ks - 1  # key row - query row
    dx = xs[None, :] - xs[:, None] + ks - 1
    return rpb[:, dy, dx].reshape(heads, N, N)


@pytest.mark.parametrize("ks,D,B,heads", [(3, 4, 1, 1), (5, 8, 2, 2), (7, 32, 2, 3), (13, 32, 1, 2)])
def test_self_attention_equivalence_full_window(ks, D, B, heads):
    q, k, v, rpb = _problem(B, heads, ks, ks, D, ks, seed=ks)
    got = oracle.forward(q, k, v, rpb, ks, 1)["out"]
    N = ks * ks
    f = lambda a: a.reshape(B, heads, N, D)
    ref = _sdpa_with_bias(f(q), f(k), f(v), _dense_bias(rpb, ks, ks))
    np.testing.assert_allclose(got.reshape(B, heads, N, D), ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("ks,d", [(3, 2), (3, 3), (7, 4), (7, 8)])
def test_self_attention_equivalence_per_residue_class(ks, d):
    """H = W = k*d: every residue class is exactly k x k, so dilated NA there is
    dense self attention on each of the d*d sub-grids (the DiNAT 56x56, d=8 and
    28x28, d=4 layers are of this kind)."""
    B, heads, D = 1, 2, 16
    L = ks * d
    q, k, v, rpb = _problem(B, heads, L, L, D, ks, seed=d)
    got = oracle.forward(q, k, v, rpb, ks, d)["out"]
    bias = _dense_bias(rpb, ks, ks)
    for ry, rx in itertools.product(range(d), range(d)):
        sub = lambda a: a[:, :, ry::d, rx::d, :].reshape(B, heads, ks * ks, D)
        ref = _sdpa_with_bias(sub(q), sub(k), sub(v), bias)
        np.testing.assert_allclose(sub(got), ref, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# sub-grid equivalence (bit-exact)


@pytest.mark.parametrize("ks,d,H,W", [(3, 2, 6, 6), (3, 2, 9, 11), (3, 3, 11, 13),
                                      (5, 2, 13, 10), (7, 3, 23, 21), (7, 4, 28, 28)])
def test_dilated_equals_na_on_each_subgrid(ks, d, H, W):
    q, k, v, rpb = _problem(2, 2, H, W, 8, ks, seed=H * W)
    full = oracle.forward(q, k, v, rpb, ks, d, scores=True)
    for ry, rx in itertools.product(range(d), range(d)):
        sl = (slice(None), slice(None), slice(ry, None, d), slice(rx, None, d))
        sub = oracle.forward(q[sl], k[sl], v[sl], rpb, ks, 1, scores=True)
        np.testing.assert_array_equal(full["out"][sl], sub["out"])
        np.testing.assert_array_equal(full["scores"][sl], sub["scores"])


# --------------------------------------------------------------------------
# translational equivariance (bit-exact on interior pixels)


def _unclamped(c, L, ks):
    r = ks // 2
    return c - r >= 0 and c + r <= L - 1


@pytest.mark.parametrize("ks,d,dy,dx", [(3, 1, 1, 2), (5, 1, 3, 1), (7, 1, 2, 5), (3, 2, 1, 3), (5, 3, 4, 2)])
def test_translational_equivariance_interior(ks, d, dy, dx):
    H = W = ks * d + 9
    q, k, v, rpb = _problem(1, 2, H + dy, W + dx, 8, ks, seed=ks + d)
    crop_a = (slice(None), slice(None), slice(0, H), slice(0, W))
    crop_b = (slice(None), slice(None), slice(dy, dy + H), slice(dx, dx + W))
    oa = oracle.forward(q[crop_a], k[crop_a], v[crop_a], rpb, ks, d)["out"]
    ob = oracle.forward(q[crop_b], k[crop_b], v[crop_b], rpb, ks, d)["out"]
    checked = 0
    for i in range(H):
        for j in range(W):
            ia, ja = i + dy, j + dx  # the same pixel in crop A's coordinates
            if ia >= H or ja >= W:
                continue
            # the window must be unclamped in both crops (in sub-grid units)
            ok = (_unclamped(i // d, (H - i % d + d - 1) // d, ks)
                  and _unclamped(j // d, (W - j % d + d - 1) // d, ks)
                  and _unclamped(ia // d, (H - ia % d + d - 1) // d, ks)
                  and _unclamped(ja // d, (W - ja % d + d - 1) // d, ks))
            if not ok:
                continue
            np.testing.assert_array_equal(ob[:, :, i, j], oa[:, :, ia, ja])
            checked += 1
    assert checked > 0


# --------------------------------------------------------------------------
# brute force: dense masked attention with an independently chosen window


def _axis_windows(L, ks, d):
    """member[i, p]: pixel p lies in query i's window; bidx[i, p]: bias index."""
    r = ks // 2
    member = np.zeros((L, L), dtype=bool)
    bidx = np.zeros((L, L), dtype=np.int64)
    for i in range(L):
        cands = [p for p in range(L) if p % d == i % d]
        c = cands.index(i)
        # the k consecutive class members whose centre slot is nearest the query
        start = min(range(len(cands) - ks + 1), key=lambda s: abs(s + r - c))
        for a in range(ks):
            p = cands[start + a]
            member[i, p] = True
            bidx[i, p] = (p - i) // d + ks - 1
    return member, bidx


def _brute_force(q, k, v, rpb, ks, d):
    B, heads, H, W, D = q.shape
    my, by = _axis_windows(H, ks, d)
    mx, bx = _axis_windows(W, ks, d)
    N = H * W
    # dense [N, N] mask and bias-index tables over (query pixel, key pixel)
    mask = (my[:, None, :, None] & mx[None, :, None, :]).reshape(N, N)
    biy = np.broadcast_to(by[:, None, :, None], (H, W, H, W)).reshape(N, N)
    bix = np.broadcast_to(bx[None, :, None, :], (H, W, H, W)).reshape(N, N)
    out = np.empty_like(q)
    for b in range(B):
        for h in range(heads):
            Q = q[b, h].reshape(N, D)
            K = k[b, h].reshape(N, D)
            V = v[b, h].reshape(N, D)
            S = Q @ K.T / np.sqrt(D) + rpb[h][biy, bix]
            S = np.where(mask, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[b, h] = (P @ V).reshape(H, W, D)
    return out


BF_CASES = []
for ks, d in [(1, 1), (1, 3), (3, 1), (3, 2), (3, 3), (5, 1), (5, 2), (7, 1), (7, 2), (5, 3)]:
    for extra_h, extra_w in [(0, 0), (1, 4), (5, 2), (3, 5)]:
        BF_CASES.append((ks, d, ks * d + extra_h, ks * d + extra_w))


@pytest.mark.parametrize("ks,d,H,W", BF_CASES)
def test_brute_force_tiny_maps(ks, d, H, W):
    q, k, v, rpb = _problem(2, 2, H, W, 5, ks, seed=7 * H + W)
    got = oracle.forward(q, k, v, rpb, ks, d)["out"]
    ref = _brute_force(q, k, v, rpb, ks, d)
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


def test_brute_force_catches_transposed_bias():
    """The brute-force pin is sensitive to the bias orientation: a transposed
    table gives a visibly different answer, so a transposition in the oracle
    could not hide."""
    q, k, v, rpb = _problem(1, 1, 9, 9, 4, 5, seed=3, bias_scale=2.0)
    ref = _brute_force(q, k, v, rpb, 5, 1)
    wrong = _brute_force(q, k, v, np.ascontiguousarray(rpb.transpose(0, 2, 1)), 5, 1)
    assert np.abs(ref - wrong).max() > 1e-3
    got = oracle.forward(q, k, v, rpb, 5, 1)["out"]
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# special cases


@pytest.mark.parametrize("d,H,W", [(1, 4, 5), (2, 5, 7), (3, 6, 3)])
def test_kernel_size_one_returns_value(d, H, W):
    q, k, v, rpb = _problem(2, 3, H, W, 6, 1, seed=11)
    got = oracle.forward(q, k, v, rpb, 1, d)["out"]
    np.testing.assert_array_equal(got, v)


@pytest.mark.parametrize("ks,d", [(3, 1), (7, 1), (5, 2), (7, 3)])
def test_constant_value_and_probabilities_sum_to_one(ks, d):
    H, W = ks * d + 3, ks * d + 1
    q, k, v, rpb = _problem(1, 2, H, W, 4, ks, seed=5)
    const = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0]), v.shape).copy()
    r = oracle.forward(q, k, const, rpb, ks, d, probs=True)
    np.testing.assert_allclose(r["out"], const, atol=1e-13, rtol=0)
    np.testing.assert_allclose(r["probs"].sum(-1), 1.0, atol=1e-14, rtol=0)
    assert (r["probs"] > 0).all()


@pytest.mark.parametrize("row", [r for r in GOLDEN_ROWS if r[0] <= 12], ids=lambda r: "L%d-k%d-d%d-i%d" % r[:4])
def test_zero_query_and_bias_give_window_mean(row):
    """q = 0 and rpb = 0 make every score equal, so the output is the plain
    mean of the values inside the window -- the window comes from the
    hand-written table."""
    L, ks, d, i, pix, _ = row
    D = 3
    v = _rand((1, 1, L, L, D), seed=L + i)
    zeros = np.zeros_like(v)
    r = oracle.forward(zeros, zeros, v, None, ks, d, idx=np.array([i * L + i]))
    expect = v[0, 0][np.ix_(pix, pix)].reshape(-1, D).mean(axis=0)
    np.testing.assert_allclose(r["out"][0], expect, atol=1e-14, rtol=0)


def test_attention_is_linear_in_map_size():
    """Scores hold B*heads*H*W*k*k entries: linear in the number of pixels."""
    ks = 5
    for H, W in [(5, 5), (10, 7), (20, 9)]:
        q, k, v, rpb = _problem(2, 3, H, W, 2, ks, seed=1)
        s = oracle.forward(q, k, v, rpb, ks, 1, scores=True)["scores"]
        assert s.size == 2 * 3 * H * W * ks * ks


def test_argmax_is_the_first_maximum():
    q, k, v, rpb = _problem(2, 2, 9, 10, 8, 3, seed=2)
    r = oracle.forward(q, k, v, rpb, 3, 1, scores=True, argmax=True)
    np.testing.assert_array_equal(r["argmax"], np.argmax(r["scores"], axis=-1))
    # exact ties resolve to the lowest slot
    z = np.zeros_like(q)
    r = oracle.forward(z, z, v, None, 3, 1, argmax=True)
    assert (r["argmax"] == 0).all()


def test_sampled_queries_match_full_run():
    q, k, v, rpb = _problem(2, 2, 12, 11, 8, 5, seed=4)
    full = oracle.forward(q, k, v, rpb, 5, 2)["out"].reshape(-1, 8)
    idx = np.array([0, 5, 17, 100, 2 * 2 * 12 * 11 - 1])
    part = oracle.forward(q, k, v, rpb, 5, 2, idx=idx)["out"]
    np.testing.assert_array_equal(part, full[idx])


@pytest.mark.parametrize("H,W,ks,d", [(6, 7, 7, 1), (7, 6, 7, 1), (13, 20, 7, 2), (8, 8, 4, 1), (8, 8, 3, 0)])
def test_oracle_rejects_invalid_problems(H, W, ks, d):
    assert not oracle.valid(H, W, ks, d)
    z = np.zeros((1, 1, H, W, 2))
    with pytest.raises(ValueError):
        oracle.forward(z, z, z, None, ks, d)
