"""GPU parity of the projections (na2d_linear) against float64 matrix
products, and of the attention block (projection -> NA -> projection)
against the oracle's block_forward.

The block stores its q|k|v projection and its attention output in the data
type (as a bf16 / fp16 network stores its tensors), so the oracle is run
with those two intermediates rounded to the data type as well; the
remaining differences are the GEMMs' fp32 accumulation order, the attention
step's 16-bit probabilities and the final rounding, which the forward
tolerance (2e-2 absolute at these magnitudes) plus one rounding of y covers.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_transformer_local_amd import inputs as I
from vision_transformer_local_amd import na2d
from vision_transformer_local_amd.inputs import BlockProblem

from parity_util import note

pytestmark = pytest.mark.gpu

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -23}


@pytest.mark.parametrize("M,N,K,dtype", [(1000, 192, 64, "bf16"), (777, 80, 96, "bf16"),
                                         (300, 256, 512, "f16"), (129, 1536, 512, "bf16"),
                                         (5, 64, 64, "f16"), (100, 48, 32, "f32"),
                                         (4000, 128, 128, "bf16")])
@pytest.mark.parametrize("bias", [True, False])
def test_linear_matches_float64(M, N, K, dtype, bias):
    note("linear M%d N%d K%d %s bias=%s" % (M, N, K, dtype, bias))
    g = torch.Generator().manual_seed(M + N + K)
    dt = _TORCH[dtype]
    x = torch.randn(M, K, generator=g).to(dt)
    w = (torch.randn(N, K, generator=g) / K ** 0.5).to(dt)
    b = torch.randn(N, generator=g).to(dt) if bias else None
    y = na2d.linear(x.cuda(), w.cuda(), None if b is None else b.cuda())
    torch.cuda.synchronize()
    ref = x.double().numpy() @ w.double().numpy().T
    if b is not None:
        ref = ref + b.double().numpy()
    got = y.cpu().double().numpy()
    # one rounding of y, plus fp32 accumulation of K products
    bound = _ULP[dtype] * np.abs(ref) + 1e-6 * K * (np.abs(x.double().numpy()) @
                                                    np.abs(w.double().numpy()).T).max()
    assert np.all(np.abs(got - ref) <= bound + 1e-30)


def _stored(dtype):
    dt = _TORCH[dtype]
    return lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).double().numpy()


BLOCKS = [
    BlockProblem(2, 20, 23, 64, 2, 7, 1, "bf16"),
    BlockProblem(2, 16, 16, 128, 4, 5, 2, "f16"),
    BlockProblem(1, 9, 9, 64, 2, 7, 2, "bf16"),      # padded to 14x14 (whole-class kernel)
    BlockProblem(2, 12, 30, 64, 2, 3, 4, "bf16"),
    BlockProblem(1, 5, 11, 64, 2, 3, 3, "bf16"),     # padded on one side (FMA kernel)
    BlockProblem(1, 7, 7, 512, 16, 7, 1, "bf16"),    # the sweep's 7x7 stage
    BlockProblem(1, 10, 9, 64, 2, 3, 2, "f32"),
]


@pytest.mark.parametrize("p", BLOCKS, ids=lambda p: p.describe().replace(" ", "_"))
def test_block_matches_oracle(p):
    note("block %s" % p.describe())
    x, w_qkv, b_qkv, rpb, w_out, b_out = I.make_block_inputs(p, seed=1)
    y = na2d.block_forward(*(t.cuda() for t in (x, w_qkv, b_qkv, rpb, w_out, b_out)), p.heads,
                           p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    ref = oracle.block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, p.heads, p.kernel_size,
                               p.dilation, stored=_stored(p.dtype))
    got = y.cpu().double().numpy()
    assert np.isfinite(got).all()
    tol = 1e-5 if p.dtype == "f32" else 2e-2
    err = np.abs(got - ref) - _ULP[p.dtype] * np.abs(ref)
    assert err.max() <= tol, "excess error %.3g for %s" % (err.max(), p.describe())


def test_block_without_biases_and_bias_table():
    p = BlockProblem(2, 14, 15, 64, 2, 7, 1, "bf16")
    note("block no biases %s" % p.describe())
    x, w_qkv, _, _, w_out, _ = I.make_block_inputs(p, seed=2)
    y = na2d.block_forward(x.cuda(), w_qkv.cuda(), None, None, w_out.cuda(), None, p.heads,
                           p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    ref = oracle.block_forward(x, w_qkv, None, None, w_out, None, p.heads, p.kernel_size,
                               p.dilation, stored=_stored(p.dtype))
    err = np.abs(y.cpu().double().numpy() - ref) - _ULP[p.dtype] * np.abs(ref)
    assert err.max() <= 2e-2


def test_block_full_size_sweep_stage():
    p = I.BLOCK_SWEEP[0]  # B128 56x56 C64 h2 k7
    note("block full size %s" % p.describe())
    x, w_qkv, b_qkv, rpb, w_out, b_out = I.make_block_inputs(p, seed=0)
    y = na2d.block_forward(*(t.cuda() for t in (x, w_qkv, b_qkv, rpb, w_out, b_out)), p.heads,
                           p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    ref = oracle.block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, p.heads, p.kernel_size,
                               p.dilation, stored=_stored(p.dtype))
    err = np.abs(y.cpu().double().numpy() - ref) - _ULP[p.dtype] * np.abs(ref)
    assert err.max() <= 2e-2, "excess error %.3g" % err.max()


def test_linear_beyond_two_gib_of_rows():
    # x spans more than 2^31 bytes: the launcher runs the rows in slices; rows
    # around the slice boundary, the first and the last rows, and a random
    # sample are checked against float64 products
    K, N = 32, 16
    slice_rows = (2 ** 31 // (2 * K)) // 128 * 128
    M = slice_rows + 1000
    note("linear M%d N%d K%d bf16 (two row slices)" % (M, N, K))
    gen = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=gen) / K ** 0.5).to(torch.bfloat16)
    b = torch.randn(N, device="cuda", generator=gen).to(torch.bfloat16)
    y = na2d.linear(x, w, b)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(slice_rows - 130, slice_rows + 130),
                                     np.arange(M - 64, M), rng.integers(0, M, 2048)]))
    idx = torch.from_numpy(rows).cuda()
    xs = x[idx].double().cpu().numpy()
    ref = xs @ w.double().cpu().numpy().T + b.double().cpu().numpy()
    got = y[idx].double().cpu().numpy()
    bound = _ULP["bf16"] * np.abs(ref) + 1e-6 * K * (np.abs(xs) @ np.abs(w.double().cpu().numpy()).T).max()
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    del x, y
    torch.cuda.empty_cache()
