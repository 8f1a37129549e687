"""GPU parity of the fused attention block (one kernel: q/k/v projection,
per-head NA, output projection) against the oracle's block_forward, with
the intermediates rounded to the data type as the kernel keeps them (q, k,
v after the projection, the heads' outputs before the output projection).

Cases span the fused kernel's block grid (16- and 14-row blocks, ragged
last block rows and columns, a map of exactly k x k), k = 3, 5, 7, both
16-bit types, and the optional biases and bias table.  The fused and the
three-launch path must agree within the same bound (they round the same
intermediates; the fused kernel's score products take the channels in
another order, so they are not bit-identical).
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

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}
_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
TOL = 2e-2  # the block tolerance of the three-launch path (see test_gpu_block)


def _stored(dtype):
    dt = _TORCH[dtype]
    return lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).double().numpy()


def _excess(got, ref, dtype):
    return float((np.abs(got - ref) - _ULP[dtype] * np.abs(ref)).max())


FUSED = [
    BlockProblem(2, 20, 23, 64, 2, 7, 1, "bf16"),   # 16-row blocks, ragged rows and columns
    BlockProblem(1, 28, 17, 64, 2, 5, 1, "f16"),    # 14-row blocks
    BlockProblem(3, 7, 7, 64, 2, 7, 1, "bf16"),     # map of exactly k x k
    BlockProblem(2, 33, 9, 64, 2, 3, 1, "bf16"),
    BlockProblem(1, 56, 56, 64, 2, 7, 1, "bf16"),   # one image of the sweep's 56x56 stage
    BlockProblem(2, 16, 40, 64, 2, 7, 1, "f16"),
]


@pytest.mark.parametrize("p", FUSED, ids=lambda p: p.describe().replace(" ", "_"))
@pytest.mark.parametrize("biases", [True, False])
def test_fused_block_matches_oracle(p, biases):
    note("fused block %s biases=%s" % (p.describe(), biases))
    x, w_qkv, b_qkv, rpb, w_out, b_out = I.make_block_inputs(p, seed=3)
    if not biases:
        b_qkv = rpb = b_out = None
    dev = [None if t is None else t.cuda() for t in (x, w_qkv, b_qkv, rpb, w_out, b_out)]
    y = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="fused")
    yu = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="unfused")
    torch.cuda.synchronize()
    ref = oracle.block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, p.heads, p.kernel_size,
                               p.dilation, stored=_stored(p.dtype))
    got = y.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = _excess(got, ref, p.dtype)
    assert err <= TOL, "excess error %.3g for %s" % (err, p.describe())
    # the two plans agree as closely as each agrees with the oracle
    gu = yu.cpu().double().numpy()
    assert np.abs(got - gu).max() <= 2 * TOL + _ULP[p.dtype] * np.abs(gu).max()


def test_fused_is_the_automatic_choice_and_deterministic():
    p = BlockProblem(2, 20, 23, 64, 2, 7, 1, "bf16")
    note("fused block auto == fused %s" % p.describe())
    dev = [t.cuda() for t in I.make_block_inputs(p, seed=4)]
    ya = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation)
    yf = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="fused")
    yf2 = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="fused")
    torch.cuda.synchronize()
    assert torch.equal(ya, yf) and torch.equal(yf, yf2)


@pytest.mark.parametrize("p", [BlockProblem(1, 9, 9, 64, 2, 7, 2, "bf16"),     # dilation
                               BlockProblem(1, 5, 11, 64, 2, 7, 1, "bf16"),    # padded map
                               BlockProblem(1, 16, 16, 128, 4, 7, 1, "bf16"),  # C = 128
                               BlockProblem(1, 10, 9, 64, 2, 3, 1, "f32"),     # fp32
                               BlockProblem(1, 16, 16, 64, 2, 9, 1, "bf16")],  # k = 9
                         ids=lambda p: p.describe().replace(" ", "_"))
def test_fused_rejects_what_it_does_not_cover(p):
    note("fused block unsupported %s" % p.describe())
    dev = [t.cuda() for t in I.make_block_inputs(p, seed=5)]
    with pytest.raises(na2d.Na2dError) as e:
        na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="fused")
    assert e.value.status == na2d.NOT_SUPPORTED


def test_fused_full_size_sweep_stage_both_plans():
    p = I.BLOCK_SWEEP[0]  # B128 56x56 C64 h2 k7
    note("fused block full size %s" % p.describe())
    cpu = I.make_block_inputs(p, seed=0)
    dev = [t.cuda() for t in cpu]
    y = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="fused")
    yu = na2d.block_forward(*dev, p.heads, p.kernel_size, p.dilation, path="unfused")
    torch.cuda.synchronize()
    # every pixel of 3 images (first, a middle one, last) against the oracle
    imgs = [0, 61, p.B - 1]
    x, w_qkv, b_qkv, rpb, w_out, b_out = cpu
    ref = oracle.block_forward(x[imgs], w_qkv, b_qkv, rpb, w_out, b_out, p.heads, p.kernel_size,
                               p.dilation, stored=_stored(p.dtype))
    got = y[imgs].cpu().double().numpy()
    assert _excess(got, ref, p.dtype) <= TOL
    gu = yu.cpu().double().numpy()
    ga = y.cpu().double().numpy()
    assert np.isfinite(ga).all()
    assert np.abs(ga - gu).max() <= 2 * TOL + _ULP[p.dtype] * np.abs(gu).max()
