"""The allocation-free backward entry point (na2d_backward_noalloc) against
na2d_backward, through the C ABI.

Both run the same kernels; the no-alloc call takes its workspace from the
library's fixed device array instead of a caller's buffer.  Every gradient sum
runs in a fixed order, so the two must agree bit for bit.  Two calls in a row
share the array: the second, smaller problem must not be disturbed by what
the first left in it.
"""
import pytest
import torch

from vision_transformer_local_amd import inputs as I
from vision_transformer_local_amd import na2d

from parity_util import note

pytestmark = pytest.mark.gpu

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _case(p, seed, bias_grad=True):
    q, k, v, rpb = I.make_inputs(p, seed)
    gen = torch.Generator("cpu").manual_seed(seed + 1000)
    dout = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(_TORCH[p.dtype])
    return [t.cuda() for t in (q, k, v, rpb, dout)]


def _outputs(q, heads, ks, bias_grad):
    side = 2 * ks - 1
    drpb = (torch.full((heads, side, side), float("nan"), dtype=torch.float32, device=q.device)
            if bias_grad else None)
    return [torch.full_like(q, float("nan")) for _ in range(3)] + [drpb]


def _compare(p, seed, bias_grad=True):
    note("no-alloc backward %s seed %d bias_grad %s" % (p.describe(), seed, bias_grad))
    q, k, v, rpb, dout = _case(p, seed, bias_grad)
    heads, ks, d = p.heads, p.kernel_size, p.dilation
    ref = na2d.backward(q, k, v, rpb, dout, ks, d, bias_grad=bias_grad)
    got = _outputs(q, heads, ks, bias_grad)
    na2d.na2d_backward_noalloc(q, k, v, rpb, dout, *got, ks, d)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "drpb"), got, ref):
        if b is None:
            assert a is None
            continue
        assert torch.equal(a, b), "%s differs from na2d_backward for %s" % (name, p.describe())


def test_noalloc_matches_backward_two_calls_shrinking():
    """A NAT-Tiny-shaped layer (16 images), then a smaller dilated f16 map
    with ragged residue classes: each bit-equal to na2d_backward."""
    big = I.Problem(16, 2, 56, 56, 32, 7, 1, "bf16")
    small = I.Problem(1, 3, 23, 19, 32, 5, 2, "f16")
    _compare(big, seed=3)
    _compare(small, seed=4)


def test_noalloc_per_lane_kernels_and_no_bias_grad():
    """fp32 (the per-lane kernels) without the bias gradient, then a bf16
    k = 13 problem with it."""
    _compare(I.Problem(2, 2, 15, 17, 32, 3, 1, "f32"), seed=5, bias_grad=False)
    _compare(I.Problem(1, 2, 30, 28, 32, 13, 2, "bf16"), seed=6)
