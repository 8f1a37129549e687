"""GPU parity of the padded forward (maps smaller than kernel*dilation,
padded below/right with per-head pad vectors, attended, cropped) against the
float64 oracle's ``forward_padded``, and bit-equality with the ordinary
forward run on explicitly padded tensors (same kernel, same values).

Whole-class maps after padding (both sides <= k*d, d a power of two,
k in {3, 5, 7}, bf16/fp16) run on the matrix cores; every other padded map
(one side padded, other dilations or kernel sizes, fp32) on the FMA kernel.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_transformer_local_amd import inputs as I
from vision_transformer_local_amd import na2d
from vision_transformer_local_amd.inputs import Problem

from parity_util import TOL, note

pytestmark = pytest.mark.gpu

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _pads(p: Problem, seed: int, given: bool):
    if not given:
        return None, None
    g = torch.Generator("cpu").manual_seed(seed + 500)
    return tuple(torch.randn(p.heads, p.D, generator=g).to(_TORCH[p.dtype]) for _ in range(2))


CASES = [
    Problem(2, 2, 48, 48, 32, 7, 8, "bf16"),   # DiNAT stage 1 of a 192x192 image
    Problem(2, 4, 20, 25, 32, 7, 4, "f16"),
    Problem(2, 2, 5, 3, 32, 3, 2, "bf16"),
    Problem(1, 2, 1, 1, 32, 5, 1, "bf16"),
    Problem(2, 3, 13, 9, 32, 7, 2, "bf16"),
    Problem(2, 2, 9, 40, 32, 5, 2, "bf16"),    # one side padded: FMA kernel
    Problem(1, 2, 10, 10, 32, 5, 3, "bf16"),   # d = 3: FMA kernel
    Problem(1, 2, 12, 12, 32, 9, 2, "f16"),    # k = 9: FMA kernel
    Problem(2, 2, 10, 7, 32, 7, 2, "f32"),
    Problem(1, 1, 2, 9, 32, 3, 3, "f32"),
]


@pytest.mark.parametrize("given", [True, False], ids=["pad_vectors", "zero_pad"])
@pytest.mark.parametrize("p", CASES, ids=lambda p: p.describe().replace(" ", "_"))
def test_padded_forward_matches_oracle(p, given):
    note("padded %s pads=%s" % (p.describe(), given))
    q, k, v, rpb = I.make_inputs(p, seed=3)
    pk, pv = _pads(p, 3, given)
    g = [t.to("cuda") for t in (q, k, v, rpb)]
    gp = [None if t is None else t.to("cuda") for t in (pk, pv)]
    out = na2d.forward_padded(*g, *gp, p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    ref = oracle.forward_padded(q, k, v, rpb, pk, pv, p.kernel_size, p.dilation)
    got = out.to("cpu").to(torch.float64).numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    assert err <= TOL[p.dtype], "max abs error %.3g for %s" % (err, p.describe())


def _same_kernel(p: Problem) -> bool:
    """Both routes run one kernel: fp32 (FMA) or a padded map that is k*d
    square with the whole-class matrix-core kernel's k and d."""
    span = p.kernel_size * p.dilation
    if p.dtype == "f32":
        return True
    return (p.H <= span and p.W <= span and p.kernel_size in (3, 5, 7)
            and p.dilation & (p.dilation - 1) == 0)


@pytest.mark.parametrize("p", [c for c in CASES if _same_kernel(c)],
                         ids=lambda p: p.describe().replace(" ", "_"))
def test_padded_forward_equals_forward_on_padded_tensors(p):
    note("padded vs explicit %s" % p.describe())
    q, k, v, rpb = (t.to("cuda") for t in I.make_inputs(p, seed=4))
    pk, pv = (t.to("cuda") for t in _pads(p, 4, True))
    span = p.kernel_size * p.dilation
    Hp, Wp = max(p.H, span), max(p.W, span)

    def pad(x, vec):
        y = vec[None, :, None, None, :].expand(p.B, p.heads, Hp, Wp, p.D).contiguous()
        y[:, :, :p.H, :p.W] = x
        return y

    qp = pad(q, torch.zeros_like(pk))
    full = na2d.forward(qp, pad(k, pk), pad(v, pv), rpb, p.kernel_size, p.dilation)
    out = na2d.forward_padded(q, k, v, rpb, pk, pv, p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    assert torch.equal(out, full[:, :, :p.H, :p.W])


def test_unpadded_maps_run_the_plain_forward():
    p = Problem(2, 2, 30, 33, 32, 7, 2, "bf16")
    note("padded no-op %s" % p.describe())
    q, k, v, rpb = (t.to("cuda") for t in I.make_inputs(p, seed=5))
    junk = torch.full((p.heads, p.D), 3.0, dtype=q.dtype, device="cuda")
    a = na2d.forward_padded(q, k, v, rpb, junk, junk, p.kernel_size, p.dilation)
    b = na2d.forward(q, k, v, rpb, p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
