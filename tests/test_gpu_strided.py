"""GPU parity of the strided forward (channels-last hidden states, a fused
QKV buffer, a padded output) against the float64 oracle, and bit-equality
with the dense-layout forward where both run the same kernel.

The inputs are the seeded [B, heads, H, W, D] tensors of every other parity
test, re-laid out on the host as the encoder keeps hidden states
([B, H, W, heads*D]); the oracle reads the dense originals.
"""
import pytest
import torch

from vision_transformer_local_amd import inputs as I
from vision_transformer_local_amd import na2d
from vision_transformer_local_amd.inputs import Problem

from parity_util import compare, note, sample_indices

pytestmark = pytest.mark.gpu


def _channels_last(x):
    """[B, heads, H, W, D] -> [B, H, W, heads*D] (contiguous copy)."""
    B, h, H, W, D = x.shape
    return x.permute(0, 2, 3, 1, 4).reshape(B, H, W, h * D).contiguous()


def _run(p: Problem, layout: str, seed=0):
    cpu = I.make_inputs(p, seed)
    q, k, v, rpb = cpu
    heads = p.heads
    grpb = rpb.to("cuda")
    if layout == "channels_last":
        gq, gk, gv = (_channels_last(t).to("cuda") for t in (q, k, v))
        out = na2d.forward_channels_last(gq, gk, gv, grpb, heads, p.kernel_size, p.dilation)
        got = na2d.heads_view(out, heads)
    elif layout == "fused_qkv":
        qkv = torch.cat([_channels_last(t) for t in (q, k, v)], dim=-1).to("cuda")
        c = heads * p.D
        out = na2d.forward_channels_last(qkv[..., :c], qkv[..., c:2 * c], qkv[..., 2 * c:],
                                         grpb, heads, p.kernel_size, p.dilation)
        got = na2d.heads_view(out, heads)
    elif layout == "padded_out":
        gq, gk, gv = (na2d.heads_view(_channels_last(t).to("cuda"), heads) for t in (q, k, v))
        wide = torch.full((p.B, p.H, p.W, heads * p.D + 32), 7.0, dtype=gq.dtype, device="cuda")
        got = na2d.heads_view(wide[..., 16:16 + heads * p.D], heads)
        na2d.na2d_forward_strided(gq, gk, gv, grpb, got, p.kernel_size, p.dilation)
        torch.cuda.synchronize()
        # the channels around the output slice are untouched
        assert (wide[..., :16] == 7.0).all() and (wide[..., 16 + heads * p.D:] == 7.0).all()
    else:
        raise ValueError(layout)
    torch.cuda.synchronize()
    return cpu, got


CASES = [
    Problem(2, 2, 20, 23, 32, 7, 1, "bf16"),
    Problem(2, 3, 31, 17, 32, 5, 2, "f16"),
    Problem(1, 4, 40, 40, 32, 7, 4, "bf16"),
    Problem(2, 2, 56, 56, 32, 7, 8, "bf16"),    # whole-class map
    Problem(2, 2, 30, 29, 32, 13, 2, "bf16"),
    Problem(1, 2, 27, 25, 32, 9, 1, "f16"),
    Problem(2, 2, 21, 19, 32, 3, 1, "f32"),     # FMA kernel
    Problem(1, 3, 16, 18, 32, 5, 3, "f32"),
]


@pytest.mark.parametrize("layout", ["channels_last", "fused_qkv", "padded_out"])
@pytest.mark.parametrize("p", CASES, ids=lambda p: p.describe().replace(" ", "_"))
def test_strided_forward_matches_oracle(p, layout):
    note("strided %s %s" % (layout, p.describe()))
    cpu, got = _run(p, layout)
    compare(p, got.contiguous(), cpu)


@pytest.mark.parametrize("p", CASES, ids=lambda p: p.describe().replace(" ", "_"))
def test_strided_forward_equals_dense_layout_bitwise(p):
    """Same kernel (the strides only change addresses), same arithmetic."""
    note("strided vs dense %s" % p.describe())
    cpu, got = _run(p, "fused_qkv")
    g = tuple(t.to("cuda") for t in cpu)
    dense = na2d.forward(*g, p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    assert torch.equal(dense, got.contiguous())


@pytest.mark.parametrize("p", [I.NAT_TINY_S1, I.DINAT_S1_D8],
                         ids=lambda p: p.describe().replace(" ", "_"))
def test_strided_forward_full_size(p):
    note("strided full size %s" % p.describe())
    cpu, got = _run(p, "channels_last")
    compare(p, got.contiguous(), cpu, idx=sample_indices(p, 60000))
    g = tuple(t.to("cuda") for t in cpu)
    dense = na2d.forward(*g, p.kernel_size, p.dilation)
    torch.cuda.synchronize()
    assert torch.equal(dense, got.contiguous())
