"""GPU parity on a (batch, head) plane beyond the matrix-core forward
kernels' 32-bit in-plane byte offsets (8192 x 4100 pixels, 2.1 GB per
tensor in bf16): the automatic forward and na2d_forward_lse take the
per-lane kernel, the unfused scores step its per-lane kernel, and an
explicit matrix-core request returns NOT_SUPPORTED.

The inputs are drawn on the device.
The oracle runs on 64 x 64 crops at the top-left and bottom-right corners:
there the map borders are the crop's, and queries at least 16 pixels inside
the crop's other two edges have windows that the crop holds whole, so the
crop's results equal the full map's for them.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_transformer_local_amd import na2d

from parity_util import TOL, note

pytestmark = pytest.mark.gpu

H, W = 8192, 4100
CROP, INNER = 64, 16


def _inputs(ks, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v = (torch.randn((1, 1, H, W, 32), generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    side = 2 * ks - 1
    rpb = (0.02 * torch.randn((1, side, side), generator=g, device="cuda")).to(torch.bfloat16)
    return q, k, v, rpb


def _crops():
    # (rows, columns) of the crop, and the crop-local slice whose queries are
    # compared
    tl = (slice(0, CROP), slice(0, CROP)), slice(0, CROP - INNER)
    br = (slice(H - CROP, H), slice(W - CROP, W)), slice(INNER, CROP)
    return [tl, br]


@pytest.mark.parametrize("ks,d", [(3, 1), (5, 2)])
def test_plane_beyond_32_bit_offsets(ks, d):
    note("large plane %dx%d k%d d%d bf16" % (H, W, ks, d))
    assert H * W * 32 * 2 > 2 ** 31
    q, k, v, rpb = _inputs(ks, seed=ks * 10 + d)
    out = na2d.forward(q, k, v, rpb, ks, d)
    out_l, lse = na2d.forward_lse(q, k, v, rpb, ks, d)
    with pytest.raises(na2d.Na2dError) as e:
        na2d.forward(q, k, v, rpb, ks, d, algo="mfma")
    assert e.value.status == na2d.NOT_SUPPORTED
    unf = na2d.forward_unfused(q, k, v, rpb, ks, d)
    torch.cuda.synchronize()
    assert torch.equal(out, out_l)
    r64 = rpb.cpu().double().numpy()
    for (rows, cols), keep in _crops():
        crop = [t[:, :, rows, cols].cpu().double().numpy() for t in (q, k, v)]
        ref = oracle.forward(*crop, r64, ks, d, lse=True)
        sel = (slice(None), slice(None), keep, keep)
        for got in (out, unf):
            g = got[:, :, rows, cols].cpu().double().numpy()[sel]
            err = float(np.abs(g - ref["out"][sel]).max())
            assert err <= TOL["bf16"], err
        gl = lse[:, :, rows, cols].cpu().double().numpy()[sel]
        assert float(np.abs(gl - ref["lse"][sel]).max()) <= 2e-5
