"""Seeded synthetic inputs for 2D (dilated) Neighborhood Attention.

This module only draws random numbers; it holds none of the operator's
arithmetic.  It is the one piece of code that both the HIP path and the CPU
oracle are fed from, so that both see identical input values.

Recipe (the same for every workload):
  * one ``torch.Generator('cpu')`` seeded with ``seed``;
  * q, k, v ~ N(0, 1) drawn in fp32, in that order, each [B, heads, H, W, D];
  * rpb = 0.02 * N(0, 1) drawn in fp32, shape [heads, 2k-1, 2k-1]
    (0.02 is a standard deviation, matching the DiNAT configuration's
    ``initializer_range`` convention);
  * everything is then rounded once to the run dtype (round-to-nearest-even).

The workloads mirror NAT / DiNAT feature maps: 56x56 is the stage-1 map of a
224x224 image after the patch-4 stem, heads 2/4/8/16 with 32 channels per
head, kernel 7 and dilations 1..8 follow the DiNAT configuration defaults, and
200x336 stands in for a detection-resolution stage-1 map.  No dataset is used.
"""
from __future__ import annotations

import dataclasses

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Problem:
    B: int
    heads: int
    H: int
    W: int
    D: int
    kernel_size: int
    dilation: int
    dtype: str = "bf16"

    @property
    def shape(self):
        return (self.B, self.heads, self.H, self.W, self.D)

    @property
    def rpb_shape(self):
        side = 2 * self.kernel_size - 1
        return (self.heads, side, side)

    @property
    def n_query_heads(self) -> int:
        return self.B * self.heads * self.H * self.W

    def describe(self) -> str:
        return (f"B{self.B} h{self.heads} {self.H}x{self.W} D{self.D} "
                f"k{self.kernel_size} d{self.dilation} {self.dtype}")


def make_inputs(p: Problem, seed: int = 0, device="cpu"):
    """Return (q, k, v, rpb) for problem ``p`` in dtype ``p.dtype``."""
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    q = torch.randn(p.shape, generator=g, dtype=torch.float32)
    k = torch.randn(p.shape, generator=g, dtype=torch.float32)
    v = torch.randn(p.shape, generator=g, dtype=torch.float32)
    rpb = 0.02 * torch.randn(p.rpb_shape, generator=g, dtype=torch.float32)
    dt = DTYPES[p.dtype]
    out = [t.to(dt) for t in (q, k, v, rpb)]
    if str(device) != "cpu":
        out = [t.to(device) for t in out]
    return tuple(out)


# The five workloads the library is measured and parity-checked on.
TINY = Problem(1, 1, 14, 14, 32, 7, 1, "f32")
NAT_TINY_S1 = Problem(64, 2, 56, 56, 32, 7, 1, "bf16")
DINAT_S1_D8 = Problem(64, 2, 56, 56, 32, 7, 8, "bf16")
DINAT_S2_D4 = Problem(64, 4, 28, 28, 32, 7, 4, "bf16")
NAT_TINY_SWEEP = tuple(Problem(128, h, s, s, 32, 7, 1, "bf16")
                       for s, h in ((56, 2), (28, 4), (14, 8), (7, 16)))
DETECTION = tuple(Problem(2, 6, 200, 336, 32, ks, d, dt)
                  for ks in (7, 13) for d in (1, 8) for dt in ("bf16", "f16"))
# DiNAT stage 1 of a 192x192 image: a 48x48 map under the d = 8 layer, which
# the layer pads to 56x56 (maybe_pad) before attending.
DINAT_S1_D8_PAD48 = Problem(64, 2, 48, 48, 32, 7, 8, "bf16")


# Attention-block inputs (channels-last features and projection weights).
@dataclasses.dataclass(frozen=True)
class BlockProblem:
    B: int
    H: int
    W: int
    C: int
    heads: int
    kernel_size: int
    dilation: int
    dtype: str = "bf16"

    def describe(self) -> str:
        return "B%d %dx%d C%d h%d k%d d%d %s" % (self.B, self.H, self.W, self.C, self.heads,
                                                  self.kernel_size, self.dilation, self.dtype)


def make_block_inputs(p: BlockProblem, seed: int = 0):
    """x ~ N(0, 1) [B, H, W, C]; w_qkv ~ N(0, 1/C) [3C, C]; b_qkv ~ 0.5 N(0, 1)
    [3C]; w_out ~ N(0, 1/C) [C, C]; b_out ~ 0.5 N(0, 1) [C]; rpb ~ 0.02 N(0, 1)
    [heads, 2k-1, 2k-1]; drawn in fp32 in that order from one seeded
    generator, then rounded once to the run dtype."""
    g = torch.Generator("cpu").manual_seed(seed)
    C, side = p.C, 2 * p.kernel_size - 1
    x = torch.randn(p.B, p.H, p.W, C, generator=g)
    w_qkv = torch.randn(3 * C, C, generator=g) / C ** 0.5
    b_qkv = 0.5 * torch.randn(3 * C, generator=g)
    w_out = torch.randn(C, C, generator=g) / C ** 0.5
    b_out = 0.5 * torch.randn(C, generator=g)
    rpb = 0.02 * torch.randn(p.heads, side, side, generator=g)
    dt = DTYPES[p.dtype]
    return tuple(t.to(dt) for t in (x, w_qkv, b_qkv, rpb, w_out, b_out))


# The NAT-Tiny sweep shapes as attention blocks (C = heads * 32).
BLOCK_SWEEP = tuple(BlockProblem(128, s, s, 32 * h, h, 7, 1, "bf16")
                    for s, h in ((56, 2), (28, 4), (14, 8), (7, 16)))
