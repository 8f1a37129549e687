"""C-ABI checks that need no GPU: the library loads, exports every function
include/na2d.h declares, and rejects every invalid call with the documented
status before touching the device (each call below is invalid in exactly one
way, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest
import torch

from vision_transformer_local_amd import na2d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "na2d.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
F32, BF16, F16 = 0, 1, 2
# fake, 16-byte aligned device addresses: never dereferenced because every
# call made with them fails validation first
P = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(8)]
NULL = ctypes.c_void_p(0)
S = ctypes.c_void_p(0)  # stream


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(na2d_[a-z_]+)\s*\(", text)))


def test_library_is_built_and_loads():
    assert os.path.exists(na2d.LIB_PATH)
    na2d.lib()


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert {"na2d_forward", "na2d_qkrpb", "na2d_softmax", "na2d_av",
            "na2d_status_string", "na2d_version", "na2d_forward_algo"} <= set(names)
    L = na2d.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert na2d.na2d_version() >= 100
    for code in range(4):
        s = na2d.na2d_status_string(code)
        assert s.startswith(["NA2D_SUCCESS", "NA2D_ERROR_INVALID_VALUE",
                             "NA2D_ERROR_NOT_SUPPORTED", "NA2D_ERROR_LAUNCH_FAILURE"][code])
    assert "unknown" in na2d.na2d_status_string(99)


# (B, heads, H, W, D, k, d, dtype) -> expected status, with valid pointers
FORWARD_CASES = [
    ((0, 1, 14, 14, 32, 7, 1, BF16), INVALID),
    ((1, 0, 14, 14, 32, 7, 1, BF16), INVALID),
    ((1, 1, 0, 14, 32, 7, 1, BF16), INVALID),
    ((1, 1, 14, -3, 32, 7, 1, BF16), INVALID),
    ((1, 1, 14, 14, 0, 7, 1, BF16), INVALID),
    ((1, 1, 14, 14, 32, 6, 1, BF16), INVALID),    # even kernel
    ((1, 1, 14, 14, 32, 0, 1, BF16), INVALID),
    ((1, 1, 14, 14, 32, -1, 1, BF16), INVALID),
    ((1, 1, 14, 14, 32, 7, 0, BF16), INVALID),    # dilation 0
    ((1, 1, 13, 14, 32, 7, 2, BF16), INVALID),    # H < k*d
    ((1, 1, 14, 13, 32, 7, 2, BF16), INVALID),    # W < k*d
    ((1, 1, 6, 6, 32, 7, 1, BF16), INVALID),      # map smaller than the window
    ((1, 1, 14, 14, 32, 7, 1, 3), INVALID),       # dtype outside the enum
    ((1, 1, 14, 14, 32, 7, 1, -1), INVALID),
    ((1 << 30, 1 << 30, 1 << 30, 1 << 30, 32, 7, 1, BF16), INVALID),  # > 2^60 elements
    ((1 << 20, 1 << 10, 1 << 15, 1 << 15, 32, 7, 1, BF16), INVALID),
    ((1, 1, 14, 14, 64, 7, 1, BF16), UNSUPPORTED),   # D != 32
    ((1, 1, 14, 14, 16, 7, 1, F32), UNSUPPORTED),
    ((1, 1, 30, 30, 32, 15, 2, BF16), UNSUPPORTED),  # k > 13 (map fits 15*2)
    ((1, 1, 30, 30, 32, 15, 1, BF16), UNSUPPORTED),
]


@pytest.mark.parametrize("args,expect", FORWARD_CASES)
def test_forward_validation(args, expect):
    L = na2d.lib()
    B, h, H, W, D, ks, d, dt = args
    assert L.na2d_forward(P[0], P[1], P[2], P[3], P[4], B, h, H, W, D, ks, d, dt, S) == expect
    for algo in (0, 1, 2, 3):
        assert L.na2d_forward_algo(P[0], P[1], P[2], P[3], P[4], B, h, H, W, D, ks, d, dt,
                                   algo, S) == expect
    assert L.na2d_qkrpb(P[0], P[1], P[3], P[4], B, h, H, W, D, ks, d, dt, S) == expect
    assert L.na2d_av(P[4], P[2], P[5], B, h, H, W, D, ks, d, dt, S) == expect
    assert L.na2d_forward_lse(*P[:6], B, h, H, W, D, ks, d, dt, S) == expect


VALID = (1, 2, 14, 14, 32, 7, 1, BF16)


@pytest.mark.parametrize("slot", [0, 1, 2, 4])
def test_forward_null_pointers(slot):
    L = na2d.lib()
    ptrs = list(P[:5])
    ptrs[slot] = NULL
    assert L.na2d_forward(*ptrs, *VALID, S) == INVALID


@pytest.mark.parametrize("slot", [0, 1, 2, 3, 4])
def test_forward_misaligned_pointers(slot):
    L = na2d.lib()
    ptrs = list(P[:5])
    ptrs[slot] = ctypes.c_void_p(ptrs[slot].value + 8)
    assert L.na2d_forward(*ptrs, *VALID, S) == INVALID


def test_forward_rejects_overlapping_output():
    L = na2d.lib()
    # out starts inside q
    out = ctypes.c_void_p(P[0].value + 1024)
    assert L.na2d_forward(P[0], P[1], P[2], P[3], out, *VALID, S) == INVALID
    assert L.na2d_forward(P[0], P[1], P[2], P[3], P[0], *VALID, S) == INVALID


@pytest.mark.parametrize("slot", [0, 1, 2, 4, 5])
def test_forward_lse_pointer_rules(slot):
    L = na2d.lib()
    ptrs = list(P[:6])
    assert L.na2d_forward_lse(*ptrs[:5], NULL, *VALID, S) == INVALID
    ptrs[slot] = NULL
    assert L.na2d_forward_lse(*ptrs, *VALID, S) == INVALID
    ptrs = list(P[:6])
    ptrs[slot] = ctypes.c_void_p(ptrs[slot].value + 4)
    assert L.na2d_forward_lse(*ptrs, *VALID, S) == INVALID


def test_forward_lse_rejects_overlaps():
    L = na2d.lib()
    B, h, H, W = VALID[:4]
    # lse ([B, heads, H, W] fp32) starting inside each input and inside out
    for src in range(5):
        inside = ctypes.c_void_p(P[src].value + 256)
        assert L.na2d_forward_lse(*P[:5], inside, *VALID, S) == INVALID, src
    # out starting 16 bytes before the end of lse
    out = ctypes.c_void_p(P[5].value + B * h * H * W * 4 - 16)
    assert L.na2d_forward_lse(*P[:4], out, P[5], *VALID, S) == INVALID


def test_forward_rejects_bad_algo_and_mfma_fp32():
    L = na2d.lib()
    B, h, H, W, D, ks, d, _ = VALID
    assert L.na2d_forward_algo(*P[:5], B, h, H, W, D, ks, d, BF16, 4, S) == INVALID
    assert L.na2d_forward_algo(*P[:5], B, h, H, W, D, ks, d, BF16, -1, S) == INVALID
    assert L.na2d_forward_algo(*P[:5], B, h, H, W, D, ks, d, F32, 2, S) == UNSUPPORTED
    assert L.na2d_forward_algo(*P[:5], B, h, H, W, D, ks, d, F32, 3, S) == UNSUPPORTED


def test_qkrpb_and_av_pointer_rules():
    L = na2d.lib()
    B, h, H, W, D, ks, d, dt = VALID
    assert L.na2d_qkrpb(NULL, P[1], P[3], P[4], B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_qkrpb(P[0], NULL, P[3], P[4], B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_qkrpb(P[0], P[1], P[3], NULL, B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_qkrpb(P[0], P[1], P[3], P[0], B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_av(NULL, P[2], P[5], B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_av(P[4], NULL, P[5], B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_av(P[4], P[2], NULL, B, h, H, W, D, ks, d, dt, S) == INVALID
    assert L.na2d_av(P[4], P[2], P[2], B, h, H, W, D, ks, d, dt, S) == INVALID
    mis = ctypes.c_void_p(P[4].value + 4)
    assert L.na2d_av(mis, P[2], P[5], B, h, H, W, D, ks, d, dt, S) == INVALID


def test_softmax_rules():
    L = na2d.lib()
    assert L.na2d_softmax(NULL, P[1], 1, 1, 14, 14, 7, S) == INVALID
    assert L.na2d_softmax(P[0], NULL, 1, 1, 14, 14, 7, S) == INVALID
    assert L.na2d_softmax(P[0], P[1], 1, 1, 14, 14, 8, S) == INVALID
    assert L.na2d_softmax(P[0], P[1], 0, 1, 14, 14, 7, S) == INVALID
    assert L.na2d_softmax(P[0], P[1], 1, 1, 6, 14, 7, S) == INVALID
    assert L.na2d_softmax(P[0], P[1], 1, 1, 30, 30, 15, S) == UNSUPPORTED
    # partial overlap is rejected (full aliasing = in place is allowed)
    part = ctypes.c_void_p(P[0].value + 64)
    assert L.na2d_softmax(P[0], part, 1, 1, 14, 14, 7, S) == INVALID


def test_binding_rejects_host_tensors_without_calling_the_library():
    q = torch.zeros(1, 1, 14, 14, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        na2d.na2d_forward(q, q, q, None, torch.empty_like(q), 7, 1)


def test_header_declares_extern_c_and_no_torch_types():
    text = open(HEADER).read()
    assert 'extern "C"' in text
    for banned in ("at::", "torch::", "c10::", "#include <torch", "#include <ATen"):
        assert banned not in text


# -- backward -------------------------------------------------------------
# pointers: q k v rpb dout dq dk dv drpb workspace (fake, 256 MB apart)
BP = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(10)]
BIG = ctypes.c_size_t(1 << 40)


def _backward(L, ptrs, args, ws_bytes=BIG):
    B, h, H, W, D, ks, d, dt = args
    return L.na2d_backward(*ptrs[:10], ws_bytes, B, h, H, W, D, ks, d, dt, S)


@pytest.mark.parametrize("args,expect", FORWARD_CASES)
def test_backward_validation(args, expect):
    L = na2d.lib()
    assert _backward(L, BP, args) == expect
    B, h, H, W, D, ks, d, dt = args
    if dt in (F32, BF16, F16):  # the size does not depend on the dtype
        assert L.na2d_backward_workspace_size(B, h, H, W, D, ks, d, 1) == 0


def test_backward_workspace_size():
    L = na2d.lib()
    B, h, H, W, D, ks, d, _ = VALID
    with_bias = L.na2d_backward_workspace_size(B, h, H, W, D, ks, d, 1)
    without = L.na2d_backward_workspace_size(B, h, H, W, D, ks, d, 0)
    assert without == B * h * H * W * 8  # log-sum-exp and dout.out per query, fp32
    assert with_bias > without
    # one workspace byte short is rejected
    assert _backward(L, BP, VALID, ctypes.c_size_t(with_bias - 1)) == INVALID


@pytest.mark.parametrize("slot", [0, 1, 2, 4, 5, 6, 7, 9])
def test_backward_null_pointers(slot):
    L = na2d.lib()
    ptrs = list(BP)
    ptrs[slot] = NULL
    assert _backward(L, ptrs, VALID) == INVALID


@pytest.mark.parametrize("slot", range(10))
def test_backward_misaligned_pointers(slot):
    L = na2d.lib()
    ptrs = list(BP)
    ptrs[slot] = ctypes.c_void_p(ptrs[slot].value + 4)
    assert _backward(L, ptrs, VALID) == INVALID


@pytest.mark.parametrize("a,b", [(5, 0), (5, 6), (6, 7), (7, 4), (8, 3), (9, 5), (9, 1),
                                 (5, 3), (8, 9)])
def test_backward_rejects_overlaps(a, b):
    """An output (or the workspace) placed on top of another buffer."""
    L = na2d.lib()
    ptrs = list(BP)
    ptrs[a] = ctypes.c_void_p(ptrs[b].value + 16)
    assert _backward(L, ptrs, VALID) == INVALID


# -- allocation-free backward: na2d_backward's rules, plus the array limit ---
WORKSPACE_LIMIT = 4


def _backward_noalloc(L, ptrs, args):
    B, h, H, W, D, ks, d, dt = args
    return L.na2d_backward_noalloc(*ptrs[:9], B, h, H, W, D, ks, d, dt, S)


@pytest.mark.parametrize("args,expect", FORWARD_CASES)
def test_backward_noalloc_validation(args, expect):
    assert _backward_noalloc(na2d.lib(), BP, args) == expect


@pytest.mark.parametrize("slot", [0, 1, 2, 4, 5, 6, 7])
def test_backward_noalloc_null_pointers(slot):
    ptrs = list(BP)
    ptrs[slot] = NULL
    assert _backward_noalloc(na2d.lib(), ptrs, VALID) == INVALID


@pytest.mark.parametrize("a,b", [(5, 0), (5, 6), (6, 7), (7, 4), (8, 3), (5, 3)])
def test_backward_noalloc_rejects_overlaps(a, b):
    ptrs = list(BP)
    ptrs[a] = ctypes.c_void_p(ptrs[b].value + 16)
    assert _backward_noalloc(na2d.lib(), ptrs, VALID) == INVALID


def test_backward_noalloc_limit():
    """A problem whose workspace exceeds the fixed array is refused with its
    own status before any HIP call (this host has no GPU); the limit is the
    documented 64 MiB and covers the largest detection layer."""
    L = na2d.lib()
    limit = L.na2d_backward_noalloc_limit()
    assert limit == 64 << 20
    big = (16, 8, 256, 256, 32, 7, 1, BF16)   # 2^23 queries: 64 MiB of lse/Dq alone
    assert L.na2d_backward_workspace_size(*big[:7], 1) > limit
    assert _backward_noalloc(L, BP, big) == WORKSPACE_LIMIT
    assert na2d.na2d_status_string(WORKSPACE_LIMIT).startswith("NA2D_ERROR_WORKSPACE_LIMIT")
    for det in ((2, 6, 200, 336, 32, 13, 1), (2, 6, 200, 336, 32, 13, 8),
                (64, 2, 56, 56, 32, 7, 1), (64, 2, 56, 56, 32, 7, 8)):
        assert 0 < L.na2d_backward_workspace_size(*det, 1) <= limit


# ---------------------------------------------------------------------------
# na2d_forward_strided: same shape rules, plus the stride rules.
def _strides(*vals):
    return (ctypes.c_int64 * 4)(*vals)


def _planar(B, h, H, W, D=32):
    return (h * H * W * D, H * W * D, W * D, D)


@pytest.mark.parametrize("args,expect", FORWARD_CASES)
def test_strided_forward_shape_validation(args, expect):
    L = na2d.lib()
    B, h, H, W, D, ks, d, dt = args
    st = _strides(*_planar(1, 1, 14, 14))  # valid strides; the shape decides
    assert L.na2d_forward_strided(P[0], P[1], P[2], P[3], P[4], B, h, H, W, D, ks, d, st, st,
                                  dt, S) == expect


# channels-last hidden states [B, H, W, heads*D] seen as [B, heads, H, W, D]
def _channels_last(B, h, H, W, D=32):
    return (H * W * h * D, D, W * h * D, h * D)


CL = _channels_last(2, 2, 14, 14)
STRIDE_CASES = [
    ((-32, 32, 28 * 32, 64), CL, INVALID),            # negative stride
    (CL, (896 * 14 * 2, 32, 896, -64), INVALID),
    ((CL[0], CL[1], CL[2], 36), CL, INVALID),         # 72-byte pixel steps: not 16-byte multiples
    (CL, (CL[0], 36, CL[2], CL[3]), INVALID),
    (CL, (CL[0], CL[1], CL[2], 16), INVALID),         # out pixels overlap (step < D)
    (CL, (CL[0], 0, CL[2], CL[3]), INVALID),          # both heads on the same out elements
    (CL, (CL[0], CL[1], 32, CL[3]), INVALID),         # rows collide with columns
    (CL, (0, CL[1], CL[2], CL[3]), INVALID),          # both batch items on the same out
    ((1 << 58, CL[1], CL[2], CL[3]), CL, INVALID),    # footprint overflow
]


@pytest.mark.parametrize("si,so,expect", STRIDE_CASES)
def test_strided_forward_stride_rules(si, so, expect):
    L = na2d.lib()
    B, h, H, W, D, ks, d = 2, 2, 14, 14, 32, 7, 1
    # q, k, v, out far apart so that only the stride rule can fail
    ptrs = [ctypes.c_void_p((1 << 40) * (i + 1)) for i in range(5)]
    assert L.na2d_forward_strided(*ptrs, B, h, H, W, D, ks, d, _strides(*si), _strides(*so),
                                  BF16, S) == expect


def test_strided_forward_null_strides_and_pointers():
    L = na2d.lib()
    st = _strides(*CL)
    args = (2, 2, 14, 14, 32, 7, 1)
    ptrs = [ctypes.c_void_p((1 << 40) * (i + 1)) for i in range(5)]
    assert L.na2d_forward_strided(*ptrs, *args, None, st, BF16, S) == INVALID
    assert L.na2d_forward_strided(*ptrs, *args, st, None, BF16, S) == INVALID
    for slot in (0, 1, 2, 4):
        p = list(ptrs)
        p[slot] = NULL
        assert L.na2d_forward_strided(*p, *args, st, st, BF16, S) == INVALID
        p[slot] = ctypes.c_void_p(ptrs[slot].value + 8)
        assert L.na2d_forward_strided(*p, *args, st, st, BF16, S) == INVALID


def test_strided_forward_rejects_out_overlapping_an_input():
    L = na2d.lib()
    st = _strides(*CL)
    args = (2, 2, 14, 14, 32, 7, 1)
    base = 1 << 40
    # a fused QKV buffer (q, k, v at channel offsets 0, 64, 128 of 192-channel
    # pixels) with out written into the same buffer's last channels
    qkv = (14 * 14 * 192, 32, 14 * 192, 192)
    q, k, v = (ctypes.c_void_p(base + off * 2) for off in (0, 64, 128))
    out = ctypes.c_void_p(base + 128 * 2 + 64)
    assert L.na2d_forward_strided(q, k, v, NULL, out, *args, _strides(*qkv), st, BF16,
                                  S) == INVALID
    # out starting inside v's footprint
    far = [ctypes.c_void_p((1 << 41) * (i + 1)) for i in range(3)]
    inside = ctypes.c_void_p(far[2].value + 4096)
    assert L.na2d_forward_strided(*far, NULL, inside, *args, st, st, BF16, S) == INVALID


# ---------------------------------------------------------------------------
# na2d_forward_padded: maps below k*d are valid; the rest as na2d_forward.
PADDED_CASES = [
    ((1, 1, 0, 5, 32, 7, 1, BF16), INVALID),
    ((1, 1, 5, 0, 32, 7, 1, BF16), INVALID),
    ((0, 1, 5, 5, 32, 7, 1, BF16), INVALID),
    ((1, 1, 5, 5, 32, 6, 1, BF16), INVALID),     # even kernel
    ((1, 1, 5, 5, 32, 7, 0, BF16), INVALID),
    ((1, 1, 5, 5, 32, 7, 1, 5), INVALID),
    ((1, 1, 5, 5, 64, 7, 1, BF16), UNSUPPORTED),  # D != 32
    ((1, 1, 5, 5, 32, 15, 1, BF16), UNSUPPORTED),
]


@pytest.mark.parametrize("args,expect", PADDED_CASES)
def test_padded_forward_validation(args, expect):
    L = na2d.lib()
    assert L.na2d_forward_padded(*P[:7], *args, S) == expect


def test_padded_forward_pointer_rules():
    L = na2d.lib()
    args = (1, 2, 5, 5, 32, 7, 2, BF16)
    for slot in (0, 1, 2, 6):
        p = list(P[:7])
        p[slot] = NULL
        assert L.na2d_forward_padded(*p, *args, S) == INVALID
    for slot in range(7):
        p = list(P[:7])
        p[slot] = ctypes.c_void_p(p[slot].value + 8)
        assert L.na2d_forward_padded(*p, *args, S) == INVALID
    # out overlapping a pad vector
    p = list(P[:7])
    p[6] = p[4]
    assert L.na2d_forward_padded(*p, *args, S) == INVALID


# ---------------------------------------------------------------------------
# na2d_linear and na2d_block_forward
LINEAR_CASES = [
    ((0, 64, 64, BF16), INVALID),
    ((128, 0, 64, BF16), INVALID),
    ((128, 64, -1, BF16), INVALID),
    ((128, 64, 64, 7), INVALID),
    ((1 << 58, 64, 64, BF16), INVALID),      # M*K beyond 2^60
    ((128, 40, 64, BF16), UNSUPPORTED),      # N % 16
    ((128, 64, 48, BF16), UNSUPPORTED),      # K % 32
]


@pytest.mark.parametrize("args,expect", LINEAR_CASES)
def test_linear_validation(args, expect):
    L = na2d.lib()
    far = [ctypes.c_void_p((1 << 44) * (i + 1)) for i in range(4)]
    assert L.na2d_linear(*far, *args, S) == expect


def test_linear_pointer_rules():
    L = na2d.lib()
    far = [ctypes.c_void_p((1 << 44) * (i + 1)) for i in range(4)]
    args = (1000, 64, 64, BF16)
    for slot in (0, 1, 3):
        p = list(far)
        p[slot] = NULL
        assert L.na2d_linear(*p, *args, S) == INVALID
    for slot in range(4):
        p = list(far)
        p[slot] = ctypes.c_void_p(p[slot].value + 8)
        assert L.na2d_linear(*p, *args, S) == INVALID
    p = list(far)
    p[3] = ctypes.c_void_p(far[0].value + 64)  # y inside x
    assert L.na2d_linear(*p, *args, S) == INVALID


def test_block_workspace_size():
    L = na2d.lib()
    assert L.na2d_block_workspace_size(2, 7, 9, 64, 2, BF16) == 2 * 7 * 9 * 4 * 64 * 2
    assert L.na2d_block_workspace_size(2, 7, 9, 64, 2, F32) == 2 * 7 * 9 * 4 * 64 * 4
    assert L.na2d_block_workspace_size(0, 7, 9, 64, 2, BF16) == 0
    assert L.na2d_block_workspace_size(2, 7, 9, 64, 2, 9) == 0


BLOCK_CASES = [
    ((2, 7, 9, 64, 3, 7, 1, BF16), INVALID),       # C % heads
    ((2, 7, 9, 64, 2, 6, 1, BF16), INVALID),       # even kernel
    ((0, 7, 9, 64, 2, 7, 1, BF16), INVALID),
    ((2, 7, 9, 64, 2, 7, 0, BF16), INVALID),
    ((2, 7, 9, 128, 2, 7, 1, BF16), UNSUPPORTED),  # D = 64
    ((2, 7, 9, 64, 2, 15, 1, BF16), UNSUPPORTED),  # k > 13
]


def _block(L, ptrs, args, ws_bytes=1 << 40):
    return L.na2d_block_forward(*ptrs, ws_bytes, *args, S)


@pytest.mark.parametrize("args,expect", BLOCK_CASES)
def test_block_validation(args, expect):
    L = na2d.lib()
    far = [ctypes.c_void_p((1 << 41) * (i + 1)) for i in range(8)]
    assert _block(L, far, args) == expect


def test_block_pointer_and_workspace_rules():
    L = na2d.lib()
    far = [ctypes.c_void_p((1 << 41) * (i + 1)) for i in range(8)]
    args = (2, 7, 9, 64, 2, 7, 2, BF16)
    need = L.na2d_block_workspace_size(2, 7, 9, 64, 2, BF16)
    assert _block(L, far, args, need - 1) == INVALID
    for slot in (0, 1, 4, 6, 7):
        p = list(far)
        p[slot] = NULL
        assert _block(L, p, args) == INVALID
    for slot in range(8):
        p = list(far)
        p[slot] = ctypes.c_void_p(p[slot].value + 8)
        assert _block(L, p, args) == INVALID
    for a, b in ((6, 0), (7, 1), (7, 6), (6, 4), (7, 3)):  # y/workspace over an input or each other
        p = list(far)
        p[a] = ctypes.c_void_p(p[b].value)
        assert _block(L, p, args) == INVALID


def _block_path(L, ptrs, args, path, ws_bytes=1 << 40):
    return L.na2d_block_forward_path(*ptrs, ws_bytes, *args, path, S)


def test_block_path_rules():
    L = na2d.lib()
    far = [ctypes.c_void_p((1 << 41) * (i + 1)) for i in range(8)]
    fusable = (2, 7, 9, 64, 2, 7, 1, BF16)
    assert _block_path(L, far, fusable, 3) == INVALID
    assert _block_path(L, far, fusable, -1) == INVALID
    # forced fused on what the fused kernel does not cover
    for args in ((2, 7, 9, 64, 2, 7, 2, BF16),     # dilation
                 (2, 5, 9, 64, 2, 7, 1, BF16),     # padded map
                 (2, 7, 9, 128, 4, 7, 1, BF16),    # C = 128
                 (2, 9, 9, 64, 2, 9, 1, BF16),     # k = 9
                 (2, 7, 9, 64, 2, 7, 1, F32)):
        assert _block_path(L, far, args, na2d.BLOCK_FUSED) == UNSUPPORTED
    # the workspace is required unless the fused kernel is forced
    p = list(far)
    p[7] = NULL
    for path in (na2d.BLOCK_AUTO, na2d.BLOCK_UNFUSED):
        assert _block_path(L, p, fusable, path, 0) == INVALID
    # forced fused still checks the other pointers and overlaps
    p[6] = NULL
    assert _block_path(L, p, fusable, na2d.BLOCK_FUSED, 0) == INVALID
    p = list(far)
    p[7] = NULL
    p[6] = ctypes.c_void_p(far[0].value)  # y over x
    assert _block_path(L, p, fusable, na2d.BLOCK_FUSED, 0) == INVALID
