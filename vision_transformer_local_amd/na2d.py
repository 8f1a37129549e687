"""Thin ctypes binding of libna2d (the C ABI in include/na2d.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, their device pointers and torch's current HIP stream are passed to the
library, and a non-zero status becomes a RuntimeError.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, the first call raises.

Layouts: q, k, v, out are contiguous [B, heads, H, W, D] on the GPU in one of
float32 / bfloat16 / float16; rpb is [heads, 2k-1, 2k-1] in the same dtype or
None (zero bias); attn is float32 [B, heads, H, W, k*k].  The strided forward
takes q, k, v, out as [B, heads, H, W, D] views with any strides whose last
one is 1 (e.g. channels-last hidden states viewed per head, see
``heads_view``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libna2d.so")

SUCCESS, INVALID_VALUE, NOT_SUPPORTED, LAUNCH_FAILURE = 0, 1, 2, 3
ALGOS = {"auto": 0, "fma": 1, "mfma": 2, "mfma_tiled": 3}
_DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}

_lib = None


class Na2dError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libna2d.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libna2d.so is not built (%s); run `python -m vision_transformer_local_amd.build`"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        L.na2d_forward.restype = i
        L.na2d_forward.argtypes = [vp] * 5 + [i] * 8 + [vp]
        L.na2d_forward_algo.restype = i
        L.na2d_forward_lse.restype = i
        L.na2d_forward_lse.argtypes = [vp] * 6 + [i] * 8 + [vp]
        L.na2d_forward_algo.argtypes = [vp] * 5 + [i] * 9 + [vp]
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.na2d_forward_strided.restype = i
        L.na2d_forward_strided.argtypes = [vp] * 5 + [i] * 7 + [i64p, i64p, i, vp]
        L.na2d_forward_padded.restype = i
        L.na2d_forward_padded.argtypes = [vp] * 7 + [i] * 8 + [vp]
        L.na2d_linear.restype = i
        L.na2d_linear.argtypes = [vp] * 4 + [ctypes.c_int64, i, i, i, vp]
        L.na2d_block_workspace_size.restype = ctypes.c_size_t
        L.na2d_block_workspace_size.argtypes = [i] * 6
        L.na2d_block_forward.restype = i
        L.na2d_block_forward.argtypes = [vp] * 8 + [ctypes.c_size_t] + [i] * 8 + [vp]
        L.na2d_block_forward_path.restype = i
        L.na2d_block_forward_path.argtypes = [vp] * 8 + [ctypes.c_size_t] + [i] * 9 + [vp]
        L.na2d_qkrpb.restype = i
        L.na2d_qkrpb.argtypes = [vp] * 4 + [i] * 8 + [vp]
        L.na2d_softmax.restype = i
        L.na2d_softmax.argtypes = [vp] * 2 + [i] * 5 + [vp]
        L.na2d_av.restype = i
        L.na2d_av.argtypes = [vp] * 3 + [i] * 8 + [vp]
        L.na2d_backward.restype = i
        L.na2d_backward.argtypes = [vp] * 10 + [ctypes.c_size_t] + [i] * 8 + [vp]
        L.na2d_backward_workspace_size.restype = ctypes.c_size_t
        L.na2d_backward_workspace_size.argtypes = [i] * 8
        L.na2d_backward_noalloc.restype = i
        L.na2d_backward_noalloc.argtypes = [vp] * 9 + [i] * 8 + [vp]
        L.na2d_backward_noalloc_limit.restype = ctypes.c_size_t
        L.na2d_backward_noalloc_limit.argtypes = []
        L.na2d_status_string.restype = ctypes.c_char_p
        L.na2d_status_string.argtypes = [i]
        L.na2d_version.restype = i
        L.na2d_version.argtypes = []
        _lib = L
    return _lib


def na2d_status_string(status: int) -> str:
    return lib().na2d_status_string(int(status)).decode()


def na2d_version() -> int:
    return int(lib().na2d_version())


def _check(status: int, what: str):
    if status != SUCCESS:
        raise Na2dError(status, "%s: %s" % (what, na2d_status_string(status)))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _qkv_shape(q: torch.Tensor):
    if q.dim() != 5:
        raise ValueError("q must be [B, heads, H, W, D]")
    if q.dtype not in _DTYPE_CODES:
        raise ValueError("dtype %s not supported" % q.dtype)
    return tuple(int(x) for x in q.shape)


def _rpb_check(rpb, q, heads, ks):
    if rpb is not None:
        side = 2 * ks - 1
        _need(rpb, "rpb", q.dtype, (heads, side, side))


def na2d_forward_algo(q, k, v, rpb, out, kernel_size: int, dilation: int, algo: str = "auto"):
    """Fused forward into ``out`` with an explicit kernel family."""
    B, heads, H, W, D = _qkv_shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, q.shape)
    _rpb_check(rpb, q, heads, kernel_size)
    st = lib().na2d_forward_algo(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(out),
                                 B, heads, H, W, D, int(kernel_size), int(dilation),
                                 _DTYPE_CODES[q.dtype], ALGOS[algo], _stream(q))
    _check(st, "na2d_forward_algo")
    return out


def na2d_forward_lse(q, k, v, rpb, out, lse, kernel_size: int, dilation: int):
    """Fused forward into ``out`` plus each query's log-sum-exp into ``lse``
    (fp32 [B, heads, H, W])."""
    B, heads, H, W, D = _qkv_shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, q.shape)
    _need(lse, "lse", torch.float32, (B, heads, H, W))
    _rpb_check(rpb, q, heads, kernel_size)
    st = lib().na2d_forward_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(out), _ptr(lse),
                                B, heads, H, W, D, int(kernel_size), int(dilation),
                                _DTYPE_CODES[q.dtype], _stream(q))
    _check(st, "na2d_forward_lse")
    return out, lse


def heads_view(x: torch.Tensor, heads: int) -> torch.Tensor:
    """Channels-last hidden states [B, H, W, heads*D] (or a channel slice of a
    fused QKV buffer) as the [B, heads, H, W, D] view the strided forward
    takes; no copy."""
    B, H, W, C = x.shape
    return x.unflatten(3, (heads, C // heads)).permute(0, 3, 1, 2, 4)


def _strided(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if t.stride(-1) != 1:
        raise ValueError("%s must have contiguous channels (last stride 1)" % name)
    return (ctypes.c_int64 * 4)(*[int(x) for x in t.stride()[:4]])


def na2d_forward_strided(q, k, v, rpb, out, kernel_size: int, dilation: int):
    """Fused forward into ``out`` on strided [B, heads, H, W, D] views: q, k
    and v must share their strides; out has its own (checked by the library:
    no aliasing, no overlap with the inputs)."""
    B, heads, H, W, D = _qkv_shape(q)
    si = _strided(q, "q", q.dtype, q.shape)
    for t, n in ((k, "k"), (v, "v")):
        if tuple(_strided(t, n, q.dtype, q.shape)) != tuple(si):
            raise ValueError("q, k and v must share their strides")
    so = _strided(out, "out", q.dtype, q.shape)
    _rpb_check(rpb, q, heads, kernel_size)
    st = lib().na2d_forward_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(out),
                                    B, heads, H, W, D, int(kernel_size), int(dilation),
                                    si, so, _DTYPE_CODES[q.dtype], _stream(q))
    _check(st, "na2d_forward_strided")
    return out


def na2d_forward_padded(q, k, v, rpb, pad_k, pad_v, out, kernel_size: int, dilation: int):
    """Fused forward into ``out`` on a map that may be smaller than
    kernel_size * dilation: padded below/right with the per-head pad vectors
    ``pad_k``/``pad_v`` ([heads, D] or None = zeros), attended, cropped."""
    B, heads, H, W, D = _qkv_shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, q.shape)
    for t, n in ((pad_k, "pad_k"), (pad_v, "pad_v")):
        if t is not None:
            _need(t, n, q.dtype, (heads, D))
    _rpb_check(rpb, q, heads, kernel_size)
    st = lib().na2d_forward_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(pad_k),
                                   _ptr(pad_v), _ptr(out), B, heads, H, W, D, int(kernel_size),
                                   int(dilation), _DTYPE_CODES[q.dtype], _stream(q))
    _check(st, "na2d_forward_padded")
    return out


def forward_padded(q, k, v, rpb, pad_k, pad_v, kernel_size: int, dilation: int):
    """Allocating ``na2d_forward_padded``."""
    return na2d_forward_padded(q, k, v, rpb, pad_k, pad_v, torch.empty_like(q), kernel_size,
                               dilation)


def forward_channels_last(q, k, v, rpb, heads: int, kernel_size: int, dilation: int):
    """Allocating forward on channels-last hidden states: q, k, v are
    [B, H, W, heads*D] tensors (or channel slices of one [B, H, W, 3*heads*D]
    buffer); returns out as a new contiguous [B, H, W, heads*D] tensor."""
    B, H, W, C = q.shape
    out = torch.empty((B, H, W, C), dtype=q.dtype, device=q.device)
    na2d_forward_strided(heads_view(q, heads), heads_view(k, heads), heads_view(v, heads), rpb,
                         heads_view(out, heads), kernel_size, dilation)
    return out


def na2d_forward(q, k, v, rpb, out, kernel_size: int, dilation: int):
    """Fused forward into ``out`` (MFMA kernel for bf16/fp16, FMA for fp32)."""
    B, heads, H, W, D = _qkv_shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, q.shape)
    _rpb_check(rpb, q, heads, kernel_size)
    st = lib().na2d_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(out),
                            B, heads, H, W, D, int(kernel_size), int(dilation),
                            _DTYPE_CODES[q.dtype], _stream(q))
    _check(st, "na2d_forward")
    return out


def na2d_qkrpb(q, k, rpb, attn, kernel_size: int, dilation: int):
    """Unfused step 1: fp32 scores q.k/sqrt(D) + bias into ``attn``."""
    B, heads, H, W, D = _qkv_shape(q)
    _need(q, "q")
    _need(k, "k", q.dtype, q.shape)
    _rpb_check(rpb, q, heads, kernel_size)
    _need(attn, "attn", torch.float32, (B, heads, H, W, kernel_size * kernel_size))
    st = lib().na2d_qkrpb(_ptr(q), _ptr(k), _ptr(rpb), _ptr(attn), B, heads, H, W, D,
                          int(kernel_size), int(dilation), _DTYPE_CODES[q.dtype], _stream(q))
    _check(st, "na2d_qkrpb")
    return attn


def na2d_softmax(attn_in, attn_out, kernel_size: int):
    """Unfused step 2: row softmax over the last (k*k) axis; may run in place."""
    _need(attn_in, "attn_in", torch.float32)
    if attn_in.dim() != 5 or attn_in.shape[-1] != kernel_size * kernel_size:
        raise ValueError("attn must be [B, heads, H, W, k*k]")
    _need(attn_out, "attn_out", torch.float32, attn_in.shape)
    B, heads, H, W, _ = (int(x) for x in attn_in.shape)
    st = lib().na2d_softmax(_ptr(attn_in), _ptr(attn_out), B, heads, H, W, int(kernel_size),
                            _stream(attn_in))
    _check(st, "na2d_softmax")
    return attn_out


def na2d_av(attn, v, out, kernel_size: int, dilation: int):
    """Unfused step 3: probability-weighted sum of value rows into ``out``."""
    B, heads, H, W, D = _qkv_shape(v)
    _need(v, "v")
    _need(attn, "attn", torch.float32, (B, heads, H, W, kernel_size * kernel_size))
    _need(out, "out", v.dtype, v.shape)
    st = lib().na2d_av(_ptr(attn), _ptr(v), _ptr(out), B, heads, H, W, D, int(kernel_size),
                       int(dilation), _DTYPE_CODES[v.dtype], _stream(v))
    _check(st, "na2d_av")
    return out


def na2d_backward_workspace_size(B, heads, H, W, D, kernel_size: int, dilation: int,
                                 with_bias_grad: bool) -> int:
    return int(lib().na2d_backward_workspace_size(B, heads, H, W, D, int(kernel_size),
                                                  int(dilation), int(bool(with_bias_grad))))


def na2d_backward(q, k, v, rpb, dout, dq, dk, dv, drpb, workspace, kernel_size: int,
                  dilation: int):
    """Backward pass into dq, dk, dv (and drpb, fp32, unless None); the
    workspace is a uint8 GPU tensor of at least na2d_backward_workspace_size
    bytes."""
    B, heads, H, W, D = _qkv_shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv")):
        _need(t, n, q.dtype, q.shape)
    _rpb_check(rpb, q, heads, kernel_size)
    side = 2 * kernel_size - 1
    if drpb is not None:
        _need(drpb, "drpb", torch.float32, (heads, side, side))
    _need(workspace, "workspace", torch.uint8)
    st = lib().na2d_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(dout),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drpb), _ptr(workspace),
                             workspace.numel(), B, heads, H, W, D, int(kernel_size),
                             int(dilation), _DTYPE_CODES[q.dtype], _stream(q))
    _check(st, "na2d_backward")
    return dq, dk, dv, drpb


def na2d_backward_noalloc(q, k, v, rpb, dout, dq, dk, dv, drpb, kernel_size: int,
                          dilation: int):
    """na2d_backward with the library's fixed device array as workspace (no
    allocation in the call)."""
    B, heads, H, W, D = _qkv_shape(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                 (dv, "dv")):
        _need(t, n, q.dtype, q.shape)
    _rpb_check(rpb, q, heads, kernel_size)
    side = 2 * kernel_size - 1
    if drpb is not None:
        _need(drpb, "drpb", torch.float32, (heads, side, side))
    st = lib().na2d_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(dout),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drpb), B, heads, H, W,
                                     D, int(kernel_size), int(dilation), _DTYPE_CODES[q.dtype],
                                     _stream(q))
    _check(st, "na2d_backward_noalloc")
    return dq, dk, dv, drpb


def na2d_backward_noalloc_limit() -> int:
    return int(lib().na2d_backward_noalloc_limit())


# -- allocating conveniences (torch allocates the outputs; nothing else) ----

def forward(q, k, v, rpb, kernel_size: int, dilation: int, algo: str = "auto"):
    out = torch.empty_like(q)
    return na2d_forward_algo(q, k, v, rpb, out, kernel_size, dilation, algo)


def forward_lse(q, k, v, rpb, kernel_size: int, dilation: int):
    """Allocating forward that also returns the per-query log-sum-exp."""
    B, heads, H, W, _ = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, heads, H, W), dtype=torch.float32, device=q.device)
    return na2d_forward_lse(q, k, v, rpb, out, lse, kernel_size, dilation)


def forward_unfused(q, k, v, rpb, kernel_size: int, dilation: int):
    B, heads, H, W, _ = q.shape
    attn = torch.empty((B, heads, H, W, kernel_size * kernel_size), dtype=torch.float32,
                       device=q.device)
    na2d_qkrpb(q, k, rpb, attn, kernel_size, dilation)
    na2d_softmax(attn, attn, kernel_size)
    out = torch.empty_like(v)
    na2d_av(attn, v, out, kernel_size, dilation)
    return out


def backward(q, k, v, rpb, dout, kernel_size: int, dilation: int, bias_grad: bool = True):
    """Allocating backward: returns (dq, dk, dv, drpb or None)."""
    B, heads, H, W, D = _qkv_shape(q)
    n = na2d_backward_workspace_size(B, heads, H, W, D, kernel_size, dilation, bias_grad)
    if n == 0:
        raise Na2dError(INVALID_VALUE, "na2d_backward_workspace_size: invalid problem")
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    side = 2 * kernel_size - 1
    drpb = (torch.empty((heads, side, side), dtype=torch.float32, device=q.device)
            if bias_grad else None)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    return na2d_backward(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, kernel_size, dilation)


def na2d_linear(x, w, b, y):
    """y = x w^T + b on the last dimension (x [..., K], w [N, K], b [N] or
    None, y [..., N]; all contiguous, same dtype)."""
    if x.dtype not in _DTYPE_CODES:
        raise ValueError("dtype %s not supported" % x.dtype)
    N, K = (int(d) for d in w.shape)
    if x.shape[-1] != K:
        raise ValueError("x must end in K = %d" % K)
    M = x.numel() // K
    _need(x, "x", x.dtype)
    _need(w, "w", x.dtype, (N, K))
    _need(y, "y", x.dtype, tuple(x.shape[:-1]) + (N,))
    if b is not None:
        _need(b, "b", x.dtype, (N,))
    st = lib().na2d_linear(_ptr(x), _ptr(w), _ptr(b), _ptr(y), M, N, K, _DTYPE_CODES[x.dtype],
                           _stream(x))
    _check(st, "na2d_linear")
    return y


def linear(x, w, b=None):
    """Allocating ``na2d_linear``."""
    return na2d_linear(x, w, b, torch.empty(tuple(x.shape[:-1]) + (w.shape[0],), dtype=x.dtype,
                                            device=x.device))


def na2d_block_workspace_size(B, H, W, C, heads, dtype) -> int:
    return int(lib().na2d_block_workspace_size(B, H, W, C, heads, _DTYPE_CODES[dtype]))


# na2d_block_path_t
BLOCK_AUTO, BLOCK_UNFUSED, BLOCK_FUSED = 0, 1, 2
_BLOCK_PATHS = {"auto": BLOCK_AUTO, "unfused": BLOCK_UNFUSED, "fused": BLOCK_FUSED}


def na2d_block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, y, workspace, heads: int,
                       kernel_size: int, dilation: int, path: str = "auto"):
    """The attention block on channels-last features x [B, H, W, C] into y:
    q/k/v projection, per-head NA (maps below k*d padded as the layer does),
    output projection.  workspace: a uint8 device tensor of at least
    ``na2d_block_workspace_size`` bytes (may be None with path="fused").
    path: "auto" (na2d_block_forward), "unfused" or "fused"
    (na2d_block_forward_path)."""
    if path not in _BLOCK_PATHS:
        raise ValueError("path must be one of %s" % sorted(_BLOCK_PATHS))
    if x.dim() != 4:
        raise ValueError("x must be [B, H, W, C]")
    B, H, W, C = (int(d) for d in x.shape)
    dt = x.dtype
    _need(x, "x", dt)
    _need(y, "y", dt, x.shape)
    _need(w_qkv, "w_qkv", dt, (3 * C, C))
    _need(w_out, "w_out", dt, (C, C))
    if b_qkv is not None:
        _need(b_qkv, "b_qkv", dt, (3 * C,))
    if b_out is not None:
        _need(b_out, "b_out", dt, (C,))
    side = 2 * kernel_size - 1
    if rpb is not None:
        _need(rpb, "rpb", dt, (heads, side, side))
    if workspace is not None or path != "fused":
        _need(workspace, "workspace", torch.uint8)
    wsn = workspace.numel() if workspace is not None else 0
    args = (_ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(rpb), _ptr(w_out), _ptr(b_out), _ptr(y),
            _ptr(workspace), wsn, B, H, W, C, heads, int(kernel_size), int(dilation),
            _DTYPE_CODES[dt])
    if path == "auto":
        st = lib().na2d_block_forward(*args, _stream(x))
        _check(st, "na2d_block_forward")
    else:
        st = lib().na2d_block_forward_path(*args, _BLOCK_PATHS[path], _stream(x))
        _check(st, "na2d_block_forward_path")
    return y


def block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, heads: int, kernel_size: int,
                  dilation: int, path: str = "auto"):
    """Allocating ``na2d_block_forward`` (y and, unless path="fused", the
    workspace)."""
    B, H, W, C = (int(d) for d in x.shape)
    ws = None
    if path != "fused":
        n = na2d_block_workspace_size(B, H, W, C, heads, x.dtype)
        if n == 0:
            raise Na2dError(INVALID_VALUE, "na2d_block_workspace_size: invalid problem")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
    return na2d_block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, torch.empty_like(x), ws, heads,
                              kernel_size, dilation, path)
