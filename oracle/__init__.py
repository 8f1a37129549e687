"""CPU oracle for the 2D (dilated) Neighborhood Attention forward and backward
passes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
library never imports it and shares no code with it; the oracle is plain C
(``na2d_oracle.c``), built with gcc and loaded through ctypes.

Everything is computed in float64 from the exact stored input values (a
bf16/fp16 input is widened exactly before it gets here).  The definition it
follows, with the reading taken for every point the source pages leave open,
is written out in the header comment of ``na2d_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "na2d_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_na2d_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/_na2d_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.na2d_oracle_forward.restype = ctypes.c_int
        lib.na2d_oracle_forward.argtypes = [
            dp, dp, dp, dp,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int,
            i64p, ctypes.c_int64,
            dp, dp, dp, dp, i32p, i32p, ctypes.c_int]
        lib.na2d_oracle_backward.restype = ctypes.c_int
        lib.na2d_oracle_backward.argtypes = [
            dp, dp, dp, dp, dp,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int,
            dp, dp, dp, dp, ctypes.c_int]
        lib.na2d_oracle_valid.restype = ctypes.c_int
        lib.na2d_oracle_valid.argtypes = [ctypes.c_int] * 4
        _lib = lib
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def host_cpus() -> int:
    """CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# A one-GPU job on the GPU host is granted a share of 16 CPUs, whatever the
# machine's own count (nproc there reports every core of the host).
MAX_THREADS = 16


def default_threads() -> int:
    """Oracle threads: every CPU available to the process, at most
    MAX_THREADS."""
    return max(1, min(MAX_THREADS, host_cpus()))


def _f64(x):
    # torch tensors and numpy arrays are both accepted; widening is exact.
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def valid(H: int, W: int, kernel_size: int, dilation: int) -> bool:
    return bool(_load().na2d_oracle_valid(H, W, kernel_size, dilation))


def forward(q, k, v, rpb, kernel_size: int, dilation: int, *, idx=None,
            scores: bool = False, probs: bool = False, lse: bool = False,
            neighbours: bool = False, argmax: bool = False, threads: int | None = None):
    """Oracle forward pass.

    q, k, v: [B, heads, H, W, D]; rpb: [heads, 2k-1, 2k-1] or None (zero bias).
    idx: optional 1-D array of flat query indices into B*heads*H*W; the
    results are then returned for those queries only, in that order.

    Returns a dict with ``out`` (shape [B, heads, H, W, D], or [len(idx), D])
    and, on request, ``scores``/``probs`` ([..., k*k]), ``lse`` ([...], the
    natural log of each query's softmax denominator), ``neighbours`` (flat
    pixel index i*W + j of each window slot n = a*k + c) and ``argmax``.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, heads, H, W, D] shape")
    B, heads, H, W, D = q.shape
    ks, dil = int(kernel_size), int(dilation)
    side = 2 * ks - 1
    if rpb is not None:
        rpb = _f64(rpb)
        if rpb.shape != (heads, side, side):
            raise ValueError("rpb must be [heads, 2k-1, 2k-1]")
    if idx is not None:
        idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1))
        nq = idx.shape[0]
        lead = (nq,)
    else:
        nq = B * heads * H * W
        lead = (B, heads, H, W)
    nk = ks * ks
    out = np.empty(lead + (D,), dtype=np.float64)
    s = np.empty(lead + (nk,), dtype=np.float64) if scores else None
    p = np.empty(lead + (nk,), dtype=np.float64) if probs else None
    ls = np.empty(lead, dtype=np.float64) if lse else None
    nb = np.empty(lead + (nk,), dtype=np.int32) if neighbours else None
    am = np.empty(lead, dtype=np.int32) if argmax else None
    rc = lib.na2d_oracle_forward(
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        _ptr(rpb, ctypes.c_double),
        B, heads, H, W, D, ks, dil,
        _ptr(idx, ctypes.c_int64), nq,
        _ptr(out, ctypes.c_double), _ptr(s, ctypes.c_double), _ptr(p, ctypes.c_double),
        _ptr(ls, ctypes.c_double),
        _ptr(nb, ctypes.c_int32), _ptr(am, ctypes.c_int32),
        threads if threads else default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the problem (status %d)" % rc)
    res = {"out": out}
    if scores:
        res["scores"] = s
    if probs:
        res["probs"] = p
    if lse:
        res["lse"] = ls
    if neighbours:
        res["neighbours"] = nb
    if argmax:
        res["argmax"] = am
    return res


def backward(q, k, v, rpb, dout, kernel_size: int, dilation: int, *,
             threads: int | None = None):
    """Oracle backward pass: gradients of sum(out * dout) with respect to q,
    k, v and the bias table.

    q, k, v, dout: [B, heads, H, W, D]; rpb: [heads, 2k-1, 2k-1] or None.
    Returns a dict with ``dq``, ``dk``, ``dv`` ([B, heads, H, W, D]) and
    ``drpb`` ([heads, 2k-1, 2k-1], also when rpb is None).
    """
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if q.ndim != 5 or k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout must share one [B, heads, H, W, D] shape")
    B, heads, H, W, D = q.shape
    ks, dil = int(kernel_size), int(dilation)
    side = 2 * ks - 1
    if rpb is not None:
        rpb = _f64(rpb)
        if rpb.shape != (heads, side, side):
            raise ValueError("rpb must be [heads, 2k-1, 2k-1]")
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    drpb = np.empty((heads, side, side), dtype=np.float64)
    rc = lib.na2d_oracle_backward(
        _ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
        _ptr(rpb, ctypes.c_double), _ptr(dout, ctypes.c_double),
        B, heads, H, W, D, ks, dil,
        _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double),
        _ptr(drpb, ctypes.c_double),
        threads if threads else default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the problem (status %d)" % rc)
    return {"dq": dq, "dk": dk, "dv": dv, "drpb": drpb}


def forward_padded(q, k, v, rpb, pad_k, pad_v, kernel_size: int, dilation: int, *,
                   threads: int | None = None):
    """Oracle of the padded forward pass (the DiNAT layer's maybe_pad: a map
    smaller than kernel_size * dilation is padded, attended, and cropped
    back; DiNAT walk-through blog, layer organisation).

    Readings: the padding goes below and to the right, up to
    H' = max(H, k*d) rows and W' = max(W, k*d) columns; a padded pixel holds
    key pad_k[h] and value pad_v[h] ([heads, D], None = zeros: the projection
    of a zero feature); windows are taken on the padded map; only the
    original H x W queries are returned.

    Written as the definition: build the padded tensors, run ``forward`` on
    the original queries' positions, reshape.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, heads, H, W, D] shape")
    B, heads, H, W, D = q.shape
    ks, dil = int(kernel_size), int(dilation)
    Hp, Wp = max(H, ks * dil), max(W, ks * dil)
    pk = np.zeros((heads, D)) if pad_k is None else _f64(pad_k)
    pv = np.zeros((heads, D)) if pad_v is None else _f64(pad_v)
    if pk.shape != (heads, D) or pv.shape != (heads, D):
        raise ValueError("pad_k and pad_v must be [heads, D]")
    qp = np.zeros((B, heads, Hp, Wp, D))
    kp = np.broadcast_to(pk[None, :, None, None, :], (B, heads, Hp, Wp, D)).copy()
    vp = np.broadcast_to(pv[None, :, None, None, :], (B, heads, Hp, Wp, D)).copy()
    qp[:, :, :H, :W] = q
    kp[:, :, :H, :W] = k
    vp[:, :, :H, :W] = v
    bb, hh, ii, jj = np.meshgrid(np.arange(B), np.arange(heads), np.arange(H), np.arange(W),
                                 indexing="ij")
    idx = (((bb * heads + hh) * Hp + ii) * Wp + jj).reshape(-1)
    out = forward(qp, kp, vp, rpb, ks, dil, idx=idx, threads=threads)["out"]
    return out.reshape(B, heads, H, W, D)


def block_forward(x, w_qkv, b_qkv, rpb, w_out, b_out, heads: int, kernel_size: int,
                  dilation: int, *, stored=None, threads: int | None = None):
    """Oracle of the attention block around the operator: the NA module of
    NAT / DiNAT (DiNAT walk-through blog, "What is DiNAT": query/key/value
    projections with bias -- the configuration's qkv_bias -- then
    natten2dqkrpb, softmax, natten2dav), closed by the output projection.

    x: [B, H, W, C] channels-last features; w_qkv [3C, C] (rows: the query,
    key and value projections, in that order), b_qkv [3C] or None; w_out
    [C, C], b_out [C] or None; head h owns channels h*D .. h*D + D - 1 of
    each projection (D = C / heads).  Maps smaller than kernel_size *
    dilation are handled as the layer does (``forward_padded``: the padded
    features project to the biases).  Returns y [B, H, W, C]:

        qkv = x w_qkv^T + b_qkv;  ctx = NA(q, k, v) per head;
        y = ctx w_out^T + b_out

    stored: optional function applied to qkv and ctx, for a network that
    stores those tensors in a narrower type (e.g. rounding to bf16); the
    default keeps every step exact.
    """
    x = _f64(x)
    if x.ndim != 4:
        raise ValueError("x must be [B, H, W, C]")
    B, H, W, C = x.shape
    if C % heads != 0:
        raise ValueError("C must be a multiple of heads")
    D = C // heads
    w_qkv, w_out = _f64(w_qkv), _f64(w_out)
    if w_qkv.shape != (3 * C, C) or w_out.shape != (C, C):
        raise ValueError("w_qkv must be [3C, C] and w_out [C, C]")
    b_qkv = np.zeros(3 * C) if b_qkv is None else _f64(b_qkv)
    b_out = np.zeros(C) if b_out is None else _f64(b_out)
    keep = stored if stored is not None else (lambda a: a)
    qkv = keep(x @ w_qkv.T + b_qkv)                             # [B, H, W, 3C]

    def heads_of(t):                                            # -> [B, heads, H, W, D]
        return np.ascontiguousarray(t.reshape(B, H, W, heads, D).transpose(0, 3, 1, 2, 4))

    q, k, v = (heads_of(qkv[..., i * C:(i + 1) * C]) for i in range(3))
    pad_k, pad_v = b_qkv[C:2 * C].reshape(heads, D), b_qkv[2 * C:].reshape(heads, D)
    ctx = forward_padded(q, k, v, rpb, pad_k, pad_v, kernel_size, dilation, threads=threads)
    ctx = keep(ctx.transpose(0, 2, 3, 1, 4).reshape(B, H, W, C))  # merge the heads
    return ctx @ w_out.T + b_out
