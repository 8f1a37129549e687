// na2d_api.hip -- the C ABI of libna2d: argument checking and dispatch.
//
// Every check runs before the first HIP call, so an invalid call has no side
// effect on the device or the stream.  See include/na2d.h for the contract.
#include "na2d_internal.h"

#include <limits.h>

#include <atomic>

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 60;   // keeps byte counts (x4) in int64
constexpr int64_t kMaxStride = (int64_t)1 << 58;  // per dimension, stride * (extent - 1)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
  if (!a || !b) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int64_t elem_bytes(na2d_dtype_t dt) { return dt == NA2D_DTYPE_F32 ? 4 : 2; }

bool dtype_ok(int dt) {
  return dt == NA2D_DTYPE_F32 || dt == NA2D_DTYPE_BF16 || dt == NA2D_DTYPE_F16;
}

// Checks shared by every entry point.  D < 0 means "no head dimension".
na2d_status_t check_shape(int B, int heads, int H, int W, int D, int ks, int dil,
                          na2d::Shape *s) {
  if (B < 1 || heads < 1 || H < 1 || W < 1 || (D != -1 && D < 1)) return NA2D_ERROR_INVALID_VALUE;
  if (ks < 1 || (ks % 2) == 0 || dil < 1) return NA2D_ERROR_INVALID_VALUE;
  // The window must fit inside every residue class: H >= k*d (else pad).
  if ((int64_t)ks * dil > H || (int64_t)ks * dil > W) return NA2D_ERROR_INVALID_VALUE;
  // B*heads*H*W*max(D, k*k) must stay below 2^60; multiply step by step so
  // the check itself cannot overflow.
  const int64_t width = (int64_t)ks * ks > (D > 0 ? D : 1) ? (int64_t)ks * ks : (D > 0 ? D : 1);
  int64_t nq = width;
  const int64_t factors[4] = {B, heads, H, W};
  for (int64_t f : factors) {
    if (nq > kMaxElems / f) return NA2D_ERROR_INVALID_VALUE;
    nq *= f;
  }
  nq /= width;
  if (D != -1 && D != na2d::kHeadDim) return NA2D_ERROR_NOT_SUPPORTED;
  if (ks > na2d::kMaxKernel) return NA2D_ERROR_NOT_SUPPORTED;
  s->B = B; s->heads = heads; s->H = H; s->W = W; s->ks = ks; s->dil = dil; s->n_query = nq;
  return NA2D_SUCCESS;
}

na2d_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return NA2D_SUCCESS;
  return e == hipErrorInvalidConfiguration ? NA2D_ERROR_NOT_SUPPORTED : NA2D_ERROR_LAUNCH_FAILURE;
}

// Bytes from the first to one past the last element a [B, heads, H, W, D]
// view with these (non-negative) strides touches.
int64_t footprint(const na2d::Strides &t, const na2d::Shape &s, int64_t elem) {
  return ((int64_t)(s.B - 1) * t.b + (int64_t)(s.heads - 1) * t.h + (int64_t)(s.H - 1) * t.y +
          (int64_t)(s.W - 1) * t.x + na2d::kHeadDim) *
         elem;
}

// True when no two elements of the view share an address: with the
// dimensions ordered by stride, each stride must step past everything the
// smaller dimensions span (size-1 dimensions impose nothing).
bool injective(const na2d::Strides &t, const na2d::Shape &s) {
  int64_t st[4] = {t.b, t.h, t.y, t.x}, ex[4] = {s.B, s.heads, s.H, s.W};
  for (int i = 0; i < 4; ++i)  // insertion sort by stride
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      int64_t a = st[j]; st[j] = st[j - 1]; st[j - 1] = a;
      a = ex[j]; ex[j] = ex[j - 1]; ex[j - 1] = a;
    }
  int64_t span = na2d::kHeadDim;  // elements covered by the smaller dimensions
  for (int i = 0; i < 4; ++i) {
    if (ex[i] == 1) continue;
    if (st[i] < span) return false;
    span += (ex[i] - 1) * st[i];
  }
  return true;
}

// The forward pass for checked shapes, pointers, strides and padding; lse
// (optional) receives the per-query log-sum-exp.
na2d_status_t forward_checked(const void *q, const void *k, const void *v, const void *rpb,
                              void *out, const na2d::Shape &s, const na2d::Strides &in,
                              const na2d::Strides &os, const na2d::Pad &pad,
                              na2d_dtype_t dtype, na2d_algo_t algo, hipStream_t stream,
                              float *lse = nullptr) {
  const bool automatic = algo == NA2D_ALGO_AUTO;
  if (automatic) algo = dtype == NA2D_DTYPE_F32 ? NA2D_ALGO_FMA : NA2D_ALGO_MFMA;
  if (algo == NA2D_ALGO_MFMA || algo == NA2D_ALGO_MFMA_TILED) {
    if (dtype == NA2D_DTYPE_F32) return NA2D_ERROR_NOT_SUPPORTED;
    bool supported = true;
    hipError_t e = na2d::launch_fused_mfma(q, k, v, rpb, out, s, in, os, pad, dtype, stream,
                                           &supported, lse, algo == NA2D_ALGO_MFMA);
    if (supported) return from_hip(e);
    if (!automatic) return NA2D_ERROR_NOT_SUPPORTED;
    // planes too large for 32-bit in-plane offsets, and padded maps that are
    // not k*d square: the FMA kernel handles them
  }
  return from_hip(na2d::launch_fused_fma(q, k, v, rpb, out, s, in, os, pad, dtype, stream, lse));
}

// Checks of the backward entry points, workspace aside; *need receives the
// workspace bytes the problem takes.
na2d_status_t check_backward(const void *q, const void *k, const void *v, const void *rpb,
                             const void *dout, void *dq, void *dk, void *dv, float *drpb, int B,
                             int heads, int H, int W, int D, int kernel_size, int dilation,
                             na2d_dtype_t dtype, na2d::Shape *s, size_t *need) {
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, H, W, D, kernel_size, dilation, s);
  if (st != NA2D_SUCCESS) return st;
  const void *ins[] = {q, k, v, dout};
  void *outs[] = {dq, dk, dv};
  for (const void *p : ins)
    if (!p || !aligned16(p)) return NA2D_ERROR_INVALID_VALUE;
  for (void *p : outs)
    if (!p || !aligned16(p)) return NA2D_ERROR_INVALID_VALUE;
  if ((rpb && !aligned16(rpb)) || (drpb && !aligned16(drpb))) return NA2D_ERROR_INVALID_VALUE;
  *need = na2d::backward_workspace_bytes(*s, drpb != nullptr);
  return NA2D_SUCCESS;
}

// True when an output (or the workspace) overlaps another output or an input.
bool overlaps_backward(const void *workspace, size_t need, const void *q, const void *k,
                       const void *v, const void *rpb, const void *dout, void *dq, void *dk,
                       void *dv, float *drpb, const na2d::Shape &s, na2d_dtype_t dtype) {
  const int64_t tbytes = s.n_query * na2d::kHeadDim * elem_bytes(dtype);
  const int64_t side = 2 * s.ks - 1;
  const int64_t bbytes = s.heads * side * side * 4;
  const int64_t rbytes = s.heads * side * side * elem_bytes(dtype);
  struct Span { const void *p; int64_t n; };
  const Span written[] = {{dq, tbytes}, {dk, tbytes}, {dv, tbytes}, {drpb, bbytes},
                          {workspace, (int64_t)need}};
  const Span read[] = {{q, tbytes}, {k, tbytes}, {v, tbytes}, {dout, tbytes}, {rpb, rbytes}};
  for (int a = 0; a < 5; ++a) {
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(written[a].p, written[a].n, written[b].p, written[b].n)) return true;
    for (const Span &r : read)
      if (overlaps(written[a].p, written[a].n, r.p, r.n)) return true;
  }
  return false;
}

// Workspace of na2d_backward_noalloc: a fixed device array, one copy per GPU
// (loaded with the library's code object, held until the process ends).  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device and kept in scratch_addr.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> scratch_addr[kMaxDevices];

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// The device address of the scratch array on the device `stream` runs on
// (the current device for the null stream).  The first call on a device
// looks it up with that device current; a concurrent first call stores the
// same value.
na2d_status_t scratch_address(hipStream_t stream, void **addr) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return NA2D_ERROR_LAUNCH_FAILURE;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess)
    return NA2D_ERROR_INVALID_VALUE;
  if (dev < 0 || dev >= kMaxDevices) return NA2D_ERROR_NOT_SUPPORTED;
  uintptr_t a = scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return NA2D_ERROR_LAUNCH_FAILURE;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return NA2D_ERROR_LAUNCH_FAILURE;
    if (e != hipSuccess || p == nullptr) return NA2D_ERROR_LAUNCH_FAILURE;
    a = reinterpret_cast<uintptr_t>(p);
    scratch_addr[dev].store(a, std::memory_order_release);
  }
  *addr = reinterpret_cast<void *>(a);
  return NA2D_SUCCESS;
}

}  // namespace

extern "C" {

na2d_status_t na2d_forward_algo(const void *q, const void *k, const void *v, const void *rpb,
                                void *out, int B, int heads, int H, int W, int D,
                                int kernel_size, int dilation, na2d_dtype_t dtype,
                                na2d_algo_t algo, hipStream_t stream) {
  na2d::Shape s;
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  if (algo != NA2D_ALGO_AUTO && algo != NA2D_ALGO_FMA && algo != NA2D_ALGO_MFMA &&
      algo != NA2D_ALGO_MFMA_TILED)
    return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, H, W, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  if (!q || !k || !v || !out) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (rpb && !aligned16(rpb)))
    return NA2D_ERROR_INVALID_VALUE;
  const int64_t tbytes = s.n_query * D * elem_bytes(dtype);
  if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, k, tbytes) ||
      overlaps(out, tbytes, v, tbytes))
    return NA2D_ERROR_INVALID_VALUE;
  if (rpb) {
    const int64_t side = 2 * kernel_size - 1;
    if (overlaps(out, tbytes, rpb, heads * side * side * elem_bytes(dtype)))
      return NA2D_ERROR_INVALID_VALUE;
  }
  const na2d::Strides pl = na2d::planar_strides(s);
  return forward_checked(q, k, v, rpb, out, s, pl, pl, na2d::no_pad(s), dtype, algo, stream);
}

na2d_status_t na2d_forward_strided(const void *q, const void *k, const void *v,
                                   const void *rpb, void *out, int B, int heads, int H, int W,
                                   int D, int kernel_size, int dilation,
                                   const int64_t *in_strides, const int64_t *out_strides,
                                   na2d_dtype_t dtype, hipStream_t stream) {
  na2d::Shape s;
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, H, W, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  if (!q || !k || !v || !out || !in_strides || !out_strides) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (rpb && !aligned16(rpb)))
    return NA2D_ERROR_INVALID_VALUE;
  const na2d::Strides in{in_strides[0], in_strides[1], in_strides[2], in_strides[3]};
  const na2d::Strides os{out_strides[0], out_strides[1], out_strides[2], out_strides[3]};
  const int64_t eb = elem_bytes(dtype);
  const int64_t all[8] = {in.b, in.h, in.y, in.x, os.b, os.h, os.y, os.x};
  const int64_t ext[4] = {B, heads, H, W};
  for (int i = 0; i < 8; ++i) {
    const int64_t t = all[i], e = ext[i % 4];
    // bounded so that footprints stay far inside int64; every pixel's D
    // channels start on a 16-byte boundary
    if (t < 0 || t > kMaxStride || (e > 1 && t > kMaxStride / (e - 1)) || (t * eb) % 16 != 0)
      return NA2D_ERROR_INVALID_VALUE;
  }
  if (!injective(os, s)) return NA2D_ERROR_INVALID_VALUE;  // out elements must not alias
  const int64_t ib = footprint(in, s, eb), ob = footprint(os, s, eb);
  if (overlaps(out, ob, q, ib) || overlaps(out, ob, k, ib) || overlaps(out, ob, v, ib))
    return NA2D_ERROR_INVALID_VALUE;
  if (rpb) {
    const int64_t side = 2 * kernel_size - 1;
    if (overlaps(out, ob, rpb, heads * side * side * eb)) return NA2D_ERROR_INVALID_VALUE;
  }
  return forward_checked(q, k, v, rpb, out, s, in, os, na2d::no_pad(s), dtype, NA2D_ALGO_AUTO,
                         stream);
}

na2d_status_t na2d_forward_padded(const void *q, const void *k, const void *v, const void *rpb,
                                  const void *pad_k, const void *pad_v, void *out, int B,
                                  int heads, int H, int W, int D, int kernel_size,
                                  int dilation, na2d_dtype_t dtype, hipStream_t stream) {
  na2d::Shape s;
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  if (H < 1 || W < 1 || kernel_size < 1 || dilation < 1) return NA2D_ERROR_INVALID_VALUE;
  // shape rules on the padded map, then the real extent
  const int64_t span = (int64_t)kernel_size * dilation;
  const int64_t Hp = H > span ? H : span, Wp = W > span ? W : span;
  if (Hp > INT_MAX || Wp > INT_MAX) return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, (int)Hp, (int)Wp, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  s.H = H;
  s.W = W;
  s.n_query = s.n_query / ((int64_t)Hp * Wp) * ((int64_t)H * W);
  if (!q || !k || !v || !out) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (rpb && !aligned16(rpb)) || (pad_k && !aligned16(pad_k)) || (pad_v && !aligned16(pad_v)))
    return NA2D_ERROR_INVALID_VALUE;
  const int64_t eb = elem_bytes(dtype);
  const int64_t tbytes = s.n_query * D * eb, pbytes = (int64_t)heads * D * eb;
  if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, k, tbytes) ||
      overlaps(out, tbytes, v, tbytes) || overlaps(out, tbytes, pad_k, pbytes) ||
      overlaps(out, tbytes, pad_v, pbytes))
    return NA2D_ERROR_INVALID_VALUE;
  if (rpb) {
    const int64_t side = 2 * kernel_size - 1;
    if (overlaps(out, tbytes, rpb, heads * side * side * eb)) return NA2D_ERROR_INVALID_VALUE;
  }
  const na2d::Strides pl = na2d::planar_strides(s);
  const na2d::Pad pad{pad_k, pad_v, (int)Hp, (int)Wp};
  return forward_checked(q, k, v, rpb, out, s, pl, pl, pad, dtype, NA2D_ALGO_AUTO, stream);
}

na2d_status_t na2d_forward(const void *q, const void *k, const void *v, const void *rpb,
                           void *out, int B, int heads, int H, int W, int D,
                           int kernel_size, int dilation, na2d_dtype_t dtype,
                           hipStream_t stream) {
  return na2d_forward_algo(q, k, v, rpb, out, B, heads, H, W, D, kernel_size, dilation, dtype,
                           NA2D_ALGO_AUTO, stream);
}

na2d_status_t na2d_forward_lse(const void *q, const void *k, const void *v, const void *rpb,
                               void *out, float *lse, int B, int heads, int H, int W, int D,
                               int kernel_size, int dilation, na2d_dtype_t dtype,
                               hipStream_t stream) {
  na2d::Shape s;
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, H, W, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  if (!q || !k || !v || !out || !lse) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse) ||
      (rpb && !aligned16(rpb)))
    return NA2D_ERROR_INVALID_VALUE;
  const int64_t tbytes = s.n_query * D * elem_bytes(dtype), lbytes = s.n_query * 4;
  const int64_t rbytes = rpb ? (int64_t)heads * (2 * kernel_size - 1) * (2 * kernel_size - 1) *
                                   elem_bytes(dtype)
                             : 0;
  struct Span {
    const void *p;
    int64_t n;
  };
  const Span read[] = {{q, tbytes}, {k, tbytes}, {v, tbytes}, {rpb, rbytes}};
  for (const Span &r : read)
    if (overlaps(out, tbytes, r.p, r.n) || overlaps(lse, lbytes, r.p, r.n))
      return NA2D_ERROR_INVALID_VALUE;
  if (overlaps(out, tbytes, lse, lbytes)) return NA2D_ERROR_INVALID_VALUE;
  const na2d::Strides pl = na2d::planar_strides(s);
  return forward_checked(q, k, v, rpb, out, s, pl, pl, na2d::no_pad(s), dtype, NA2D_ALGO_AUTO,
                         stream, lse);
}

na2d_status_t na2d_linear(const void *x, const void *w, const void *b, void *y, int64_t M,
                          int N, int K, na2d_dtype_t dtype, hipStream_t stream) {
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  if (M < 1 || N < 1 || K < 1 || M > kMaxElems / N || M > kMaxElems / K)
    return NA2D_ERROR_INVALID_VALUE;
  if (!x || !w || !y) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (b && !aligned16(b)))
    return NA2D_ERROR_INVALID_VALUE;
  const int64_t eb = elem_bytes(dtype);
  const int64_t yb = M * N * eb;
  if (overlaps(y, yb, x, M * K * eb) || overlaps(y, yb, w, (int64_t)N * K * eb) ||
      overlaps(y, yb, b, N * eb))
    return NA2D_ERROR_INVALID_VALUE;
  if (!na2d::linear_supported(N, K)) return NA2D_ERROR_NOT_SUPPORTED;
  return from_hip(na2d::launch_linear(x, w, b, y, M, N, K, dtype, stream));
}

size_t na2d_block_workspace_size(int B, int H, int W, int C, int heads, na2d_dtype_t dtype) {
  if (!dtype_ok(dtype) || B < 1 || H < 1 || W < 1 || C < 1 || heads < 1) return 0;
  const int64_t M = (int64_t)B * H * W;
  if (M > kMaxElems / (4 * (int64_t)C)) return 0;
  return (size_t)(M * 4 * C * elem_bytes(dtype));
}

na2d_status_t na2d_block_forward(const void *x, const void *w_qkv, const void *b_qkv,
                                 const void *rpb, const void *w_out, const void *b_out,
                                 void *y, void *workspace, size_t workspace_bytes, int B, int H,
                                 int W, int C, int heads, int kernel_size, int dilation,
                                 na2d_dtype_t dtype, hipStream_t stream) {
  return na2d_block_forward_path(x, w_qkv, b_qkv, rpb, w_out, b_out, y, workspace,
                                 workspace_bytes, B, H, W, C, heads, kernel_size, dilation, dtype,
                                 NA2D_BLOCK_AUTO, stream);
}

na2d_status_t na2d_block_forward_path(const void *x, const void *w_qkv, const void *b_qkv,
                                      const void *rpb, const void *w_out, const void *b_out,
                                      void *y, void *workspace, size_t workspace_bytes, int B,
                                      int H, int W, int C, int heads, int kernel_size,
                                      int dilation, na2d_dtype_t dtype, na2d_block_path_t path,
                                      hipStream_t stream) {
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  if (path != NA2D_BLOCK_AUTO && path != NA2D_BLOCK_UNFUSED && path != NA2D_BLOCK_FUSED)
    return NA2D_ERROR_INVALID_VALUE;
  if (B < 1 || H < 1 || W < 1 || C < 1 || heads < 1 || kernel_size < 1 || dilation < 1)
    return NA2D_ERROR_INVALID_VALUE;
  if (C % heads != 0) return NA2D_ERROR_INVALID_VALUE;
  const int D = C / heads;
  // the attention step: shape rules on the padded map (maps below k*d are
  // padded as the layer does), then the real extent
  const int64_t span = (int64_t)kernel_size * dilation;
  const int64_t Hp = H > span ? H : span, Wp = W > span ? W : span;
  if (Hp > INT_MAX || Wp > INT_MAX) return NA2D_ERROR_INVALID_VALUE;
  na2d::Shape s;
  na2d_status_t st = check_shape(B, heads, (int)Hp, (int)Wp, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  s.H = H;
  s.W = W;
  s.n_query = s.n_query / ((int64_t)Hp * Wp) * ((int64_t)H * W);
  const int64_t M = (int64_t)B * H * W;
  if (M > kMaxElems / (4 * (int64_t)C)) return NA2D_ERROR_INVALID_VALUE;
  // the fused kernel needs no workspace: a forced fused call may pass none
  const bool fused = path != NA2D_BLOCK_UNFUSED &&
                     na2d::block_fused_supported(H, W, C, heads, kernel_size, dilation, dtype);
  if (path == NA2D_BLOCK_FUSED && !fused) return NA2D_ERROR_NOT_SUPPORTED;
  const bool need_ws = path != NA2D_BLOCK_FUSED;
  if (!x || !w_qkv || !w_out || !y || (need_ws && !workspace)) return NA2D_ERROR_INVALID_VALUE;
  const void *ptrs[] = {x, w_qkv, b_qkv, rpb, w_out, b_out, y, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return NA2D_ERROR_INVALID_VALUE;
  const int64_t eb = elem_bytes(dtype);
  const size_t need = na2d_block_workspace_size(B, H, W, C, heads, dtype);
  if (need == 0) return NA2D_ERROR_INVALID_VALUE;
  if (need_ws && workspace_bytes < need) return NA2D_ERROR_INVALID_VALUE;
  const int64_t side = 2 * kernel_size - 1;
  struct Span {
    const void *p;
    int64_t n;
  };
  const Span read[] = {{x, M * C * eb},          {w_qkv, 3LL * C * C * eb},
                       {b_qkv, 3LL * C * eb},    {rpb, heads * side * side * eb},
                       {w_out, (int64_t)C * C * eb}, {b_out, C * eb}};
  // (the workspace is validated whenever the three-launch path may run, also
  // when the automatic choice then takes the fused kernel)
  const int64_t wsn = need_ws ? (int64_t)need : 0;
  const Span written[] = {{y, M * C * eb}, {workspace, wsn}};
  for (const Span &wr : written)
    for (const Span &rd : read)
      if (overlaps(wr.p, wr.n, rd.p, rd.n)) return NA2D_ERROR_INVALID_VALUE;
  if (overlaps(y, M * C * eb, workspace, wsn)) return NA2D_ERROR_INVALID_VALUE;
  if (fused)
    return from_hip(na2d::launch_block_fused(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W,
                                             kernel_size, dtype, stream));
  if (!na2d::linear_planar_supported(M, C, heads) || !na2d::linear_supported(C, C))
    return NA2D_ERROR_NOT_SUPPORTED;
  // 1. q, k, v = x w_qkv^T + b_qkv, written as three dense [B, heads, H, W, D]
  //    tensors (each head's rows contiguous, so the attention reads no line
  //    shared with another head's or another projection's channels)
  char *qkv = (char *)workspace;
  const int64_t third = M * C * eb;
  char *ctx = qkv + 3 * third;
  hipError_t e =
      na2d::launch_linear_qkv_planar(x, w_qkv, b_qkv, qkv, B, H * W, C, heads, dtype, stream);
  if (e != hipSuccess) return from_hip(e);
  // 2. per-head attention into ctx [M, C] (channels-last, the output
  //    projection's input); padded pixels carry the key/value biases (the
  //    projection of a zero feature)
  const na2d::Strides in = na2d::planar_strides(s);
  const na2d::Strides os{(int64_t)H * W * C, D, (int64_t)W * C, C};
  const char *bq = (const char *)b_qkv;
  const na2d::Pad pad{bq ? bq + C * eb : nullptr, bq ? bq + 2 * C * eb : nullptr, (int)Hp,
                      (int)Wp};
  st = forward_checked(qkv, qkv + third, qkv + 2 * third, rpb, ctx, s, in, os, pad, dtype,
                       NA2D_ALGO_AUTO, stream);
  if (st != NA2D_SUCCESS) return st;
  // 3. y = ctx w_out^T + b_out
  return from_hip(na2d::launch_linear(ctx, w_out, b_out, y, M, C, C, dtype, stream));
}

na2d_status_t na2d_qkrpb(const void *q, const void *k, const void *rpb, float *attn,
                         int B, int heads, int H, int W, int D, int kernel_size,
                         int dilation, na2d_dtype_t dtype, hipStream_t stream) {
  na2d::Shape s;
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, H, W, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  if (!q || !k || !attn) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(attn) || (rpb && !aligned16(rpb)))
    return NA2D_ERROR_INVALID_VALUE;
  const int64_t tbytes = s.n_query * D * elem_bytes(dtype);
  const int64_t abytes = s.n_query * kernel_size * kernel_size * 4;
  if (overlaps(attn, abytes, q, tbytes) || overlaps(attn, abytes, k, tbytes))
    return NA2D_ERROR_INVALID_VALUE;
  if (rpb) {
    const int64_t side = 2 * kernel_size - 1;
    if (overlaps(attn, abytes, rpb, heads * side * side * elem_bytes(dtype)))
      return NA2D_ERROR_INVALID_VALUE;
  }
  return from_hip(na2d::launch_qkrpb(q, k, rpb, attn, s, dtype, stream));
}

na2d_status_t na2d_softmax(const float *attn_in, float *attn_out, int B, int heads, int H,
                           int W, int kernel_size, hipStream_t stream) {
  na2d::Shape s;
  // Rows only need the window to be well formed; dilation plays no role here.
  na2d_status_t st = check_shape(B, heads, H, W, -1, kernel_size, 1, &s);
  if (st != NA2D_SUCCESS) return st;
  if (!attn_in || !attn_out) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(attn_in) || !aligned16(attn_out)) return NA2D_ERROR_INVALID_VALUE;
  const int64_t abytes = s.n_query * kernel_size * kernel_size * 4;
  if (attn_in != attn_out && overlaps(attn_in, abytes, attn_out, abytes))
    return NA2D_ERROR_INVALID_VALUE;
  return from_hip(na2d::launch_softmax(attn_in, attn_out, s, stream));
}

na2d_status_t na2d_av(const float *attn, const void *v, void *out, int B, int heads, int H,
                      int W, int D, int kernel_size, int dilation, na2d_dtype_t dtype,
                      hipStream_t stream) {
  na2d::Shape s;
  if (!dtype_ok(dtype)) return NA2D_ERROR_INVALID_VALUE;
  na2d_status_t st = check_shape(B, heads, H, W, D, kernel_size, dilation, &s);
  if (st != NA2D_SUCCESS) return st;
  if (!attn || !v || !out) return NA2D_ERROR_INVALID_VALUE;
  if (!aligned16(attn) || !aligned16(v) || !aligned16(out)) return NA2D_ERROR_INVALID_VALUE;
  const int64_t tbytes = s.n_query * D * elem_bytes(dtype);
  const int64_t abytes = s.n_query * kernel_size * kernel_size * 4;
  if (overlaps(out, tbytes, v, tbytes) || overlaps(out, tbytes, attn, abytes))
    return NA2D_ERROR_INVALID_VALUE;
  return from_hip(na2d::launch_av(attn, v, out, s, dtype, stream));
}

size_t na2d_backward_workspace_size(int B, int heads, int H, int W, int D, int kernel_size,
                                    int dilation, int with_bias_grad) {
  na2d::Shape s;
  if (check_shape(B, heads, H, W, D, kernel_size, dilation, &s) != NA2D_SUCCESS) return 0;
  return na2d::backward_workspace_bytes(s, with_bias_grad != 0);
}

na2d_status_t na2d_backward(const void *q, const void *k, const void *v, const void *rpb,
                            const void *dout, void *dq, void *dk, void *dv, float *drpb,
                            void *workspace, size_t workspace_bytes, int B, int heads, int H,
                            int W, int D, int kernel_size, int dilation, na2d_dtype_t dtype,
                            hipStream_t stream) {
  na2d::Shape s;
  size_t need = 0;
  na2d_status_t st = check_backward(q, k, v, rpb, dout, dq, dk, dv, drpb, B, heads, H, W, D,
                                    kernel_size, dilation, dtype, &s, &need);
  if (st != NA2D_SUCCESS) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < need)
    return NA2D_ERROR_INVALID_VALUE;
  if (overlaps_backward(workspace, need, q, k, v, rpb, dout, dq, dk, dv, drpb, s, dtype))
    return NA2D_ERROR_INVALID_VALUE;
  return from_hip(na2d::launch_backward(q, k, v, rpb, dout, dq, dk, dv, drpb, workspace, s, dtype,
                                        stream));
}

na2d_status_t na2d_backward_noalloc(const void *q, const void *k, const void *v,
                                    const void *rpb, const void *dout, void *dq, void *dk,
                                    void *dv, float *drpb, int B, int heads, int H, int W, int D,
                                    int kernel_size, int dilation, na2d_dtype_t dtype,
                                    hipStream_t stream) {
  na2d::Shape s;
  size_t need = 0;
  na2d_status_t st = check_backward(q, k, v, rpb, dout, dq, dk, dv, drpb, B, heads, H, W, D,
                                    kernel_size, dilation, dtype, &s, &need);
  if (st != NA2D_SUCCESS) return st;
  if (need > kScratchBytes) return NA2D_ERROR_WORKSPACE_LIMIT;  // before any HIP call
  if (overlaps_backward(nullptr, 0, q, k, v, rpb, dout, dq, dk, dv, drpb, s, dtype))
    return NA2D_ERROR_INVALID_VALUE;
  void *ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != NA2D_SUCCESS) return st;
  if (overlaps_backward(ws, need, q, k, v, rpb, dout, dq, dk, dv, drpb, s, dtype))
    return NA2D_ERROR_INVALID_VALUE;
  // the same kernels as na2d_backward, with the device array as workspace
  // (they only write it before reading it: nothing needs clearing)
  return from_hip(na2d::launch_backward(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, dtype,
                                        stream));
}

size_t na2d_backward_noalloc_limit(void) { return kScratchBytes; }

const char *na2d_status_string(na2d_status_t status) {
  switch (status) {
    case NA2D_SUCCESS: return "NA2D_SUCCESS: no error";
    case NA2D_ERROR_INVALID_VALUE:
      return "NA2D_ERROR_INVALID_VALUE: invalid argument (sizes, kernel_size, dilation, "
             "map smaller than kernel_size*dilation, NULL/unaligned pointer, dtype, overlap)";
    case NA2D_ERROR_NOT_SUPPORTED:
      return "NA2D_ERROR_NOT_SUPPORTED: valid but not implemented (D != 32, kernel_size > 13, "
             "MFMA with fp32, or grid too large)";
    case NA2D_ERROR_LAUNCH_FAILURE: return "NA2D_ERROR_LAUNCH_FAILURE: kernel launch failed";
    case NA2D_ERROR_WORKSPACE_LIMIT:
      return "NA2D_ERROR_WORKSPACE_LIMIT: the problem needs more workspace than the "
             "allocation-free entry point's fixed device array holds "
             "(na2d_backward_noalloc_limit() bytes)";
  }
  return "unknown na2d status";
}

int na2d_version(void) { return 100; }

}  // extern "C"
