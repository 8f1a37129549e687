// na2d_internal.h -- helpers shared by the kernels of libna2d (gfx950 only).
//
// Index conventions (NAT repository README, introduction: edge pixels are
// special cases; DiNAT walk-through blog, "What is DiNAT": dilation d samples
// every d-th pixel and keeps k*k tokens):
//   a pixel row i belongs to residue class ry = i % d at sub-grid row ci = i / d;
//   that class has Ly = ceil((H - ry) / d) rows;
//   the query's window covers sub-grid rows [sy, sy + k) with
//   sy = clamp(ci - k/2, 0, Ly - k)  (centred, shifted inward at the borders);
//   the same holds for columns.
// All kernels below work in these sub-grid coordinates and translate to
// pixel rows ry + d * row only when they touch memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/na2d.h"

namespace na2d {

constexpr int kHeadDim = 32;      // D supported by this build
constexpr int kMaxKernel = 13;    // largest supported kernel_size
constexpr float kLog2e = 1.4426950408889634f;
// The matrix-core kernel addresses a (batch, head) plane with 32-bit byte
// offsets and 24-bit pixel products: planes must hold fewer pixels than this.
constexpr int64_t kMaxPlanePixels = int64_t(1) << 24;

__host__ __device__ __forceinline__ int window_start(int c, int len, int ks) {
  int s = c - ks / 2;
  s = s < 0 ? 0 : s;
  return s > len - ks ? len - ks : s;
}

__host__ __device__ __forceinline__ int class_len(int n, int residue, int dil) {
  return (n - residue + dil - 1) / dil;
}

// Element traits: load widening to fp32 and RNE narrowing on store.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Elem<__bf16> {
  static __device__ __forceinline__ float to_f(__bf16 x) { return static_cast<float>(x); }
  static __device__ __forceinline__ __bf16 from_f(float x) { return static_cast<__bf16>(x); }
};
template <> struct Elem<_Float16> {
  static __device__ __forceinline__ float to_f(_Float16 x) { return static_cast<float>(x); }
  static __device__ __forceinline__ _Float16 from_f(float x) { return static_cast<_Float16>(x); }
};

// Workgroups of one dispatch are handed to the 8 XCDs of the chip
// round-robin (id % 8).  Renumber them so that each XCD receives one
// contiguous run of logical ids: neighbouring tiles, which share halo rows
// and (for d > 1) cache lines of adjacent residue classes, then meet in the
// same L2.
__device__ __forceinline__ int xcd_contiguous_id(int bid, int n) {
  constexpr int kXcds = 8;
  const int per = n / kXcds, rem = n % kXcds;
  const int x = bid % kXcds, slot = bid / kXcds;
  return x * per + (x < rem ? x : rem) + slot;
}

// Compute units of the current device, queried at every launch: the runtime
// answers from its cached device properties, and keeping no copy here leaves
// the library without mutable global state (concurrent first launches from
// several host threads need no synchronisation).
inline int device_compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

// Division by a divisor fixed at launch: n / d == (umulhi(n, mul) + n) >> shr
// for 0 <= n < 2^31 (round-up multiplier method of Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994).  Replaces
// the ~40-instruction scalar division sequence in workgroup-id decoding.
struct FastDiv {
  uint32_t div, mul, shr;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.mul) + n) >> f.shr;
}

// Problem description passed by value to every kernel.
struct Shape {
  int B, heads, H, W, ks, dil;
  int64_t n_query;  // B * heads * H * W
};

// Element strides of a tensor seen as [B, heads, H, W, D] with D contiguous:
// element (b, h, i, j, e) sits at b*b + h*h + i*y + j*x + e.  The dense
// layout is one choice of strides; channels-last hidden states
// ([B, H, W, heads*D], DiNAT walk-through blog, encoder section) another.
struct Strides {
  int64_t b, h, y, x;
};

inline Strides planar_strides(const Shape &s) {
  const int64_t px = kHeadDim, row = (int64_t)s.W * px, plane = (int64_t)s.H * row;
  return Strides{plane * s.heads, plane, row, px};
}

inline bool is_planar(const Strides &t, const Shape &s) {
  const Strides p = planar_strides(s);
  return t.b == p.b && t.h == p.h && t.y == p.y && t.x == p.x;
}

// Padding of a map smaller than kernel_size * dilation (the DiNAT layer's
// maybe_pad): the operator runs on an Hp x Wp map (Hp = max(H, k*d), the same
// for Wp) whose pixels at row >= H or column >= W hold the head's pad key
// and value (D-vectors, [heads, D]; NULL = zeros).  Shape keeps the real H, W.
struct Pad {
  const void *k, *v;
  int Hp, Wp;
};

inline Pad no_pad(const Shape &s) { return Pad{nullptr, nullptr, s.H, s.W}; }

// Launchers (one per kernel family); each returns hipSuccess or the launch
// error.  Argument checking happens before these are reached.  q, k and v
// share the strides `in`; out has its own.  lse (optional, fp32, one value
// per query in dense [B, heads, H, W] order) receives each query's natural
// log-sum-exp of its window scores; the matrix-core launchers take it for
// dense [B, heads, H, W, D] q/k/v only (else *supported = false).
hipError_t launch_fused_fma(const void *q, const void *k, const void *v, const void *rpb,
                            void *out, const Shape &s, const Strides &in, const Strides &out_st,
                            const Pad &pad, na2d_dtype_t dt, hipStream_t st,
                            float *lse = nullptr);
// stream: the row-streaming kernel may run (maps without dilation, k <= 7,
// no log-sum-exp output); false keeps to the block-tiled kernels.
hipError_t launch_fused_mfma(const void *q, const void *k, const void *v, const void *rpb,
                             void *out, const Shape &s, const Strides &in,
                             const Strides &out_st, const Pad &pad, na2d_dtype_t dt,
                             hipStream_t st, bool *supported, float *lse = nullptr,
                             bool stream = true);
// Whole-sub-grid kernel (H == W == k*d); sets *supported = false when the
// problem is not of that kind.  Strides in bytes (mfma::ByteStrides).
namespace mfma {
struct ByteStrides;
}
hipError_t launch_dense_mfma(const void *q, const void *k, const void *v, const void *rpb,
                             void *out, const Shape &s, const mfma::ByteStrides &in,
                             const mfma::ByteStrides &out_st, const Pad &pad,
                             na2d_dtype_t dt, hipStream_t st, bool *supported,
                             float *lse = nullptr);
// Row-streaming kernel (k in {3, 5, 7}, 16-bit data, maps -- with dilation d
// dividing H and W, residue classes -- at k = 7 more than 32 columns wide and
// at least 16 rows high, at k = 3 and 5 at least k columns and max(k, 4)
// rows); byte strides as the general kernel's; lse (optional) as the general
// kernel's, dense q only.
bool stream_mfma_supported(const Shape &s, na2d_dtype_t dt);
hipError_t launch_stream_mfma(const void *q, const void *k, const void *v, const void *rpb,
                              void *out, float *lse, const Shape &s,
                              const mfma::ByteStrides &si, const mfma::ByteStrides &so,
                              na2d_dtype_t dt, hipStream_t st);
// Scores + bias of the unfused path on the matrix cores (bf16/fp16, k <= 9,
// planes within the general forward kernel's 32-bit offsets); *supported =
// false otherwise.
hipError_t launch_scores_mfma(const void *q, const void *k, const void *rpb, float *attn,
                              const Shape &s, na2d_dtype_t dt, hipStream_t st, bool *supported);
hipError_t launch_qkrpb(const void *q, const void *k, const void *rpb, float *attn,
                        const Shape &s, na2d_dtype_t dt, hipStream_t st);
hipError_t launch_softmax(const float *in, float *out, const Shape &s, hipStream_t st);
// Backward pass (three kernels); ws holds backward_workspace_bytes(s, drpb).
// The matrix-core kernels take bf16/fp16 with 3 <= k <= 13, the per-lane
// kernels everything else.
size_t backward_workspace_bytes(const Shape &s, bool with_bias);
bool backward_mfma_supported(const Shape &s, na2d_dtype_t dt);
size_t backward_mfma_workspace_bytes(const Shape &s, bool with_bias);
hipError_t launch_backward_mfma(const void *q, const void *k, const void *v, const void *rpb,
                                const void *dout, void *dq, void *dk, void *dv, float *drpb,
                                void *ws, const Shape &s, na2d_dtype_t dt, hipStream_t st);
hipError_t launch_backward(const void *q, const void *k, const void *v, const void *rpb,
                           const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                           const Shape &s, na2d_dtype_t dt, hipStream_t st);
hipError_t launch_av(const float *attn, const void *v, void *out, const Shape &s,
                     na2d_dtype_t dt, hipStream_t st);
// y[M, N] = x[M, K] . w[N, K]^T + b (b may be null); N % 16 == 0, K % 32 == 0.
bool linear_supported(int N, int K);
hipError_t launch_linear(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                         int K, na2d_dtype_t dt, hipStream_t st);
// The attention block in one kernel (projections, attention, projection):
// C = 64 in 2 heads, k in {3, 5, 7}, no dilation, no padding, bf16 / fp16.
bool block_fused_supported(int H, int W, int C, int heads, int ks, int dil, na2d_dtype_t dt);
hipError_t launch_block_fused(const void *x, const void *w_qkv, const void *b_qkv,
                              const void *rpb, const void *w_out, const void *b_out, void *y,
                              int B, int H, int W, int ks, na2d_dtype_t dt, hipStream_t st);
// The q|k|v projection (w[3C, C]) of B*HW pixels written head-planar: three
// dense [B, heads, H, W, C/heads] tensors at y, y + B*HW*C, y + 2*B*HW*C.
bool linear_planar_supported(int64_t pixels, int C, int heads);
hipError_t launch_linear_qkv_planar(const void *x, const void *w, const void *b, void *y, int B,
                                    int HW, int C, int heads, na2d_dtype_t dt, hipStream_t st);

}  // namespace na2d
