// na2d_backward.hip -- backward pass of 2D (dilated) Neighborhood Attention.
//
// Gradients of sum(out * dout) with respect to q, k, v and the bias table
// (chain rule through the DiNAT module's natten2dqkrpb -> softmax -> natten2dav,
// DiNAT walk-through blog, "What is DiNAT").  For a query i with window keys n,
// scale c = 1/sqrt(D) and P recomputed from the forward definition:
//
//   dP[i,n] = dout_i . v_n,    Dq_i = sum_n P[i,n] dP[i,n]
//   dS[i,n] = P[i,n] (dP[i,n] - Dq_i)
//   dq_i    = c sum_n dS[i,n] k_n
//   dk_n    = c sum_{i : n in window(i)} dS[i,n] q_i
//   dv_n    =   sum_{i : n in window(i)} P[i,n] dout_i
//   drpb[h][offset(i,n)] += dS[i,n]
//
// Three kernels, all accumulating in fp32:
//   1. bwd_query_kernel: one lane per query, three passes over its window:
//      the log-sum-exp L_i of the scores; P and dP (parked in LDS) and their
//      dot product Dq_i; dS and dq_i.  L_i and Dq_i go to the workspace, and
//      the workgroup's share of the bias gradient (summed in a fixed order)
//      too.  Dq is formed from P and dP rather than from the rounded forward
//      output, so the gradients carry no rounding of out.
//   2. bwd_key_kernel: one lane per key: walks the queries whose windows hold
//      the key (an interval per axis, see key_queries), recomputes P and dS
//      from L and Dq, and accumulates dk and dv.
//   3. bwd_bias_reduce_kernel: adds the per-workgroup bias tables of each
//      head in workgroup order.
// Every result is a fixed-order sum, so the pass is deterministic.
#include <limits.h>

#include "na2d_internal.h"

namespace na2d {
namespace {

constexpr int kBwdThreads = 256;

// Threads per workgroup of the per-query kernel: its LDS holds two k*k rows
// (P and dP, then dS) per lane.
template <int KS> struct QueryGroup {
  static constexpr int THREADS = KS <= 5 ? 256 : (KS <= 9 ? 128 : 64);
};

template <typename T>
__device__ __forceinline__ void load_row(const T *__restrict__ p, float (&x)[kHeadDim]) {
#pragma unroll
  for (int e = 0; e < kHeadDim; ++e) x[e] = Elem<T>::to_f(p[e]);
}

// The query rows (in sub-grid steps) whose clamped windows contain key row
// y of a class of length L: [lo, hi].  window_start is non-decreasing with
// steps of at most one, so the set is an interval: a query c holds y iff
// window_start(c) <= y <= window_start(c) + k - 1.
__device__ __forceinline__ void key_queries(int y, int L, int ks, int &lo, int &hi) {
  const int r = ks / 2;
  lo = y - ks + 1 <= 0 ? 0 : y - r;
  hi = y >= L - ks ? L - 1 : min(y + r, L - 1);
}

struct PlanePos {
  int64_t plane, base;  // plane index b*heads + h, element offset of the plane
  int h, i, j;          // head, pixel row and column
  bool valid;
};

__device__ __forceinline__ PlanePos plane_pos(const Shape &s, int chunks, int threads) {
  PlanePos p;
  p.plane = blockIdx.x / chunks;
  const int pix = (int)(blockIdx.x % chunks) * threads + (int)threadIdx.x;
  p.valid = pix < s.H * s.W;
  const int px = p.valid ? pix : 0;
  p.i = px / s.W;
  p.j = px % s.W;
  p.h = (int)(p.plane % s.heads);
  p.base = p.plane * (int64_t)s.H * s.W * kHeadDim;
  return p;
}

// Kernel 1: per query.  Workspace: lse[n_query], dq_dot[n_query] (fp32), and
// when drpb is wanted, one (2k-1)^2 table per workgroup.
template <typename T, int KS>
__global__ __launch_bounds__(QueryGroup<KS>::THREADS) void bwd_query_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, const T *__restrict__ dout, T *__restrict__ dq,
    float *__restrict__ lse, float *__restrict__ dqdot, float *__restrict__ bias_part, Shape s,
    int chunks) {
  constexpr int NK = KS * KS, SIDE = 2 * KS - 1, TQ = QueryGroup<KS>::THREADS;
  // per lane: P of its window keys, and dP, later overwritten with dS (read
  // by the fixed-order bias sum together with the window offsets)
  __shared__ float pl[NK * TQ], dsl[NK * TQ];  // [n][lane]: lanes are consecutive
  __shared__ int offl[TQ];                     // -1: lane holds no query

  const PlanePos pp = plane_pos(s, chunks, TQ);
  const int d = s.dil;
  const int ry = pp.i % d, ci = pp.i / d, Ly = class_len(s.H, ry, d);
  const int rx = pp.j % d, cj = pp.j / d, Lx = class_len(s.W, rx, d);
  const int sy = window_start(ci, Ly, KS), sx = window_start(cj, Lx, KS);
  const int64_t qoff = pp.base + ((int64_t)pp.i * s.W + pp.j) * kHeadDim;
  const float scale = 1.0f / sqrtf((float)kHeadDim);

  float qv[kHeadDim], g[kHeadDim], acc[kHeadDim];
  load_row(q + qoff, qv);
  load_row(dout + qoff, g);
  // Pass 1: online max / sum of the scores (registers hold one key at a
  // time; the scores are recomputed in pass 2).
  auto score = [&](int a, int c, int64_t &ko) -> float {
    ko = pp.base + ((int64_t)(ry + (sy + a) * d) * s.W + rx + (sx + c) * d) * kHeadDim;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < kHeadDim; ++e) dot = fmaf(qv[e], Elem<T>::to_f(k[ko + e]), dot);
    float b = 0.f;
    if (rpb != nullptr)
      b = Elem<T>::to_f(rpb[(int64_t)pp.h * SIDE * SIDE + (sy + a - ci + KS - 1) * SIDE +
                             (sx + c - cj + KS - 1)]);
    return fmaf(dot, scale, b);
  };
  float mx = -INFINITY, sum = 0.f;
#pragma unroll 1
  for (int a = 0; a < KS; ++a)
#pragma unroll 1
    for (int c = 0; c < KS; ++c) {
      int64_t ko;
      const float x = score(a, c, ko);
      const float m2 = fmaxf(mx, x);
      sum = sum * expf(mx - m2) + expf(x - m2);
      mx = m2;
    }
  const float L = mx + logf(sum);
  const int lane = threadIdx.x;
  // Pass 2: P, dP and Dq = sum P dP.
  float dqd = 0.f;
#pragma unroll 1
  for (int a = 0; a < KS; ++a)
#pragma unroll 1
    for (int c = 0; c < KS; ++c) {
      int64_t ko;
      const float p = expf(score(a, c, ko) - L);
      float dp = 0.f;
#pragma unroll
      for (int e = 0; e < kHeadDim; ++e) dp = fmaf(g[e], Elem<T>::to_f(v[ko + e]), dp);
      dqd = fmaf(p, dp, dqd);
      pl[(a * KS + c) * TQ + lane] = p;
      dsl[(a * KS + c) * TQ + lane] = dp;
    }
  // Pass 3: dS and dq.
#pragma unroll
  for (int e = 0; e < kHeadDim; ++e) acc[e] = 0.f;
#pragma unroll 1
  for (int a = 0; a < KS; ++a)
#pragma unroll 1
    for (int c = 0; c < KS; ++c) {
      const int n = a * KS + c;
      const int64_t ko =
          pp.base + ((int64_t)(ry + (sy + a) * d) * s.W + rx + (sx + c) * d) * kHeadDim;
      const float ds = pl[n * TQ + lane] * (dsl[n * TQ + lane] - dqd);
      dsl[n * TQ + lane] = ds;
#pragma unroll
      for (int e = 0; e < kHeadDim; ++e) acc[e] = fmaf(ds, Elem<T>::to_f(k[ko + e]), acc[e]);
    }
  if (pp.valid) {
    const int64_t qi = qoff / kHeadDim;
#pragma unroll
    for (int e = 0; e < kHeadDim; ++e) dq[qoff + e] = Elem<T>::from_f(acc[e] * scale);
    lse[qi] = L;
    dqdot[qi] = dqd;
  }
  if (bias_part == nullptr) return;  // uniform: the whole grid skips the bias gradient
  // Bias gradient of this workgroup, in a fixed order: every lane has parked
  // its k*k dS values and parks its window offset (sy - ci + k-1,
  // sx - cj + k-1) in LDS; thread t then sums table entry t over the lanes
  // in lane order.
  offl[lane] = pp.valid ? (sy - ci + KS - 1) * SIDE + (sx - cj + KS - 1) : -1;
  __syncthreads();
  for (int t = lane; t < SIDE * SIDE; t += TQ) {
    const int ty = t / SIDE, tx = t % SIDE;
    float tot = 0.f;
    for (int l = 0; l < TQ; ++l) {
      const int o = offl[l];
      if (o < 0) continue;
      const int a = ty - o / SIDE, c = tx - o % SIDE;
      if ((unsigned)a < (unsigned)KS && (unsigned)c < (unsigned)KS) tot += dsl[(a * KS + c) * TQ + l];
    }
    bias_part[(int64_t)blockIdx.x * SIDE * SIDE + t] = tot;
  }
}

// Kernel 2: per key.
template <typename T, int KS>
__global__ __launch_bounds__(kBwdThreads) void bwd_key_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, const T *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ dqdot, T *__restrict__ dk, T *__restrict__ dv, Shape s,
    int chunks) {
  constexpr int SIDE = 2 * KS - 1;
  const PlanePos pp = plane_pos(s, chunks, kBwdThreads);
  if (!pp.valid) return;
  const int d = s.dil;
  const int ry = pp.i % d, ky = pp.i / d, Ly = class_len(s.H, ry, d);
  const int rx = pp.j % d, kx = pp.j / d, Lx = class_len(s.W, rx, d);
  const int64_t koff = pp.base + ((int64_t)pp.i * s.W + pp.j) * kHeadDim;
  const float scale = 1.0f / sqrtf((float)kHeadDim);
  float kv[kHeadDim], vv[kHeadDim], gk[kHeadDim], gv[kHeadDim];
  load_row(k + koff, kv);
  load_row(v + koff, vv);
#pragma unroll
  for (int e = 0; e < kHeadDim; ++e) gk[e] = gv[e] = 0.f;
  int ylo, yhi, xlo, xhi;
  key_queries(ky, Ly, KS, ylo, yhi);
  key_queries(kx, Lx, KS, xlo, xhi);
#pragma unroll 1
  for (int cy = ylo; cy <= yhi; ++cy) {
    const int dy = ky - cy;  // key minus query, sub-grid steps
#pragma unroll 1
    for (int cx = xlo; cx <= xhi; ++cx) {
      const int dx = kx - cx;
      const int64_t qpix = (int64_t)(ry + cy * d) * s.W + rx + cx * d;
      const int64_t qo = pp.base + qpix * kHeadDim;
      const int64_t qi = qo / kHeadDim;
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < kHeadDim; ++e) {
        dot = fmaf(Elem<T>::to_f(q[qo + e]), kv[e], dot);
        dp = fmaf(Elem<T>::to_f(dout[qo + e]), vv[e], dp);
      }
      float b = 0.f;
      if (rpb != nullptr)
        b = Elem<T>::to_f(rpb[(int64_t)pp.h * SIDE * SIDE + (dy + KS - 1) * SIDE + (dx + KS - 1)]);
      const float p = expf(fmaf(dot, scale, b) - lse[qi]);
      const float ds = p * (dp - dqdot[qi]);
#pragma unroll
      for (int e = 0; e < kHeadDim; ++e) {
        gv[e] = fmaf(p, Elem<T>::to_f(dout[qo + e]), gv[e]);
        gk[e] = fmaf(ds, Elem<T>::to_f(q[qo + e]), gk[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kHeadDim; ++e) {
    dk[koff + e] = Elem<T>::from_f(gk[e] * scale);
    dv[koff + e] = Elem<T>::from_f(gv[e]);
  }
}

// Kernel 3: drpb[h][t] = sum over the workgroups of head h (in order) of
// their tables.  Workgroup w of kernel 1 covers plane w / chunks (chunks of
// that kernel).
__global__ __launch_bounds__(kBwdThreads) void bwd_bias_reduce_kernel(
    const float *__restrict__ bias_part, float *__restrict__ drpb, int B, int heads,
    int chunks, int side2) {
  const int t = blockIdx.x * kBwdThreads + threadIdx.x;
  if (t >= heads * side2) return;
  const int h = t / side2, e = t % side2;
  float tot = 0.f;
  for (int b = 0; b < B; ++b) {
    const int64_t plane = (int64_t)b * heads + h;
    for (int c = 0; c < chunks; ++c) tot += bias_part[(plane * chunks + c) * side2 + e];
  }
  drpb[t] = tot;
}

template <typename T, int KS>
hipError_t launch_bwd_t(const void *q, const void *k, const void *v, const void *rpb,
                        const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                        const Shape &s, hipStream_t st) {
  constexpr int SIDE = 2 * KS - 1, TQ = QueryGroup<KS>::THREADS;
  const int qchunks = (s.H * s.W + TQ - 1) / TQ;
  const int kchunks = (s.H * s.W + kBwdThreads - 1) / kBwdThreads;
  const int64_t qwg = (int64_t)s.B * s.heads * qchunks, kwg = (int64_t)s.B * s.heads * kchunks;
  if (qwg > INT_MAX || kwg > INT_MAX) return hipErrorInvalidConfiguration;
  float *lse = (float *)ws;
  float *dqdot = lse + s.n_query;
  float *bias_part = drpb != nullptr ? dqdot + s.n_query : nullptr;
  bwd_query_kernel<T, KS><<<dim3((unsigned)qwg), TQ, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (const T *)dout, (T *)dq, lse,
      dqdot, bias_part, s, qchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_key_kernel<T, KS><<<dim3((unsigned)kwg), kBwdThreads, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (const T *)dout, lse, dqdot,
      (T *)dk, (T *)dv, s, kchunks);
  e = hipGetLastError();
  if (e != hipSuccess || drpb == nullptr) return e;
  const int n = s.heads * SIDE * SIDE;
  bwd_bias_reduce_kernel<<<dim3((unsigned)((n + kBwdThreads - 1) / kBwdThreads)), kBwdThreads, 0,
                           st>>>(bias_part, drpb, s.B, s.heads, qchunks, SIDE * SIDE);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dtype(const void *q, const void *k, const void *v, const void *rpb,
                            const void *dout, void *dq, void *dk, void *dv, float *drpb,
                            void *ws, const Shape &s, hipStream_t st) {
  switch (s.ks) {
    case 1: return launch_bwd_t<T, 1>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 3: return launch_bwd_t<T, 3>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 5: return launch_bwd_t<T, 5>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 7: return launch_bwd_t<T, 7>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 9: return launch_bwd_t<T, 9>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 11: return launch_bwd_t<T, 11>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 13: return launch_bwd_t<T, 13>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Large enough for either family of kernels (the size does not depend on
// the data type, which picks the family).
size_t backward_workspace_bytes(const Shape &s, bool with_bias) {
  const int side = 2 * s.ks - 1;
  const int tq = s.ks <= 5 ? QueryGroup<5>::THREADS
                           : (s.ks <= 9 ? QueryGroup<9>::THREADS : QueryGroup<13>::THREADS);
  const int64_t chunks = ((int64_t)s.H * s.W + tq - 1) / tq;
  size_t n = (size_t)s.n_query * 2 * sizeof(float);
  if (with_bias) n += (size_t)s.B * s.heads * chunks * side * side * sizeof(float);
  const size_t m = backward_mfma_workspace_bytes(s, with_bias);
  return n > m ? n : m;
}

hipError_t launch_backward(const void *q, const void *k, const void *v, const void *rpb,
                           const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                           const Shape &s, na2d_dtype_t dt, hipStream_t st) {
  if (backward_mfma_supported(s, dt))
    return launch_backward_mfma(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, dt, st);
  switch (dt) {
    case NA2D_DTYPE_F32:
      return launch_bwd_dtype<float>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case NA2D_DTYPE_BF16:
      return launch_bwd_dtype<__bf16>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case NA2D_DTYPE_F16:
      return launch_bwd_dtype<_Float16>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace na2d
