// na2d_scalar.hip -- scalar-FMA kernels of libna2d:
//   * the fused forward pass with one lane per query (every dtype), and
//   * the unfused three-kernel path that mirrors the DiNAT module's
//     natten2dqkrpb -> softmax(dim=-1) -> natten2dav decomposition
//     (DiNAT walk-through blog, section "What is DiNAT").
// Head dimension is fixed at 32; every lane keeps its query row and its
// output accumulator in registers and reads key/value rows through the L1/L2
// caches (rows are 64-128 contiguous bytes).
#include "na2d_internal.h"

namespace na2d {
namespace {

constexpr int D = kHeadDim;

template <typename T>
__device__ __forceinline__ void load_row(const T *__restrict__ p, float (&r)[D]) {
#pragma unroll
  for (int e = 0; e < D; ++e) r[e] = Elem<T>::to_f(p[e]);
}

// Decoded query position: plane = b*heads + h, pixel (i, j), and the window.
struct QueryPos {
  int64_t plane;
  int h, i, j, ry, rx, ci, cj, sy, sx;
};

// Windows are taken on the Hp x Wp map (Hp = H, Wp = W without padding).
__device__ __forceinline__ QueryPos decode_query(int64_t t, const Shape &s, int Hp = 0,
                                                 int Wp = 0) {
  QueryPos p;
  const int64_t hw = (int64_t)s.H * s.W;
  p.plane = t / hw;
  const int pix = (int)(t - p.plane * hw);
  p.i = pix / s.W;
  p.j = pix - p.i * s.W;
  p.h = (int)(p.plane % s.heads);
  p.ry = p.i % s.dil;
  p.ci = p.i / s.dil;
  p.rx = p.j % s.dil;
  p.cj = p.j / s.dil;
  p.sy = window_start(p.ci, class_len(Hp > 0 ? Hp : s.H, p.ry, s.dil), s.ks);
  p.sx = window_start(p.cj, class_len(Wp > 0 ? Wp : s.W, p.rx, s.dil), s.ks);
  return p;
}

// Bias of window slot (a, c) for this query, read from rpb[h][dy+k-1][dx+k-1].
template <typename T>
__device__ __forceinline__ float bias_of(const T *__restrict__ rpb, const QueryPos &p,
                                         const Shape &s, int a, int c) {
  if (!rpb) return 0.f;
  const int side = 2 * s.ks - 1;
  const int dy = p.sy + a - p.ci + s.ks - 1;
  const int dx = p.sx + c - p.cj + s.ks - 1;
  return Elem<T>::to_f(rpb[((int64_t)p.h * side + dy) * side + dx]);
}

// ---------------------------------------------------------------------------
// Fused forward, one lane per query, online softmax.
template <typename T>
__global__ __launch_bounds__(256) void fused_fma_kernel(const T *__restrict__ q,
                                                        const T *__restrict__ k,
                                                        const T *__restrict__ v,
                                                        const T *__restrict__ rpb,
                                                        T *__restrict__ out, Shape s,
                                                        Strides si, Strides so, Pad pad,
                                                        float *__restrict__ lse) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= s.n_query) return;
  const QueryPos p = decode_query(t, s, pad.Hp, pad.Wp);
  // keys and values of padded pixels (zeros when no vectors are given)
  float pk[D], pv[D];
  const bool padded = pad.Hp > s.H || pad.Wp > s.W;
  if (padded) {
#pragma unroll
    for (int e = 0; e < D; ++e) pk[e] = pv[e] = 0.f;
    if (pad.k) load_row((const T *)pad.k + (int64_t)p.h * D, pk);
    if (pad.v) load_row((const T *)pad.v + (int64_t)p.h * D, pv);
  }
  const int64_t bb = p.plane / s.heads;
  const int64_t ibase = bb * si.b + p.h * si.h;
  const T *kp = k + ibase;
  const T *vp = v + ibase;
  const float scale = 1.0f / sqrtf((float)D);

  float qr[D];
  load_row(q + ibase + p.i * si.y + p.j * si.x, qr);
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int a = 0; a < s.ks; ++a) {
    const int row = p.ry + (p.sy + a) * s.dil;
    for (int c = 0; c < s.ks; ++c) {
      const int col = p.rx + (p.sx + c) * s.dil;
      const int64_t off = row * si.y + col * si.x;
      const bool real = !padded || (row < s.H && col < s.W);
      float kr[D];
      if (real) {
        load_row(kp + off, kr);
      } else {
#pragma unroll
        for (int e = 0; e < D; ++e) kr[e] = pk[e];
      }
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qr[e], kr[e], dot);
      const float sc = dot * scale + bias_of(rpb, p, s, a, c);
      if (sc > m) {  // new running maximum: rescale what was accumulated
        const float corr = expf(m - sc);
        l *= corr;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] *= corr;
        m = sc;
      }
      const float pr = expf(sc - m);
      l += pr;
      float vr[D];
      if (real) {
        load_row(vp + off, vr);
      } else {
#pragma unroll
        for (int e = 0; e < D; ++e) vr[e] = pv[e];
      }
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pr, vr[e], acc[e]);
    }
  }
  // t is the query's index in dense [B, heads, H, W] order
  if (lse) lse[t] = m + logf(l);
  const float inv = 1.0f / l;
  T *o = out + bb * so.b + p.h * so.h + p.i * so.y + p.j * so.x;
#pragma unroll
  for (int e = 0; e < D; ++e) o[e] = Elem<T>::from_f(acc[e] * inv);
}

// ---------------------------------------------------------------------------
// Unfused step 1: one lane per (query, neighbour slot); slot fastest so the
// fp32 score stores are contiguous.
template <typename T>
__global__ __launch_bounds__(256) void qkrpb_kernel(const T *__restrict__ q,
                                                    const T *__restrict__ k,
                                                    const T *__restrict__ rpb,
                                                    float *__restrict__ attn, Shape s) {
  const int nk = s.ks * s.ks;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= s.n_query * nk) return;
  const int64_t qi = t / nk;
  const int n = (int)(t - qi * nk);
  const int a = n / s.ks, c = n - a * s.ks;
  const QueryPos p = decode_query(qi, s);
  const int64_t hw = (int64_t)s.H * s.W;
  const int row = p.ry + (p.sy + a) * s.dil;
  const int col = p.rx + (p.sx + c) * s.dil;
  const T *kr = k + p.plane * hw * D + ((int64_t)row * s.W + col) * D;
  const T *qr = q + qi * D;
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) dot = fmaf(Elem<T>::to_f(qr[e]), Elem<T>::to_f(kr[e]), dot);
  attn[t] = dot * (1.0f / sqrtf((float)D)) + bias_of(rpb, p, s, a, c);
}

// Unfused step 2: 64 rows per workgroup staged through LDS so that global
// loads and stores are contiguous; one lane finishes one row.
constexpr int kSoftmaxRows = 64;

__global__ __launch_bounds__(kSoftmaxRows) void softmax_kernel(const float *__restrict__ in,
                                                               float *__restrict__ out,
                                                               int64_t rows, int nk) {
  extern __shared__ float buf[];  // kSoftmaxRows * nk
  const int64_t r0 = (int64_t)blockIdx.x * kSoftmaxRows;
  const int nrows = rows - r0 < kSoftmaxRows ? (int)(rows - r0) : kSoftmaxRows;
  const int n = nrows * nk;
  const float *src = in + r0 * nk;
  for (int e = threadIdx.x; e < n; e += kSoftmaxRows) buf[e] = src[e];
  __syncthreads();
  if ((int)threadIdx.x < nrows) {
    float *row = buf + threadIdx.x * nk;  // nk is odd: rows hit distinct banks
    float m = -INFINITY;
    for (int e = 0; e < nk; ++e) m = fmaxf(m, row[e]);
    float sum = 0.f;
    for (int e = 0; e < nk; ++e) {
      const float x = expf(row[e] - m);
      row[e] = x;
      sum += x;
    }
    const float inv = 1.0f / sum;
    for (int e = 0; e < nk; ++e) row[e] *= inv;
  }
  __syncthreads();
  float *dst = out + r0 * nk;
  for (int e = threadIdx.x; e < n; e += kSoftmaxRows) dst[e] = buf[e];
}

// Unfused step 3: one lane per (query, channel); the 32 lanes of a query read
// one contiguous value row per neighbour and share the probability.
template <typename T>
__global__ __launch_bounds__(256) void av_kernel(const float *__restrict__ attn,
                                                 const T *__restrict__ v,
                                                 T *__restrict__ out, Shape s) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= s.n_query * D) return;
  const int64_t qi = t / D;
  const int e = (int)(t - qi * D);
  const QueryPos p = decode_query(qi, s);
  const int64_t hw = (int64_t)s.H * s.W;
  const T *vp = v + p.plane * hw * D + e;
  const float *pr = attn + qi * s.ks * s.ks;
  float acc = 0.f;
  for (int a = 0; a < s.ks; ++a) {
    const int row = p.ry + (p.sy + a) * s.dil;
    for (int c = 0; c < s.ks; ++c) {
      const int col = p.rx + (p.sx + c) * s.dil;
      acc = fmaf(pr[a * s.ks + c], Elem<T>::to_f(vp[((int64_t)row * s.W + col) * D]), acc);
    }
  }
  out[t] = Elem<T>::from_f(acc);
}

// 1-D grid of 256-lane workgroups over `work` items, or false when too large.
bool grid_for(int64_t work, int per_block, dim3 *grid) {
  const int64_t blocks = (work + per_block - 1) / per_block;
  if (blocks > INT32_MAX) return false;
  *grid = dim3((unsigned)blocks);
  return true;
}

}  // namespace

hipError_t launch_fused_fma(const void *q, const void *k, const void *v, const void *rpb,
                            void *out, const Shape &s, const Strides &in, const Strides &out_st,
                            const Pad &pad, na2d_dtype_t dt, hipStream_t st, float *lse) {
  dim3 grid;
  if (!grid_for(s.n_query, 256, &grid)) return hipErrorInvalidConfiguration;
  switch (dt) {
    case NA2D_DTYPE_F32:
      fused_fma_kernel<float><<<grid, 256, 0, st>>>((const float *)q, (const float *)k,
                                                   (const float *)v, (const float *)rpb,
                                                   (float *)out, s, in, out_st, pad, lse);
      break;
    case NA2D_DTYPE_BF16:
      fused_fma_kernel<__bf16><<<grid, 256, 0, st>>>((const __bf16 *)q, (const __bf16 *)k,
                                                    (const __bf16 *)v, (const __bf16 *)rpb,
                                                    (__bf16 *)out, s, in, out_st, pad, lse);
      break;
    case NA2D_DTYPE_F16:
      fused_fma_kernel<_Float16><<<grid, 256, 0, st>>>(
          (const _Float16 *)q, (const _Float16 *)k, (const _Float16 *)v, (const _Float16 *)rpb,
          (_Float16 *)out, s, in, out_st, pad, lse);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_qkrpb(const void *q, const void *k, const void *rpb, float *attn,
                        const Shape &s, na2d_dtype_t dt, hipStream_t st) {
  dim3 grid;
  if (!grid_for(s.n_query * s.ks * s.ks, 256, &grid)) return hipErrorInvalidConfiguration;
  switch (dt) {
    case NA2D_DTYPE_F32:
      qkrpb_kernel<float><<<grid, 256, 0, st>>>((const float *)q, (const float *)k,
                                               (const float *)rpb, attn, s);
      break;
    case NA2D_DTYPE_BF16:
      qkrpb_kernel<__bf16><<<grid, 256, 0, st>>>((const __bf16 *)q, (const __bf16 *)k,
                                                (const __bf16 *)rpb, attn, s);
      break;
    case NA2D_DTYPE_F16:
      qkrpb_kernel<_Float16><<<grid, 256, 0, st>>>((const _Float16 *)q, (const _Float16 *)k,
                                                  (const _Float16 *)rpb, attn, s);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_softmax(const float *in, float *out, const Shape &s, hipStream_t st) {
  dim3 grid;
  if (!grid_for(s.n_query, kSoftmaxRows, &grid)) return hipErrorInvalidConfiguration;
  const int nk = s.ks * s.ks;
  const size_t lds = sizeof(float) * kSoftmaxRows * nk;
  softmax_kernel<<<grid, kSoftmaxRows, lds, st>>>(in, out, s.n_query, nk);
  return hipGetLastError();
}

hipError_t launch_av(const float *attn, const void *v, void *out, const Shape &s,
                     na2d_dtype_t dt, hipStream_t st) {
  dim3 grid;
  if (!grid_for(s.n_query * D, 256, &grid)) return hipErrorInvalidConfiguration;
  switch (dt) {
    case NA2D_DTYPE_F32:
      av_kernel<float><<<grid, 256, 0, st>>>(attn, (const float *)v, (float *)out, s);
      break;
    case NA2D_DTYPE_BF16:
      av_kernel<__bf16><<<grid, 256, 0, st>>>(attn, (const __bf16 *)v, (__bf16 *)out, s);
      break;
    case NA2D_DTYPE_F16:
      av_kernel<_Float16><<<grid, 256, 0, st>>>(attn, (const _Float16 *)v, (_Float16 *)out, s);
      break;
  }
  return hipGetLastError();
}

}  // namespace na2d
