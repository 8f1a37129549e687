// na2d_linear.hip -- the projections around the attention operator:
// y[M, N] = x[M, K] . w[N, K]^T + b[N] (the layout of a Linear layer's
// weight), with x, y channels-last features (one row per pixel).  The NAT /
// DiNAT attention module projects its features to queries, keys and values
// with bias (DiNAT walk-through blog, "What is DiNAT"; the configuration's
// qkv_bias) and closes with an output projection.
//
// Matrix-core kernel (bf16 / fp16, fp32 accumulation): a workgroup computes
// a 128-pixel x TN-feature tile, four waves of 64 pixels x TN/2 features.
// The product is formed transposed, y^T = w . x^T, so that each lane ends up
// with 4 consecutive features of one pixel (one 8-byte store) and the bias
// is the accumulator input.  K advances in chunks of 32: the chunk's w and x
// rows are copied to LDS by the direct global->LDS path (16 bytes per lane,
// chunks XOR-swizzled by row against bank conflicts) into one buffer while
// the other is read.  fp32 data takes a scalar kernel.
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kTM = 128;     // pixels per workgroup tile
constexpr int kKC = 32;      // K per chunk (one MFMA)
constexpr int kThreads = 256;

template <int TN> struct LinGeom {
  static constexpr int WN = TN / 2;          // features per wave
  static constexpr int FB = WN / 16;         // feature blocks per wave
  static constexpr int TB = 64 / 16;         // pixel blocks per wave
  static constexpr int XB = kTM * kKC * 2;   // bytes of a staged x chunk
  static constexpr int WB = TN * kKC * 2;    // bytes of a staged w chunk
};

// Copies rows [r0, r0 + R) (clamped to n - 1) x K-chunk c of a row-major
// [n, K] 16-bit matrix into buf: row r at r * 64 bytes, logical 16-byte chunk
// j at position j ^ ((r >> 1) & 3).  R * 4 slots, 64 per copy instruction.
template <int R>
__device__ __forceinline__ void stage_rows(const char *src, int64_t n, int K, int64_t r0, int c,
                                           char *buf, int wave, int lane) {
  constexpr int NI = R * 4 / 64;
#pragma unroll
  for (int j = 0; j < (NI + 3) / 4; ++j) {
    const int ins = wave + 4 * j;
    if (ins < NI) {
      const int slot = ins * 64 + lane, row = slot >> 2, pos = slot & 3;
      const int lch = pos ^ ((row >> 1) & 3);
      const int64_t rr = min(r0 + row, n - 1);
      const char *p = src + (rr * K + (int64_t)c * kKC + lch * 8) * 2;
      __builtin_amdgcn_global_load_lds((const void *)p, (lds_void *)(buf + ins * 1024), 16, 0, 0);
    }
  }
}

template <typename T, int TN>
__global__ __launch_bounds__(kThreads) void linear_mfma_kernel(const T *__restrict__ x,
                                                               const T *__restrict__ w,
                                                               const T *__restrict__ b,
                                                               T *__restrict__ y, int64_t M,
                                                               int N, int K, int ntn) {
  using G = LinGeom<TN>;
  using vec = typename Mma<T>::vec;
  __shared__ __attribute__((aligned(16))) char xs0[G::XB], ws0[G::WB];
  __shared__ __attribute__((aligned(16))) char xs1[G::XB], ws1[G::WB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int64_t tile = blockIdx.x;
  const int64_t m0 = (tile / ntn) * kTM;
  const int n0 = (int)(tile % ntn) * TN;
  const int wm = wave >> 1, wn = wave & 1;  // this wave: pixels m0 + 64wm.., features n0 + WN wn..
  const int nchunks = K / kKC;

  // accumulators start at the bias of their features
  f32x4 acc[G::TB][G::FB];
#pragma unroll
  for (int fb = 0; fb < G::FB; ++fb) {
    const int f = min(n0 + wn * G::WN + fb * 16 + 4 * g, N - 4);
    f32x4 bias = {0.f, 0.f, 0.f, 0.f};
    if (b != nullptr)
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[i] = Elem<T>::to_f(b[f + i]);
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb) acc[tb][fb] = bias;
  }

  // LDS offsets of this lane's operands within a staged chunk: row r, logical
  // chunk g (the swizzle of row r depends on r only through bits 1-2, which
  // are those of ql)
  const int sw = 16 * (g ^ ((ql >> 1) & 3));
  auto compute = [&](const char *xs, const char *ws) {
    vec a[G::FB], bx[G::TB];
#pragma unroll
    for (int fb = 0; fb < G::FB; ++fb)
      a[fb] = *(const vec *)(ws + (wn * G::WN + fb * 16 + ql) * 64 + sw);
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb)
      bx[tb] = *(const vec *)(xs + (wm * 64 + tb * 16 + ql) * 64 + sw);
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb)
#pragma unroll
      for (int fb = 0; fb < G::FB; ++fb) acc[tb][fb] = Mma<T>::run(a[fb], bx[tb], acc[tb][fb]);
  };
  const char *xc = (const char *)x, *wc = (const char *)w;
  stage_rows<kTM>(xc, M, K, m0, 0, xs0, wave, lane);
  stage_rows<TN>(wc, N, K, n0, 0, ws0, wave, lane);
  __syncthreads();
  for (int c = 0; c < nchunks; c += 2) {
    if (c + 1 < nchunks) {
      stage_rows<kTM>(xc, M, K, m0, c + 1, xs1, wave, lane);
      stage_rows<TN>(wc, N, K, n0, c + 1, ws1, wave, lane);
    }
    compute(xs0, ws0);
    __syncthreads();
    if (c + 1 >= nchunks) break;
    if (c + 2 < nchunks) {
      stage_rows<kTM>(xc, M, K, m0, c + 2, xs0, wave, lane);
      stage_rows<TN>(wc, N, K, n0, c + 2, ws0, wave, lane);
    }
    compute(xs1, ws1);
    __syncthreads();
  }

  // lane (g, ql) holds features f..f+3 of pixel m for each (tb, fb)
  typedef __attribute__((ext_vector_type(4))) T vec4;
#pragma unroll
  for (int tb = 0; tb < G::TB; ++tb) {
    const int64_t m = m0 + wm * 64 + tb * 16 + ql;
    if (m >= M) continue;
#pragma unroll
    for (int fb = 0; fb < G::FB; ++fb) {
      const int f = n0 + wn * G::WN + fb * 16 + 4 * g;
      if (f >= N) continue;
      vec4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = static_cast<T>(acc[tb][fb][i]);
      *(u32x2 *)(y + m * N + f) = __builtin_bit_cast(u32x2, r);
    }
  }
}

// fp32: one lane per (pixel, 4 features), K-loop in fp32 FMA.
__global__ __launch_bounds__(kThreads) void linear_fma_kernel(const float *__restrict__ x,
                                                              const float *__restrict__ w,
                                                              const float *__restrict__ b,
                                                              float *__restrict__ y, int64_t M,
                                                              int N, int K) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int nq = N / 4;
  if (t >= M * nq) return;
  const int64_t m = t / nq;
  const int f = (int)(t % nq) * 4;
  float acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = b != nullptr ? b[f + i] : 0.f;
  const float *xr = x + m * K;
  for (int kk = 0; kk < K; ++kk) {
    const float xv = xr[kk];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(xv, w[(int64_t)(f + i) * K + kk], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) y[m * N + f + i] = acc[i];
}

template <typename T, int TN>
hipError_t launch_mfma(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                       int K, hipStream_t st) {
  const int64_t ntm = (M + kTM - 1) / kTM, ntn = (N + TN - 1) / TN;
  if (ntm * ntn > INT_MAX) return hipErrorInvalidConfiguration;
  linear_mfma_kernel<T, TN><<<dim3((unsigned)(ntm * ntn)), kThreads, 0, st>>>(
      (const T *)x, (const T *)w, (const T *)b, (T *)y, M, N, K, (int)ntn);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_tn(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                     int K, hipStream_t st) {
  // 128-feature tiles when they divide N, else 64 (at most one ragged tile)
  if (N % 128 == 0) return launch_mfma<T, 128>(x, w, b, y, M, N, K, st);
  return launch_mfma<T, 64>(x, w, b, y, M, N, K, st);
}

}  // namespace

bool linear_supported(int N, int K) { return N % 16 == 0 && K % kKC == 0; }

hipError_t launch_linear(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                         int K, na2d_dtype_t dt, hipStream_t st) {
  switch (dt) {
    case NA2D_DTYPE_BF16: return launch_tn<__bf16>(x, w, b, y, M, N, K, st);
    case NA2D_DTYPE_F16: return launch_tn<_Float16>(x, w, b, y, M, N, K, st);
    case NA2D_DTYPE_F32: {
      const int64_t work = M * (N / 4), blocks = (work + kThreads - 1) / kThreads;
      if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
      linear_fma_kernel<<<dim3((unsigned)blocks), kThreads, 0, st>>>(
          (const float *)x, (const float *)w, (const float *)b, (float *)y, M, N, K);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace na2d
