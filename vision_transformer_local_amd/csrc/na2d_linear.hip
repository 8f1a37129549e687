// na2d_linear.hip -- the projections around the attention operator:
// y[M, N] = x[M, K] . w[N, K]^T + b[N] (the layout of a Linear layer's
// weight), with x, y channels-last features (one row per pixel).  The NAT /
// DiNAT attention module projects its features to queries, keys and values
// with bias (DiNAT walk-through blog, "What is DiNAT"; the configuration's
// qkv_bias) and closes with an output projection.
//
// Matrix-core kernel (bf16 / fp16, fp32 accumulation): a workgroup computes
// a 128-pixel x TN-feature tile (TN = N up to 192 features, so that x is read
// once), four waves of 64 pixels x TN/2 features.
// The product is formed transposed, y^T = w . x^T, so that each lane ends up
// with 4 consecutive features of one pixel (one 8-byte store) and the bias
// is the accumulator input.  K advances in chunks of 32: each lane loads its
// 16-byte pieces of the chunk's w and x rows into registers two chunks ahead
// of the one being multiplied and writes them to one of two LDS buffers
// (16-byte pieces XOR-swizzled by row against bank conflicts) while the other
// is read, so that a long K loop (few tiles, wide K) is not one memory
// latency per chunk.  fp32 data takes a scalar kernel.
//
// Output layouts: y[M, N] row-major, or -- for the block's q|k|v projection,
// N = 3C, C = heads*D -- head-planar: feature n = t*C + h*D + e of pixel
// m = b*HW + p goes to ((t*B + b)*heads + h)*HW*D + p*D + e, i.e. three dense
// [B, heads, H, W, D] tensors, which the attention kernels then read without
// cache lines shared between heads.
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kTMax = 128;   // largest pixel tile (row slices are multiples of it)
constexpr int kKC = 32;      // K per chunk (one MFMA)
constexpr int kThreads = 256;
constexpr int64_t kSmallGrid = 4 * 256;  // tiles below which 64-pixel tiles are used

// A TM-pixel x TN-feature tile: the four waves split it TM/64 ways along the
// pixels and 4 / (TM/64) ways along the features, 64 pixels x WN features each.
template <int TM, int TN> struct LinGeom {
  static constexpr int WMW = TM / 64, WNW = 4 / WMW;  // waves along pixels, features
  static constexpr int WN = TN / WNW;        // features per wave
  static constexpr int FB = WN / 16;         // feature blocks per wave
  static constexpr int TB = 64 / 16;         // pixel blocks per wave
  static constexpr int XB = TM * kKC * 2;    // bytes of a staged x chunk
  static constexpr int WB = TN * kKC * 2;    // bytes of a staged w chunk
  static_assert((TM == 64 || TM == 128) && WN % 16 == 0, "tile shape");
};

// A chunk's x and w pieces held by one lane between its load and its LDS write.
template <int TM, int TN> struct ChunkRegs {
  u32x4 x[TM / 64], w[TN / 64];
};

// Rows [r0, r0 + R) (clamped to n - 1) x K-chunk c of a row-major [n, K]
// 16-bit matrix, as staged in LDS: row r at r * 64 bytes, logical 16-byte
// piece j at position j ^ ((r >> 1) & 3).  The R * 4 pieces are numbered by
// their LDS position (slot = 4 r + position); the 256 lanes take slots
// 256 j + tid, R / 64 each.  A lane's byte offsets of its pieces in chunk 0
// are fixed for the whole K loop (the matrix spans less than 2^31 bytes);
// chunk c adds the uniform c * 64 bytes, so that a load costs no vector
// arithmetic.
template <int R>
__device__ __forceinline__ void row_offsets(int64_t n, int K, int64_t r0, int tid,
                                            uint32_t *off) {
  static_assert(R % 64 == 0, "pieces must split evenly over the workgroup");
#pragma unroll
  for (int j = 0; j < R / 64; ++j) {
    const int slot = j * kThreads + tid, row = slot >> 2, pos = slot & 3;
    const int lch = pos ^ ((row >> 1) & 3);
    const int64_t rr = min(r0 + row, n - 1);
    off[j] = (uint32_t)((rr * K + lch * 8) * 2);
  }
}

template <int R>
__device__ __forceinline__ void load_rows(const char *src, int c, const uint32_t *off, u32x4 *v) {
#pragma unroll
  for (int j = 0; j < R / 64; ++j)
    v[j] = *(const u32x4 *)((src + c * (kKC * 2)) + off[j]);
}

template <int R>
__device__ __forceinline__ void write_rows(char *buf, int tid, const u32x4 *v) {
#pragma unroll
  for (int j = 0; j < R / 64; ++j) *(u32x4 *)(buf + (j * kThreads + tid) * 16) = v[j];
}

// Workgroups go to the eight XCDs round-robin by id, each XCD with its own
// L2.  Tile indices are handed out so that every XCD takes one contiguous
// range of them: the feature tiles of a pixel tile, which read the same x
// rows, then mostly share an L2.  A bijection on [0, n).
__device__ __forceinline__ uint32_t xcd_tile(uint32_t id, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, xcd = id % 8;
  return xcd * q + min(xcd, r) + id / 8;
}

// Head-planar output: pixels per image (HW), C, head dim (D), images, heads.
struct PlanarOut {
  FastDiv hw, c, d;
  int B, heads;
};

// Element offset of feature f (a multiple of 4, so f..f+3 stay in one head)
// within the head-planar output, without the pixel's part.
__device__ __forceinline__ int64_t planar_feature(uint32_t f, const PlanarOut &po) {
  const uint32_t t = fast_div(f, po.c), r = f - t * po.c.div;
  const uint32_t h = fast_div(r, po.d), e = r - h * po.d.div;
  return ((int64_t)t * po.B * po.heads + h) * ((int64_t)po.hw.div * po.d.div) + e;
}

// Element offset of pixel m = b*HW + p within the head-planar output.
__device__ __forceinline__ int64_t planar_pixel(uint32_t m, const PlanarOut &po) {
  const uint32_t bb = fast_div(m, po.hw), p = m - bb * po.hw.div;
  return ((int64_t)bb * po.heads * po.hw.div + p) * po.d.div;
}

// x, M: a slice of rows (under 2^31 bytes); y: the slice's rows for
// row-major output, the whole output for head-planar output, whose pixel
// index adds mbase.
template <typename T, int TM, int TN, bool PLANAR>
__global__ __launch_bounds__(kThreads) void linear_mfma_kernel(const T *__restrict__ x,
                                                               const T *__restrict__ w,
                                                               const T *__restrict__ b,
                                                               T *__restrict__ y, int64_t M,
                                                               int N, int K, int ntn,
                                                               PlanarOut po, int64_t mbase) {
  using G = LinGeom<TM, TN>;
  using vec = typename Mma<T>::vec;
  __shared__ __attribute__((aligned(16))) char xs0[G::XB], ws0[G::WB];
  __shared__ __attribute__((aligned(16))) char xs1[G::XB], ws1[G::WB];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t m0 = (tile / ntn) * TM;
  const int n0 = (int)(tile % ntn) * TN;
  // this wave: pixels m0 + 64wm.., features n0 + WN wn..
  const int wm = wave / G::WNW, wn = wave % G::WNW;
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
  ChunkRegs<TM, TN> r0, r1;  // chunks c + 1 and c + 2 (alternately) in flight
  uint32_t xoff[TM / 64], woff[TN / 64];
  row_offsets<TM>(M, K, m0, tid, xoff);
  row_offsets<TN>(N, K, n0, tid, woff);
  auto load = [&](int c, ChunkRegs<TM, TN> &r) {
    load_rows<TM>(xc, c, xoff, r.x);
    load_rows<TN>(wc, c, woff, r.w);
  };
  auto write = [&](const ChunkRegs<TM, TN> &r, char *xs, char *ws) {
    write_rows<TM>(xs, tid, r.x);
    write_rows<TN>(ws, tid, r.w);
  };
  // chunk c sits in LDS buffer c % 2 and, before that, in registers r(c % 2);
  // the barrier closing step c ends every wave's reads of buffer c % 2 and
  // publishes chunk c + 1's writes.  The steady-state loop has no branch
  // inside (chunks c + 1 and c + 3 exist), which keeps the compiler's waits
  // for the loads exact; the last steps follow it.
  auto step = [&](int c, const char *xs, const char *ws, char *xn, char *wn2,
                  ChunkRegs<TM, TN> &rn) {
    compute(xs, ws);
    if (c + 1 < nchunks) write(rn, xn, wn2);
    if (c + 3 < nchunks) load(c + 3, rn);
    __syncthreads();
  };
  load(0, r0);
  if (nchunks > 1) load(1, r1);
  write(r0, xs0, ws0);
  if (nchunks > 2) load(2, r0);
  __syncthreads();
  int c = 0;
  for (; c + 4 < nchunks; c += 2) {
    compute(xs0, ws0);
    write(r1, xs1, ws1);
    load(c + 3, r1);
    __syncthreads();
    compute(xs1, ws1);
    write(r0, xs0, ws0);
    load(c + 4, r0);
    __syncthreads();
  }
  // at most four chunks remain, the first in buffer 0
  if (c < nchunks) step(c, xs0, ws0, xs1, ws1, r1);
  if (c + 1 < nchunks) step(c + 1, xs1, ws1, xs0, ws0, r0);
  if (c + 2 < nchunks) step(c + 2, xs0, ws0, xs1, ws1, r1);
  if (c + 3 < nchunks) step(c + 3, xs1, ws1, xs0, ws0, r0);

  // lane (g, ql) holds features f..f+3 of pixel m for each (tb, fb)
  typedef __attribute__((ext_vector_type(4))) T vec4;
  int64_t fofs[G::FB];  // planar: the features' part of the output offset
  if constexpr (PLANAR) {
#pragma unroll
    for (int fb = 0; fb < G::FB; ++fb)
      fofs[fb] = planar_feature((uint32_t)min(n0 + wn * G::WN + fb * 16 + 4 * g, N - 4), po);
  }
#pragma unroll
  for (int tb = 0; tb < G::TB; ++tb) {
    const int64_t m = m0 + wm * 64 + tb * 16 + ql;
    if (m >= M) continue;
    const int64_t mofs = PLANAR ? planar_pixel((uint32_t)(mbase + m), po) : 0;
#pragma unroll
    for (int fb = 0; fb < G::FB; ++fb) {
      const int f = n0 + wn * G::WN + fb * 16 + 4 * g;
      if (f >= N) continue;
      vec4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = static_cast<T>(acc[tb][fb][i]);
      T *dst = PLANAR ? y + fofs[fb] + mofs : y + m * N + f;
      *(u32x2 *)dst = __builtin_bit_cast(u32x2, r);
    }
  }
}

// fp32: one lane per (pixel, 4 features), K-loop in fp32 FMA.
template <bool PLANAR>
__global__ __launch_bounds__(kThreads) void linear_fma_kernel(const float *__restrict__ x,
                                                              const float *__restrict__ w,
                                                              const float *__restrict__ b,
                                                              float *__restrict__ y, int64_t M,
                                                              int N, int K, PlanarOut po) {
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
  float *dst = PLANAR ? y + planar_pixel((uint32_t)m, po) + planar_feature((uint32_t)f, po)
                      : y + m * N + f;
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = acc[i];
}

hipError_t launch_fma(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                      int K, const PlanarOut *po, hipStream_t st) {
  const int64_t work = M * (N / 4), blocks = (work + kThreads - 1) / kThreads;
  if (blocks > INT_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (po != nullptr)
    linear_fma_kernel<true><<<grid, kThreads, 0, st>>>((const float *)x, (const float *)w,
                                                       (const float *)b, (float *)y, M, N, K,
                                                       *po);
  else
    linear_fma_kernel<false><<<grid, kThreads, 0, st>>>((const float *)x, (const float *)w,
                                                        (const float *)b, (float *)y, M, N, K,
                                                        PlanarOut{});
  return hipGetLastError();
}

// Launches over slices of at most 2^31 bytes of x (a multiple of the tile
// rows), so that the kernel's per-lane offsets fit 32 bits.
template <typename T, int TM, int TN>
hipError_t launch_mfma_tm(const void *x, const void *w, const void *b, void *y, int64_t M,
                          int N, int K, const PlanarOut *po, hipStream_t st) {
  const int64_t row_bytes = (int64_t)K * sizeof(T);
  const int64_t slice = ((int64_t(1) << 31) / row_bytes) / kTMax * kTMax;
  if (slice < kTMax) return hipErrorInvalidValue;  // excluded by linear_supported
  for (int64_t mb = 0; mb < M; mb += slice) {
    const int64_t ms = M - mb < slice ? M - mb : slice;
    const int64_t ntm = (ms + TM - 1) / TM, ntn = (N + TN - 1) / TN;
    if (ntm * ntn > INT_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(ntm * ntn));
    const T *xs = (const T *)x + mb * K;
    if (po != nullptr)
      linear_mfma_kernel<T, TM, TN, true><<<grid, kThreads, 0, st>>>(
          xs, (const T *)w, (const T *)b, (T *)y, ms, N, K, (int)ntn, *po, mb);
    else
      linear_mfma_kernel<T, TM, TN, false><<<grid, kThreads, 0, st>>>(
          xs, (const T *)w, (const T *)b, (T *)y + mb * N, ms, N, K, (int)ntn, PlanarOut{}, 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// 64-pixel tiles when 128-pixel ones would not give every compute unit
// several workgroups and K is short (at most 256: a few chunks per tile, so
// that more workgroups in flight pay off; with longer K the doubled weight
// reads of the smaller tiles measured slower), 128 otherwise.
template <typename T, int TN>
hipError_t launch_mfma(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                       int K, const PlanarOut *po, hipStream_t st) {
  const int64_t tiles128 = (M + 127) / 128 * ((N + TN - 1) / TN);
  if (tiles128 < kSmallGrid && K <= 256)
    return launch_mfma_tm<T, 64, TN>(x, w, b, y, M, N, K, po, st);
  return launch_mfma_tm<T, 128, TN>(x, w, b, y, M, N, K, po, st);
}

template <typename T>
hipError_t launch_tn(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                     int K, const PlanarOut *po, hipStream_t st) {
  // N <= 192: one tile across all features (N rounded up to a multiple of
  // 64), so that x is read once; wider N: 128-feature tiles when they divide
  // N, else 64 (one ragged tile at most).  Wider tiles need more registers
  // than two waves per SIMD allow, which costs more than the x re-reads
  // (mostly L2 hits: the feature tiles of a pixel tile share an XCD).
  const int tn = N <= 192 ? (N + 63) / 64 * 64 : N % 128 == 0 ? 128 : 64;
  switch (tn) {
    case 192: return launch_mfma<T, 192>(x, w, b, y, M, N, K, po, st);
    case 128: return launch_mfma<T, 128>(x, w, b, y, M, N, K, po, st);
    default: return launch_mfma<T, 64>(x, w, b, y, M, N, K, po, st);
  }
}

}  // namespace

// N % 16: whole 16-feature output blocks; K % 32: whole chunks; the weight
// (and a 128-row slice of x) spans less than 2^31 bytes.
bool linear_supported(int N, int K) {
  return N % 16 == 0 && K % kKC == 0 && (int64_t)N * K * 2 < (int64_t(1) << 31) &&
         (int64_t)kTMax * K * 2 < (int64_t(1) << 31);
}

hipError_t launch_linear(const void *x, const void *w, const void *b, void *y, int64_t M, int N,
                         int K, na2d_dtype_t dt, hipStream_t st) {
  switch (dt) {
    case NA2D_DTYPE_BF16: return launch_tn<__bf16>(x, w, b, y, M, N, K, nullptr, st);
    case NA2D_DTYPE_F16: return launch_tn<_Float16>(x, w, b, y, M, N, K, nullptr, st);
    case NA2D_DTYPE_F32: return launch_fma(x, w, b, y, M, N, K, nullptr, st);
  }
  return hipErrorInvalidValue;
}

bool linear_planar_supported(int64_t pixels, int C, int heads) {
  // pixel and feature indices in 32 bits; 4-feature groups within one head
  return pixels < (int64_t(1) << 31) && C % heads == 0 && (C / heads) % 4 == 0 &&
         linear_supported(3 * C, C);
}

hipError_t launch_linear_qkv_planar(const void *x, const void *w, const void *b, void *y, int B,
                                    int HW, int C, int heads, na2d_dtype_t dt, hipStream_t st) {
  const PlanarOut po{make_fastdiv((uint32_t)HW), make_fastdiv((uint32_t)C),
                     make_fastdiv((uint32_t)(C / heads)), B, heads};
  const int64_t M = (int64_t)B * HW;
  switch (dt) {
    case NA2D_DTYPE_BF16: return launch_tn<__bf16>(x, w, b, y, M, 3 * C, C, &po, st);
    case NA2D_DTYPE_F16: return launch_tn<_Float16>(x, w, b, y, M, 3 * C, C, &po, st);
    case NA2D_DTYPE_F32: return launch_fma(x, w, b, y, M, 3 * C, C, &po, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace na2d
