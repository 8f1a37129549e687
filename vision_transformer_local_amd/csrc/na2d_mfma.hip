// na2d_mfma.hip -- fused forward pass of 2D (dilated) Neighborhood Attention
// on the CDNA4 matrix cores (bf16 / fp16 inputs, fp32 accumulation, D = 32).
//
// The operator is the one the DiNAT module composes from natten2dqkrpb,
// softmax(dim=-1) and natten2dav (DiNAT walk-through blog, "What is DiNAT");
// here the three steps run in one kernel and the k*k attention weights of a
// query never leave registers.
//
// Work decomposition
//   * Everything is expressed in residue-class (sub-grid) coordinates: with
//     dilation d, the pixels (ry + d*ci, rx + d*cj) of one class (ry, rx) form
//     an ordinary map on which the operator is plain neighborhood attention.
//   * A workgroup (4 waves) owns an RY x RX block of one class of one
//     (batch, head) plane.  It stages the block's key/value halo -- the union
//     of its queries' clamped windows, at most (RY+k-1) x (RX+k) sub-grid
//     pixels -- in LDS once: K row-major (16-byte chunks swizzled against bank
//     conflicts), V transposed to [channel][pixel] so that the matrix cores can
//     contract over pixels.
//   * A wave processes 16-query tiles (TY x TX sub-grid pixels).  The tile's
//     keys are NB = TY + k - 1 halo rows x 16 columns (the columns start at an
//     even LDS column so V reads are dword aligned).  Scores are produced
//     transposed, S^T = K . Q^T, one v_mfma_f32_16x16x32 per halo row, so that
//     each lane ends up holding scores of ONE query: the softmax reductions
//     need only two cross-lane steps, and the probabilities are already laid
//     out as the B operand of the second product out^T = V^T . P^T.
//   * The relative-position bias (pre-multiplied by sqrt(D)) and the window
//     mask (-inf outside the query's clamped window) enter as the accumulator
//     input of the score MFMA, so they cost no extra pass over the scores.
#include "na2d_internal.h"

#include <limits.h>

namespace na2d {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<_Float16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 run(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Tile geometry per kernel size.  A tile's 16 key columns must cover its
// TX queries' windows plus one column of alignment slack: TX + k <= 16.
template <int KS> struct Geometry {
  static constexpr int TY = KS <= 7 ? 2 : (KS <= 11 ? 4 : 8);  // tile rows
  static constexpr int TX = 16 / TY;                           // tile columns
  static constexpr int RY = KS <= 11 ? 8 : 16;                 // block rows per workgroup
  static constexpr int RX = KS <= 7 ? 32 : (KS <= 11 ? 16 : 8);  // block columns
  static constexpr int NB = TY + KS - 1;                       // key rows per tile (even)
  static constexpr int HRM = RY + KS - 1;                      // staged rows (max)
  static constexpr int HCM = (RX + KS + 1) & ~1;               // staged columns (max, even)
  // V^T channel stride in elements; an odd number of dwords spreads the 16
  // channels one wave reads over distinct banks.
  static constexpr int CSTR = (HRM * HCM) % 4 == 2 ? HRM * HCM : HRM * HCM + 2;
  static constexpr int SIDE = 2 * KS - 1;
  static constexpr int MARGIN = TY * SIDE + 32;  // keeps masked bias reads in bounds
  static_assert(TX + KS <= 16, "key columns do not cover the tile");
  static_assert(NB % 2 == 0, "PV consumes key rows in pairs");
};

constexpr int kThreads = 256;
constexpr float kSqrtD = 5.656854249492380f;  // sqrt(32)

template <typename T, int KS>
__global__ __launch_bounds__(kThreads) void fused_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, Shape s, int nby, int nbx, int total) {
  using G = Geometry<KS>;
  using vec = typename Mma<T>::vec;
  constexpr int TY = G::TY, TX = G::TX, RY = G::RY, RX = G::RX, NB = G::NB;
  constexpr int SIDE = G::SIDE, MARGIN = G::MARGIN, CSTR = G::CSTR;
  constexpr int D = kHeadDim;

  __shared__ u32x4 k_lds[G::HRM * G::HCM * 4];      // [pixel][chunk^swz] 16 B chunks
  __shared__ unsigned int vt_lds[D * CSTR / 2];     // [channel][pixel pair]
  __shared__ float b_lds[SIDE * SIDE + 2 * MARGIN]; // bias * sqrt(D), zero margins

  const int tid = threadIdx.x;
  const int dil = s.dil;
  int id = xcd_contiguous_id(blockIdx.x, total);
  const int rx = id % dil;
  id /= dil;
  const int bx = id % nbx;
  id /= nbx;
  const int by = id % nby;
  id /= nby;
  const int ry = id % dil;
  const int64_t plane = id / dil;
  const int h = (int)(plane % s.heads);

  const int Ly = class_len(s.H, ry, dil), Lx = class_len(s.W, rx, dil);
  const int rc0 = by * RY, cc0 = bx * RX;
  if (rc0 >= Ly || cc0 >= Lx) return;  // this class has fewer rows/columns
  const int rc1 = min(rc0 + RY, Ly), cc1 = min(cc0 + RX, Lx);
  // Halo = union of the block's windows (window starts are monotone).
  const int hy0 = window_start(rc0, Ly, KS), hy1 = window_start(rc1 - 1, Ly, KS) + KS;
  const int hx0 = window_start(cc0, Lx, KS), hx1 = window_start(cc1 - 1, Lx, KS) + KS;
  const int hx0e = hx0 & ~1;  // even LDS column origin
  const int HR = hy1 - hy0, HC = (hx1 - hx0e + 1) & ~1;

  const int64_t hw = (int64_t)s.H * s.W;
  const T *kp = k + plane * hw * D;
  const T *vp = v + plane * hw * D;

  // ---- stage bias, K and V^T -------------------------------------------
  for (int e = tid; e < SIDE * SIDE + 2 * MARGIN; e += kThreads) {
    const int t = e - MARGIN;
    float b = 0.f;
    if (rpb != nullptr && t >= 0 && t < SIDE * SIDE)
      b = Elem<T>::to_f(rpb[(int64_t)h * SIDE * SIDE + t]) * kSqrtD;
    b_lds[e] = b;
  }
  const int nkeys = HR * HC;
  for (int e = tid; e < nkeys * 4; e += kThreads) {
    const int key = e >> 2, ch = e & 3;
    const int row = key / HC, col = key - row * HC;
    const int gy = ry + (hy0 + row) * dil;
    const int gx = rx + min(hx0e + col, Lx - 1) * dil;
    k_lds[key * 4 + (ch ^ ((key >> 1) & 3))] =
        *(const u32x4 *)(kp + ((int64_t)gy * s.W + gx) * D + ch * 8);
  }
  for (int e = tid; e < nkeys * 2; e += kThreads) {  // (nkeys/2 pairs) x 4 chunks
    const int pr = e >> 2, ch = e & 3;
    const int key0 = pr * 2;
    const int row = key0 / HC, col = key0 - row * HC;
    const int64_t rowoff = (int64_t)(ry + (hy0 + row) * dil) * s.W;
    const int gx0 = rx + min(hx0e + col, Lx - 1) * dil;
    const int gx1 = rx + min(hx0e + col + 1, Lx - 1) * dil;
    const u32x4 a = *(const u32x4 *)(vp + (rowoff + gx0) * D + ch * 8);
    const u32x4 b = *(const u32x4 *)(vp + (rowoff + gx1) * D + ch * 8);
    unsigned int *dst = vt_lds + (ch * 8) * (CSTR / 2) + (key0 >> 1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // dword w of a chunk = channels 2w, 2w+1
      dst[(2 * w) * (CSTR / 2)] = (a[w] & 0xffffu) | (b[w] << 16);
      dst[(2 * w + 1) * (CSTR / 2)] = (a[w] >> 16) | (b[w] & 0xffff0000u);
    }
  }
  __syncthreads();

  // ---- 16-query tiles ----------------------------------------------------
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15, g = lane >> 4;
  const int nty = (rc1 - rc0 + TY - 1) / TY, ntx = (cc1 - cc0 + TX - 1) / TX;
  const float c2 = kLog2e / kSqrtD;  // exp(S - Smax) = exp2((acc - accmax) * c2)
  const int chA = 8 * (ql >> 2) + (ql & 3);  // V^T row of this lane (+4 for block 1)

  for (int tile = wave; tile < nty * ntx; tile += kThreads / 64) {
    const int ty = tile / ntx, tx = tile - ty * ntx;
    const int tci0 = rc0 + ty * TY, tcj0 = cc0 + tx * TX;
    int ci = tci0 + ql / TX, cj = tcj0 + ql % TX;
    const bool valid = ci < rc1 && cj < cc1;
    ci = min(ci, rc1 - 1);  // ragged tile: recompute a real query, store nothing
    cj = min(cj, cc1 - 1);
    const int sy = window_start(ci, Ly, KS), sx = window_start(cj, Lx, KS);
    const int Y0 = window_start(tci0, Ly, KS), X0 = window_start(tcj0, Lx, KS);
    const int X0a = X0 - ((X0 - hx0e) & 1);  // even LDS column
    const int lrow0 = Y0 - hy0, lcol0 = X0a - hx0e;

    const int64_t qoff =
        plane * hw * D + ((int64_t)(ry + ci * dil) * s.W + rx + cj * dil) * D + g * 8;
    const vec qv = __builtin_bit_cast(vec, *(const u32x4 *)(q + qoff));

    // S^T rows: key (Y0 + a, X0a + 4g + i) against query ql, i = 0..3.
    const int rowrel = Y0 - sy, colrel = X0a + 4 * g - sx;
    const int bbase = MARGIN + (Y0 - ci + KS - 1) * SIDE + (X0a + 4 * g - cj + KS - 1);
    f32x4 sc[NB];
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const bool rok = (unsigned)(rowrel + a) < (unsigned)KS;
      f32x4 cinit;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rok && (unsigned)(colrel + i) < (unsigned)KS;
        const float b = b_lds[bbase + a * SIDE + i];
        cinit[i] = ok ? b : -INFINITY;
      }
      const int lr = min(lrow0 + a, HR - 1), lc = min(lcol0 + ql, HC - 1);
      const int key = lr * HC + lc;
      const vec kv = __builtin_bit_cast(vec, k_lds[key * 4 + (g ^ ((key >> 1) & 3))]);
      sc[a] = Mma<T>::run(kv, qv, cinit);
    }

    // softmax over the query's k*k keys: 4 lane groups hold disjoint keys
    float mx = -INFINITY;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[a][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mc = mx * c2;
    float l = 0.f;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[a][i], c2, -mc));
        sc[a][i] = p;
        l += p;
      }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);

    // out^T = V^T . P^T over pairs of key rows (32 keys per MFMA)
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    const int colA = lcol0 + 4 * g;
    const int c01 = min(colA, HC - 2), c23 = min(colA + 2, HC - 2);
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) {
      vec pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<T>(sc[2 * j][i]);
        pb[4 + i] = static_cast<T>(sc[2 * j + 1][i]);
      }
      const int r0 = min(lrow0 + 2 * j, HR - 1), r1 = min(lrow0 + 2 * j + 1, HR - 1);
      const int k00 = (r0 * HC + c01) >> 1, k01 = (r0 * HC + c23) >> 1;
      const int k10 = (r1 * HC + c01) >> 1, k11 = (r1 * HC + c23) >> 1;
      const unsigned int *v0 = vt_lds + chA * (CSTR / 2);
      const unsigned int *v1 = vt_lds + (chA + 4) * (CSTR / 2);
      const u32x4 w0 = {v0[k00], v0[k01], v0[k10], v0[k11]};
      const u32x4 w1 = {v1[k00], v1[k01], v1[k10], v1[k11]};
      o0 = Mma<T>::run(__builtin_bit_cast(vec, w0), pb, o0);
      o1 = Mma<T>::run(__builtin_bit_cast(vec, w1), pb, o1);
    }

    // lane holds channels 8g..8g+3 (o0) and 8g+4..8g+7 (o1) of query ql
    if (valid) {
      const float inv = 1.0f / l;
      vec res;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        res[i] = static_cast<T>(o0[i] * inv);
        res[4 + i] = static_cast<T>(o1[i] * inv);
      }
      *(u32x4 *)(out + qoff) = __builtin_bit_cast(u32x4, res);
    }
  }
}

template <typename T, int KS>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *rpb, void *out,
                    const Shape &s, hipStream_t st) {
  using G = Geometry<KS>;
  const int Lymax = class_len(s.H, 0, s.dil), Lxmax = class_len(s.W, 0, s.dil);
  const int nby = (Lymax + G::RY - 1) / G::RY, nbx = (Lxmax + G::RX - 1) / G::RX;
  const int64_t total = (int64_t)s.B * s.heads * s.dil * s.dil * nby * nbx;
  if (total > INT_MAX) return hipErrorInvalidConfiguration;
  fused_mfma_kernel<T, KS><<<dim3((unsigned)total), kThreads, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (T *)out, s, nby, nbx,
      (int)total);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, hipStream_t st, bool *supported) {
  switch (s.ks) {
    case 1: return launch_t<T, 1>(q, k, v, rpb, out, s, st);
    case 3: return launch_t<T, 3>(q, k, v, rpb, out, s, st);
    case 5: return launch_t<T, 5>(q, k, v, rpb, out, s, st);
    case 7: return launch_t<T, 7>(q, k, v, rpb, out, s, st);
    case 9: return launch_t<T, 9>(q, k, v, rpb, out, s, st);
    case 11: return launch_t<T, 11>(q, k, v, rpb, out, s, st);
    case 13: return launch_t<T, 13>(q, k, v, rpb, out, s, st);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_fused_mfma(const void *q, const void *k, const void *v, const void *rpb,
                             void *out, const Shape &s, na2d_dtype_t dt, hipStream_t st,
                             bool *supported) {
  *supported = true;
  if (dt == NA2D_DTYPE_BF16) return launch_dtype<__bf16>(q, k, v, rpb, out, s, st, supported);
  if (dt == NA2D_DTYPE_F16) return launch_dtype<_Float16>(q, k, v, rpb, out, s, st, supported);
  *supported = false;
  return hipSuccess;
}

}  // namespace na2d
