// na2d_dense.hip -- fused forward pass for maps whose residue classes are
// exactly k x k (H == W == k*d, d a power of two): every query attends to its
// whole class.  See the comment on dense_mfma_kernel.
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// ---------------------------------------------------------------------------
// Whole-sub-grid windows: H == k*d and W == k*d (d a power of two).
//
// Then every residue class is exactly k x k and every query's clamped window
// is its entire class, so the operator is dense attention with bias inside
// each class (the NAT README's self-attention equivalence, applied per
// class).  The class is flattened: its N = k*k queries form ceil(N/16)
// tiles and its N keys NKB blocks of 16 (padded with zero pixels, masked
// with -inf).  The accumulator input (bias * sqrt(D), -inf on padding) of a
// (tile, key block) pair is the same for every class of a head, so each wave
// computes it once for the tiles it owns.
//
// A workgroup owns SG consecutive classes of one head, ordered (b, ry, rx)
// with rx fastest, so for d > 1 the classes of one workgroup read whole
// pixel rows.
template <int KS> struct DenseGeometry {
  static constexpr int N = KS * KS;
  static constexpr int NT = (N + 15) / 16;             // query tiles per class
  static constexpr int NKB = ((N + 15) / 16 + 1) & ~1; // key blocks (even)
  static constexpr int NK = NKB * 16;                  // padded keys per class
  static constexpr int SG = 8;                         // classes per workgroup
  static constexpr int NTW = (NT + kWaves - 1) / kWaves;  // tiles per wave
  static constexpr int VSTR = NK + 2;  // V^T channel stride (elements): odd dword count
  static constexpr int SIDE = 2 * KS - 1;
};

template <typename T, int KS>
__global__ __launch_bounds__(kThreads) void dense_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, Shape s, FastDiv fitems, int total,
    int log2d) {
  using G = DenseGeometry<KS>;
  using vec = typename Mma<T>::vec;
  constexpr int N = G::N, NT = G::NT, NKB = G::NKB, NK = G::NK, SG = G::SG, NTW = G::NTW;
  constexpr int VSTR = G::VSTR, SIDE = G::SIDE;
  constexpr int D = kHeadDim;
  constexpr int VCLS = D * VSTR / 2;  // dwords of V^T per class

  __shared__ u32x4 k_lds[SG * NK * 4];         // [class][key][chunk ^ swz]
  __shared__ unsigned int vt_lds[SG * VCLS];   // [class][channel][key pair]
  __shared__ float b_lds[SIDE * SIDE];         // bias * sqrt(D)

  const int tid = threadIdx.x;
  const int dil = s.dil;
  const uint32_t id = xcd_contiguous_id(blockIdx.x, total);
  const int h = fast_div(id, fitems);
  const int per_head = s.B << (2 * log2d);  // classes of one head
  const int c0 = (id - h * fitems.div) * SG;
  const int ncls = min(SG, per_head - c0);
  const int64_t hw = (int64_t)s.H * s.W;

  // class c of this workgroup -> (plane, ry, rx)
  // (dilation is a power of two here, so the decode is shifts and masks)
  auto class_pos = [&](int c, int64_t &plane, int &ry, int &rx) {
    const int j = c0 + c;
    rx = j & (dil - 1);
    ry = (j >> log2d) & (dil - 1);
    plane = (int64_t)(j >> (2 * log2d)) * s.heads + h;
  };

  // ---- stage: all loads first (unconditional, clamped), then LDS writes --
  // A thread owns one (key, 16-byte chunk) slot of a class and visits the
  // workgroup's classes; a load address is a uniform per-class base plus the
  // thread's fixed 32-bit byte offset.
  constexpr int KPC = NK * 4, KCPP = kThreads / KPC;        // K items per class, classes/pass
  constexpr int VPC = (NK / 2) * 4, VCPP = kThreads / VPC;  // V items per class, classes/pass
  static_assert(KCPP * KPC == kThreads && VCPP * VPC == kThreads, "class items must tile 256");
  constexpr int KIT = SG / KCPP, VIT = SG / VCPP;
  const unsigned rowb = (unsigned)dil * (unsigned)s.W * (unsigned)(D * sizeof(T));
  const unsigned colb = (unsigned)dil * (unsigned)(D * sizeof(T));
  // byte offset of pixel (0, 0) of class c (clamped to the workgroup's classes)
  auto cls_off = [&](int c) -> int64_t {
    const int j = c0 + min(c, ncls - 1);
    const int rxx = j & (dil - 1), ryy = (j >> log2d) & (dil - 1);
    const int64_t pl = (int64_t)(j >> (2 * log2d)) * s.heads + h;
    return ((pl * hw + (int64_t)ryy * s.W + rxx) * D) * (int64_t)sizeof(T);
  };
  auto pick = [&](int it, int cpp, int sub) -> int64_t {
    int64_t o = cls_off(it * cpp);
#pragma unroll
    for (int u = 1; u < 4; ++u)
      if (u < cpp && sub == u) o = cls_off(it * cpp + u);
    return o;
  };

  const int ksub = tid / KPC, kkey = (tid % KPC) >> 2, kch = tid & 3;
  const int kkc = min(kkey, N - 1);
  const unsigned koff = (unsigned)(kkc / KS) * rowb + (unsigned)(kkc % KS) * colb + kch * 16;
  u32x4 kreg[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it)
    kreg[it] = *(const u32x4 *)((const char *)k + pick(it, KCPP, ksub) + koff);

  const int vsub = tid / VPC, vpr = (tid % VPC) >> 2, vch = tid & 3;
  const int vk0 = min(2 * vpr, N - 1), vk1 = min(2 * vpr + 1, N - 1);
  const unsigned voff0 = (unsigned)(vk0 / KS) * rowb + (unsigned)(vk0 % KS) * colb + vch * 16;
  const unsigned voff1 = (unsigned)(vk1 / KS) * rowb + (unsigned)(vk1 % KS) * colb + vch * 16;
  u32x4 va[VIT], vb2[VIT];
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const char *base = (const char *)v + pick(it, VCPP, vsub);
    va[it] = *(const u32x4 *)(base + voff0);
    vb2[it] = *(const u32x4 *)(base + voff1);
  }
  for (int e = tid; e < SIDE * SIDE; e += kThreads)
    b_lds[e] = rpb != nullptr ? Elem<T>::to_f(rpb[(int64_t)h * SIDE * SIDE + e]) * kSqrtD : 0.f;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  {
    // padding keys must hold finite values: zeros
    u32x4 *dst = k_lds + (ksub * NK + kkey) * 4 + (kch ^ ((kkey >> 1) & 3));
#pragma unroll
    for (int it = 0; it < KIT; ++it) dst[it * KCPP * NK * 4] = kkey < N ? kreg[it] : zero4;
  }
  {
    unsigned int *dst = vt_lds + vsub * VCLS + (vch * 8) * (VSTR / 2) + vpr;
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const u32x4 a = 2 * vpr < N ? va[it] : zero4, b = 2 * vpr + 1 < N ? vb2[it] : zero4;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dst[it * VCPP * VCLS + (2 * w) * (VSTR / 2)] = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);
        dst[it * VCPP * VCLS + (2 * w + 1) * (VSTR / 2)] =
            __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);
      }
    }
  }
  __syncthreads();

  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const float c2 = kLog2e / kSqrtD;
  const int chA = 8 * (ql >> 2) + (ql & 3);
  vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);

  // accumulator inputs of this wave's tiles
  f32x4 cint[NTW][NKB];
#pragma unroll
  for (int tw = 0; tw < NTW; ++tw) {
    const int nq = min((wave + tw * kWaves) * 16 + ql, N - 1);
    const int qa = nq / KS, qb = nq % KS;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nk = kb * 16 + 4 * g + i;
        const int ka = nk / KS, kc = nk % KS;
        cint[tw][kb][i] = nk < N ? b_lds[(ka - qa + KS - 1) * SIDE + (kc - qb + KS - 1)] : -INFINITY;
      }
  }

  for (int c = 0; c < ncls; ++c) {
    int64_t plane;
    int ry, rx;
    class_pos(c, plane, ry, rx);
    const u32x4 *kc = k_lds + c * NK * 4;
    const unsigned int *vc = vt_lds + c * VCLS;
#pragma unroll
    for (int tw = 0; tw < NTW; ++tw) {
      const int t = wave + tw * kWaves;
      if (t >= NT) break;
      const int nq0 = t * 16 + ql;
      const int nq = min(nq0, N - 1);
      const int64_t qoff =
          (plane * hw + (int64_t)(ry + (nq / KS) * dil) * s.W + rx + (nq % KS) * dil) * D + g * 8;
      const vec qv = __builtin_bit_cast(vec, *(const u32x4 *)(q + qoff));
      f32x4 sc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int key = kb * 16 + ql;
        sc[kb] = Mma<T>::run(__builtin_bit_cast(vec, kc[key * 4 + (g ^ ((key >> 1) & 3))]), qv,
                             cint[tw][kb]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][i]);
      mx = group_max(mx);
      const float mc = mx * c2;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], c2, -mc));
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f}, o2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NKB / 2; ++j) {
        vec pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = static_cast<T>(sc[2 * j][i]);
          pb[4 + i] = static_cast<T>(sc[2 * j + 1][i]);
        }
        // keys 32j + 4g .. +3 and 32j + 16 + 4g .. +3 of channel chA (+4)
        const unsigned int *r = vc + chA * (VSTR / 2) + 16 * j + 2 * g;
        constexpr int C4 = 4 * (VSTR / 2);
        const u32x4 w0 = {r[0], r[1], r[8], r[9]};
        const u32x4 w1 = {r[C4], r[C4 + 1], r[C4 + 8], r[C4 + 9]};
        o0 = Mma<T>::run(__builtin_bit_cast(vec, w0), pb, o0);
        o1 = Mma<T>::run(__builtin_bit_cast(vec, w1), pb, o1);
        o2 = Mma<T>::run(ones, pb, o2);
      }
      if (nq0 < N) {
        const float inv = __builtin_amdgcn_rcpf(o2[0]);
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
}

template <typename T, int KS>
hipError_t launch_dense(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, hipStream_t st) {
  using G = DenseGeometry<KS>;
  const int64_t per_head = (int64_t)s.B * s.dil * s.dil;
  const int64_t items_per_head = (per_head + G::SG - 1) / G::SG;
  const int64_t total = items_per_head * s.heads;
  if (total > INT_MAX || per_head > INT_MAX) return hipErrorInvalidConfiguration;
  int log2d = 0;
  while ((1 << log2d) < s.dil) ++log2d;
  dense_mfma_kernel<T, KS><<<dim3((unsigned)total), kThreads, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (T *)out, s,
      make_fastdiv((uint32_t)items_per_head), (int)total, log2d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_mfma(const void *q, const void *k, const void *v, const void *rpb,
                             void *out, const Shape &s, na2d_dtype_t dt, hipStream_t st,
                             bool *supported) {
  *supported = true;
  const bool pow2_dil = (s.dil & (s.dil - 1)) == 0;
  if ((int64_t)s.ks * s.dil != s.H || (int64_t)s.ks * s.dil != s.W || !pow2_dil ||
      (s.ks != 3 && s.ks != 5 && s.ks != 7) || dt == NA2D_DTYPE_F32) {
    *supported = false;
    return hipSuccess;
  }
  if (dt == NA2D_DTYPE_BF16) {
    switch (s.ks) {
      case 3: return launch_dense<__bf16, 3>(q, k, v, rpb, out, s, st);
      case 5: return launch_dense<__bf16, 5>(q, k, v, rpb, out, s, st);
      default: return launch_dense<__bf16, 7>(q, k, v, rpb, out, s, st);
    }
  }
  switch (s.ks) {
    case 3: return launch_dense<_Float16, 3>(q, k, v, rpb, out, s, st);
    case 5: return launch_dense<_Float16, 5>(q, k, v, rpb, out, s, st);
    default: return launch_dense<_Float16, 7>(q, k, v, rpb, out, s, st);
  }
}

}  // namespace na2d
