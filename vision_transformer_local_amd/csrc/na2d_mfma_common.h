// na2d_mfma_common.h -- matrix-core helpers shared by the fused kernels of
// libna2d (gfx950: v_mfma_f32_16x16x32_{bf16,f16}, v_permlane{16,32}_swap).
#pragma once

#include "na2d_internal.h"

namespace na2d {
namespace mfma {

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

constexpr float kSqrtD = 5.656854249492380f;  // sqrt(32)

// Byte strides of a q/k/v (or out) view [B, heads, H, W, D]: batch and head
// as 64-bit offsets, pixel row and column as 32-bit offsets within one
// (batch, head) plane.
struct ByteStrides {
  int64_t b, h;
  uint32_t y, x;
};

// Byte strides, or false when a (batch, head) plane's span does not fit the
// kernels' 32-bit in-plane offsets, a row or column stride does not fit the
// 24-bit multiplies that form them (16 MB; every realistic map), or a stride
// is negative.
inline bool byte_strides(const Strides &t, const Shape &s, int64_t elem, ByteStrides *out) {
  if (t.b < 0 || t.h < 0 || t.y < 0 || t.x < 0) return false;
  const int64_t span = ((int64_t)(s.H - 1) * t.y + (int64_t)(s.W - 1) * t.x + kHeadDim) * elem;
  if (span > (int64_t(1) << 31)) return false;
  if (t.y * elem >= (int64_t(1) << 24) || t.x * elem >= (int64_t(1) << 24)) return false;
  *out = ByteStrides{t.b * elem, t.h * elem, (uint32_t)(t.y * elem), (uint32_t)(t.x * elem)};
  return true;
}

// Maximum over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the 4 lane groups (lanes l, l^16, l^32, l^48); every lane of a
// group gets the same value.
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr float kLn2 = 0.6931471805599453f;

// Natural log-sum-exp of a query's window scores z = acc / sqrt(D) from the
// softmax's reference mc = max(acc) * log2(e) / sqrt(D) and the sum l of
// exp2(acc * log2(e) / sqrt(D) - mc) over the window (l >= 1: the maximum
// contributes 1): ln sum exp(z) = (mc + log2 l) * ln 2.
__device__ __forceinline__ float window_lse(float mc, float l) {
  return (mc + __builtin_amdgcn_logf(l)) * kLn2;
}

}  // namespace mfma
}  // namespace na2d
