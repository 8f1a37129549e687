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
// Unfused path.  Each workgroup owns a run of query pixels of one (batch,
// head) plane: the plane comes from the workgroup id (one fixed-divisor
// division per workgroup), the pixel from the lane, so no lane divides a
// 64-bit index.  Planes must hold fewer than 2^31 pixels.

typedef __attribute__((ext_vector_type(4))) float f32x4v;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2v;

// Workgroup numbering of an unfused launch (kUnfusedQueries queries per
// workgroup, `chunks` workgroups per plane) and the divisors of the pixel
// decoding.
constexpr int kUnfusedQueries = 64;
static_assert(4 * kUnfusedQueries == 256, "four lanes per query in a 256-lane workgroup");

struct UnfusedGrid {
  FastDiv chunks, W, dil, heads;
};

// Sub-grid position and window of in-plane pixel pix (32-bit arithmetic).
struct PixPos {
  int i, j, ry, rx, ci, cj, sy, sx;
};

__device__ __forceinline__ PixPos decode_pixel(int pix, const Shape &s, const UnfusedGrid &g) {
  PixPos p;
  p.i = (int)fast_div((uint32_t)pix, g.W);
  p.j = pix - p.i * s.W;
  p.ci = (int)fast_div((uint32_t)p.i, g.dil);
  p.ry = p.i - p.ci * s.dil;
  p.cj = (int)fast_div((uint32_t)p.j, g.dil);
  p.rx = p.j - p.cj * s.dil;
  const int Ly = (int)fast_div((uint32_t)(s.H - p.ry + s.dil - 1), g.dil);
  const int Lx = (int)fast_div((uint32_t)(s.W - p.rx + s.dil - 1), g.dil);
  p.sy = window_start(p.ci, Ly, s.ks);
  p.sx = window_start(p.cj, Lx, s.ks);
  return p;
}

// Dot product of eight consecutive channels: 16-bit data two channels per
// instruction (fp32 accumulation), fp32 data one fused multiply-add per
// channel.  (The 32-bit words are copied out of their vectors before the bit
// cast: casting a vector element in place was compiled as if every element
// were the first.)
template <typename T> struct Dot8;
template <> struct Dot8<float> {
  f32x4v lo, hi;
  __device__ __forceinline__ void load(const float *p) {
    lo = ((const f32x4v *)p)[0];
    hi = ((const f32x4v *)p)[1];
  }
  __device__ __forceinline__ float dot(const float *k) const {
    const f32x4v a = ((const f32x4v *)k)[0], b = ((const f32x4v *)k)[1];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(lo[i], a[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(hi[i], b[i], acc);
    return acc;
  }
};
template <typename T> struct Dot8Half {
  u32x4v r;
  __device__ __forceinline__ void load(const T *p) { r = *(const u32x4v *)p; }
  __device__ __forceinline__ float dot(const T *k) const {
    const u32x4v kv = *(const u32x4v *)k;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned int qw = r[i], kw = kv[i];
      if constexpr (sizeof(T) == 2 && __is_same(T, __bf16))
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, qw),
                                              __builtin_bit_cast(bf16x2v, kw), acc, false);
      else
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2v, qw), __builtin_bit_cast(f16x2v, kw),
                                     acc, false);
    }
    return acc;
  }
};
template <> struct Dot8<__bf16> : Dot8Half<__bf16> {};
template <> struct Dot8<_Float16> : Dot8Half<_Float16> {};

// Sum over the 4 lanes of a quad (lanes 4m .. 4m+3); every lane gets it.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Eight consecutive channels, widened to fp32 / narrowed with RNE.
template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&f)[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4v a = ((const f32x4v *)p)[0], b = ((const f32x4v *)p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  } else {
    typedef __attribute__((ext_vector_type(8))) T t8;
    const t8 w = *(const t8 *)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(w[i]);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T *p, const float (&f)[8]) {
  if constexpr (sizeof(T) == 4) {
    ((f32x4v *)p)[0] = f32x4v{f[0], f[1], f[2], f[3]};
    ((f32x4v *)p)[1] = f32x4v{f[4], f[5], f[6], f[7]};
  } else {
    typedef __attribute__((ext_vector_type(8))) T t8;
    t8 w;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = static_cast<T>(f[i]);
    *(t8 *)p = w;
  }
}

// The k*k scores of the query at in-plane pixel pix, for lane j of its quad
// (see qkrpb_kernel): lane j writes the scores of window columns c = j
// (mod 4) to out[a*k + c].
template <typename T, int KS>
__device__ __forceinline__ void score_window(const T *__restrict__ q, const T *__restrict__ k,
                                             const T *__restrict__ rpb, const Shape &s,
                                             const UnfusedGrid &g, uint32_t plane, int hw,
                                             int pix, int j, float *out) {
  const PixPos p = decode_pixel(pix, s, g);
  const int h = (int)(plane - fast_div(plane, g.heads) * (uint32_t)s.heads);
  const int64_t pq = (int64_t)plane * hw + pix;  // query index
  Dot8<T> qs;
  qs.load(q + pq * D + 8 * j);
  const T *kp = k + ((int64_t)plane * hw + p.rx + p.sx * s.dil) * D + 8 * j;
  const int64_t step = (int64_t)s.dil * D;
  constexpr int side = 2 * KS - 1;
  const T *br = rpb != nullptr ? rpb + ((int64_t)h * side + (p.sy - p.ci + KS - 1)) * side +
                                     (p.sx - p.cj + KS - 1)
                               : nullptr;
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int a = 0; a < KS; ++a) {
    const T *kr = kp + (int64_t)(p.ry + (p.sy + a) * s.dil) * s.W * D;
    float dot[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) dot[c] = quad_sum(qs.dot(kr + c * step));
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      if ((c & 3) == j) {
        const float bias = br != nullptr ? Elem<T>::to_f(br[a * side + c]) : 0.f;
        out[a * KS + c] = dot[c] * scale + bias;
      }
    }
  }
}

// Unfused step 1 (scores + bias): a quad of lanes per query, lane j of the
// quad owning channels 8j .. 8j+7, so that a load instruction reads whole
// 64-byte key pixels of consecutive queries; the quad sums its partial dot
// products, and lane j puts the scores of window columns c = j (mod 4) into
// LDS, from where the workgroup writes its 64 queries' score rows
// (contiguous in attn) with consecutive lanes on consecutive floats.  KS = k
// (the window loops unroll).
template <typename T, int KS>
__global__ __launch_bounds__(256) void qkrpb_kernel(const T *__restrict__ q,
                                                    const T *__restrict__ k,
                                                    const T *__restrict__ rpb,
                                                    float *__restrict__ attn, Shape s,
                                                    UnfusedGrid g) {
  constexpr int KK = KS * KS, NQ = kUnfusedQueries;
  __shared__ float rows[NQ * KK];
  const int tid = threadIdx.x, j = tid & 3, lq = tid >> 2;
  const uint32_t plane = fast_div(blockIdx.x, g.chunks);
  const int chunk = (int)(blockIdx.x - plane * g.chunks.div);
  const int hw = s.H * s.W;
  const int nq = min(NQ, hw - chunk * NQ);  // queries of this workgroup
  if (lq < nq)  // whole quads take the same branch
    score_window<T, KS>(q, k, rpb, s, g, plane, hw, chunk * NQ + lq, j, rows + lq * KK);
  __syncthreads();
  float *dst = attn + ((int64_t)plane * hw + chunk * NQ) * KK;
  for (int e = tid; e < nq * KK; e += 256) dst[e] = rows[e];
}

// Unfused step 2 (softmax over the last axis): a workgroup of 256 lanes
// stages `rows` rows of k*k scores into LDS with direct global->LDS copies
// (4 bytes per lane, contiguous), one lane finishes one row (odd row lengths
// spread the lanes over distinct banks), and the workgroup writes the rows
// back contiguously.
constexpr int kSoftmaxThreads = 256;

__global__ __launch_bounds__(kSoftmaxThreads) void softmax_kernel(const float *__restrict__ in,
                                                                  float *__restrict__ out,
                                                                  int64_t nrows_total, int nk,
                                                                  int rows) {
  extern __shared__ float buf[];  // rows * nk
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * rows;
  const int nrows = nrows_total - r0 < rows ? (int)(nrows_total - r0) : rows;
  const int n = nrows * nk;
  const float *src = in + r0 * nk;
  // lane l of a copy lands 4 l bytes past the wave's (uniform) LDS address
  const int lane = tid & 63, wbase = __builtin_amdgcn_readfirstlane(tid >> 6) * 64;
  for (int e0 = wbase; e0 < n; e0 += kSoftmaxThreads)
    if (e0 + lane < n)
      __builtin_amdgcn_global_load_lds((const void *)(src + e0 + lane),
                                       (__attribute__((address_space(3))) void *)(buf + e0), 4,
                                       0, 0);
  __syncthreads();  // also completes the copies
  if (tid < nrows) {
    float *row = buf + tid * nk;
    float m = -INFINITY;
    for (int e = 0; e < nk; ++e) m = fmaxf(m, row[e]);
    float sum = 0.f;
    for (int e = 0; e < nk; ++e) {
      const float x = __expf(row[e] - m);
      row[e] = x;
      sum += x;
    }
    const float inv = 1.0f / sum;
    for (int e = 0; e < nk; ++e) row[e] *= inv;
  }
  __syncthreads();
  float *dst = out + r0 * nk;
  for (int e = tid; e < n; e += kSoftmaxThreads) dst[e] = buf[e];
}

// Unfused step 3 (weighted sum of values): four lanes per query, eight
// channels each (16- or 32-byte value reads); 64 queries per workgroup,
// whose probability rows (contiguous in attn) are first copied into LDS with
// direct global->LDS copies.  KS = k: a window row's value loads issue
// together.
template <typename T, int KS>
__global__ __launch_bounds__(256) void av_kernel(const float *__restrict__ attn,
                                                 const T *__restrict__ v,
                                                 T *__restrict__ out, Shape s, UnfusedGrid g) {
  constexpr int KK = KS * KS, NQ = kUnfusedQueries;
  __shared__ float prob[NQ * KK];
  const int tid = threadIdx.x;
  const uint32_t plane = fast_div(blockIdx.x, g.chunks);
  const int chunk = (int)(blockIdx.x - plane * g.chunks.div);
  const int hw = s.H * s.W;
  const int nq = min(NQ, hw - chunk * NQ);  // queries of this workgroup
  {
    // lane l of a copy lands 4 l bytes past the wave's (uniform) LDS address
    const float *src = attn + ((int64_t)plane * hw + chunk * NQ) * KK;
    const int lane = tid & 63, wbase = __builtin_amdgcn_readfirstlane(tid >> 6) * 64;
    for (int e0 = wbase; e0 < nq * KK; e0 += 256)
      if (e0 + lane < nq * KK)
        __builtin_amdgcn_global_load_lds((const void *)(src + e0 + lane),
                                         (__attribute__((address_space(3))) void *)(prob + e0),
                                         4, 0, 0);
  }
  __syncthreads();  // also completes the copies
  const int lq = tid >> 2;
  if (lq >= nq) return;
  const int pix = chunk * NQ + lq;
  const int part = tid & 3;  // channels 8 part .. 8 part + 7
  const PixPos p = decode_pixel(pix, s, g);
  const int64_t pq = (int64_t)plane * hw + pix;
  const float *pr = prob + lq * KK;
  const T *vp = v + ((int64_t)plane * hw + p.rx + p.sx * s.dil) * D + 8 * part;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const int64_t step = (int64_t)s.dil * D;
  for (int a = 0; a < KS; ++a) {
    const int row = p.ry + (p.sy + a) * s.dil;
    const T *vr = vp + (int64_t)row * s.W * D;
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const float w = pr[a * KS + c];
      float f[8];
      load8<T>(vr + c * step, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, f[i], acc[i]);
    }
  }
  store8<T>(out + pq * D + 8 * part, acc);
}

// Launch functors: run<KS>() launches the kernel instantiated for k = KS.
template <typename T> struct QkrpbLaunch {
  template <int KS>
  static void run(dim3 grid, hipStream_t st, const void *q, const void *k, const void *rpb,
                  float *attn, const Shape &s, const UnfusedGrid &g) {
    qkrpb_kernel<T, KS><<<grid, 256, 0, st>>>((const T *)q, (const T *)k, (const T *)rpb, attn,
                                               s, g);
  }
};
template <typename T> struct AvLaunch {
  template <int KS>
  static void run(dim3 grid, hipStream_t st, const float *attn, const void *v, void *out,
                  const Shape &s, const UnfusedGrid &g) {
    av_kernel<T, KS><<<grid, 256, 0, st>>>(attn, (const T *)v, (T *)out, s, g);
  }
};

// Dispatches an odd kernel size 1..13 to its instantiation.
template <typename L, typename... A>
hipError_t launch_ks(int ks, dim3 grid, hipStream_t st, A... args) {
  switch (ks) {
    case 1: L::template run<1>(grid, st, args...); break;
    case 3: L::template run<3>(grid, st, args...); break;
    case 5: L::template run<5>(grid, st, args...); break;
    case 7: L::template run<7>(grid, st, args...); break;
    case 9: L::template run<9>(grid, st, args...); break;
    case 11: L::template run<11>(grid, st, args...); break;
    case 13: L::template run<13>(grid, st, args...); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Workgroups of an unfused launch, or false when
// the plane or the grid is too large for 32-bit workgroup arithmetic.
bool unfused_grid(const Shape &s, UnfusedGrid *g, dim3 *grid) {
  constexpr int per = kUnfusedQueries;
  const int64_t hw = (int64_t)s.H * s.W;
  if (hw >= ((int64_t)1 << 31)) return false;
  const int64_t chunks = (hw + per - 1) / per;
  const int64_t planes = (int64_t)s.B * s.heads;
  if (planes * chunks > INT32_MAX) return false;
  g->chunks = make_fastdiv((uint32_t)chunks);
  g->W = make_fastdiv((uint32_t)s.W);
  g->dil = make_fastdiv((uint32_t)s.dil);
  g->heads = make_fastdiv((uint32_t)s.heads);
  *grid = dim3((unsigned)(planes * chunks));
  return true;
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
  bool mfma = false;
  const hipError_t e = launch_scores_mfma(q, k, rpb, attn, s, dt, st, &mfma);
  if (mfma) return e;
  UnfusedGrid g;
  dim3 grid;
  if (!unfused_grid(s, &g, &grid)) return hipErrorInvalidConfiguration;
  switch (dt) {
    case NA2D_DTYPE_F32: return launch_ks<QkrpbLaunch<float>>(s.ks, grid, st, q, k, rpb, attn, s, g);
    case NA2D_DTYPE_BF16:
      return launch_ks<QkrpbLaunch<__bf16>>(s.ks, grid, st, q, k, rpb, attn, s, g);
    case NA2D_DTYPE_F16:
      return launch_ks<QkrpbLaunch<_Float16>>(s.ks, grid, st, q, k, rpb, attn, s, g);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_softmax(const float *in, float *out, const Shape &s, hipStream_t st) {
  const int nk = s.ks * s.ks;
  // rows per workgroup: as many as 64 KB of LDS holds, 64 to 256
  int rows = kSoftmaxThreads;
  while (rows > 64 && (int64_t)rows * nk * 4 > 64 * 1024) rows /= 2;
  const int64_t blocks = (s.n_query + rows - 1) / rows;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const size_t lds = sizeof(float) * rows * nk;
  softmax_kernel<<<dim3((unsigned)blocks), kSoftmaxThreads, lds, st>>>(in, out, s.n_query, nk,
                                                                       rows);
  return hipGetLastError();
}

hipError_t launch_av(const float *attn, const void *v, void *out, const Shape &s,
                     na2d_dtype_t dt, hipStream_t st) {
  UnfusedGrid g;
  dim3 grid;
  if (!unfused_grid(s, &g, &grid)) return hipErrorInvalidConfiguration;
  switch (dt) {
    case NA2D_DTYPE_F32: return launch_ks<AvLaunch<float>>(s.ks, grid, st, attn, v, out, s, g);
    case NA2D_DTYPE_BF16: return launch_ks<AvLaunch<__bf16>>(s.ks, grid, st, attn, v, out, s, g);
    case NA2D_DTYPE_F16: return launch_ks<AvLaunch<_Float16>>(s.ks, grid, st, attn, v, out, s, g);
  }
  return hipErrorInvalidValue;
}

}  // namespace na2d
