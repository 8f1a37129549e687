// na2d_backward_mfma.hip -- backward pass of 2D (dilated) Neighborhood
// Attention on the CDNA4 matrix cores (bf16 / fp16 inputs, fp32
// accumulation, D = 32, k = 3..13).
//
// Gradients of sum(out * dout) through the DiNAT module's natten2dqkrpb ->
// softmax -> natten2dav chain (DiNAT walk-through blog, "What is DiNAT"),
// with z = q.k / sqrt(D) + bias, P = softmax(z) over the query's clamped
// k x k window:
//   dP = dout . v,  Dq = sum_n P dP,  dS = P (dP - Dq),
//   dq = sum_n dS k / sqrt(D),  dk = sum_i dS q / sqrt(D),  dv = sum_i P dout,
//   drpb[offset(i, n)] += dS.
//
// Work decomposition (residue-class coordinates throughout, as in the
// forward kernel): blocks of RY x RX pixels of one class of one plane, one
// wave per 16-pixel tile (TY x TX), one block per workgroup.
//   * Query kernel (bwd_query_mfma): per query tile, the K/V halo of the
//     block is in LDS.  Scores S^T = K . Q^T and dP^T = V . dout^T are one
//     v_mfma_f32_16x16x32 per key row each (the bias and window mask enter
//     as the accumulator input); softmax, Dq and dS stay in registers; dq^T
//     = K^T . dS^T reads K transposed (ds_read_b64_tr_b16).  dS is split
//     into a 16-bit head and a 16-bit remainder, two products each, so the
//     gradient carries no 16-bit rounding of dS.  Writes dq, the
//     log-sum-exp and Dq of every query, and this block's bias-gradient
//     table.
//   * Key kernel (bwd_key_mfma): per key tile, the Q/dout halo of the block
//     -- every query whose clamped window reaches the block's keys, with its
//     log-sum-exp and Dq -- is in LDS.  S = Q . K^T and dP = dout . V^T are
//     formed for two query rows at a time (the roles of the forward kernel
//     with queries and keys exchanged), P and dS are recomputed, and
//     dv^T = dout^T . P, dk^T = Q^T . dS accumulate (again head + remainder).
//     Near the borders the set of queries reaching a key is larger than
//     the k x k interior one; the tile loops over exactly its rows and
//     16-column chunks.
//   * The bias gradient: each wave adds its tile's dS into its own LDS table
//     with one 16-lane group at a time (its lanes hold distinct queries, so
//     no two lanes of one add meet at an entry holding a nonzero term), the
//     block sums its waves' tables in wave order, and a last kernel sums the
//     blocks of each head in a fixed tree.  The pass is deterministic.
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Query rows [inv_lo, inv_hi] whose clamped windows hold key row y of a class
// of length L (window starts are non-decreasing in steps of at most one).
__host__ __device__ constexpr int inv_lo(int y, int ks) { return y - ks + 1 <= 0 ? 0 : y - ks / 2; }
__host__ __device__ constexpr int inv_hi(int y, int L, int ks) {
  return y >= L - ks ? L - 1 : (y + ks / 2 < L - 1 ? y + ks / 2 : L - 1);
}

// Longest query interval [inv_lo(y0), inv_hi(y1)] over runs y0..y1 of n key
// rows starting at multiples of n, over every class length L >= ks (the
// border effects of the two ends separate well before the bound on L).
constexpr int max_inv_span(int ks, int n) {
  int best = 0;
  for (int L = ks; L <= 4 * (n + 2 * ks); ++L)
    for (int y0 = 0; y0 < L; y0 += n) {
      const int y1 = (y0 + n < L ? y0 + n : L) - 1;
      const int span = inv_hi(y1, L, ks) - inv_lo(y0, ks) + 1;
      best = span > best ? span : best;
    }
  return best;
}

template <int KS> struct BG {
  static constexpr int TY = KS <= 9 ? 2 : 4, TX = 16 / TY;  // tile: TY x TX pixels
  static constexpr int RY = 16, RX = 8;                       // block: RY x RX pixels
  static constexpr int NTX = RX / TX, WAVES = (RY / TY) * NTX, THREADS = 64 * WAVES;
  static constexpr int NB = TY + KS - 1;  // key rows reached by a query tile
  static constexpr int SIDE = 2 * KS - 1, NT = SIDE * SIDE;
  // query kernel: K/V halo of a query block (a tile reads 16 columns from its
  // first window column)
  static constexpr int HR = RY + KS - 1;
  static constexpr int HC = (RX - TX + 16) > (RX + KS - 1) ? (RX - TX + 16) : (RX + KS - 1);
  // key kernel: Q/dout halo of a key block, plus one row for the second row
  // of a tile's last (odd) pair
  static constexpr int QR = max_inv_span(KS, RY) + 1, QC = max_inv_span(KS, RX);
};

constexpr float kInvSqrtD = 0.17677669529663687f;  // 1 / sqrt(32)

// Sum over the 4 lane groups (lanes l, l^16, l^32, l^48); every lane of a
// group gets the same value.
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// One block of the decomposition: plane, class and first pixel (sub-grid).
struct Block {
  int64_t plane;
  int h, ry, rx, Ly, Lx, y0, x0;
  bool ok;  // false when the class is too short to reach this block
};

__device__ __forceinline__ Block block_at(int id, const Shape &s, int nby, int nbx, int RY,
                                          int RX) {
  Block b;
  const int bx = id % nbx;
  id /= nbx;
  const int by = id % nby;
  id /= nby;
  b.rx = id % s.dil;
  id /= s.dil;
  b.ry = id % s.dil;
  b.plane = id / s.dil;
  b.h = (int)(b.plane % s.heads);
  b.Ly = class_len(s.H, b.ry, s.dil);
  b.Lx = class_len(s.W, b.rx, s.dil);
  b.y0 = by * RY;
  b.x0 = bx * RX;
  b.ok = b.y0 < b.Ly && b.x0 < b.Lx;
  return b;
}

// In-plane pixel index of class pixel (row, col).
__device__ __forceinline__ unsigned pixel_of(const Shape &s, const Block &b, int row, int col) {
  return (unsigned)(b.ry + row * s.dil) * (unsigned)s.W + (unsigned)(b.rx + col * s.dil);
}

// Copies the class pixels rows [r0, r1] x cols [c0, c1] (clamped beyond:
// rows/columns past r1/c1 repeat the last one, so every LDS pixel is finite
// real data) into buf as [ROWS][COLS] 64-byte pixels, 16-byte chunks
// XOR-swizzled by (column >> 1) & 3, with the direct global->LDS path.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ void stage_halo(const T *__restrict__ src, const Shape &s,
                                           const Block &b, int r0, int r1, int c0, int c1,
                                           char *buf, int wave, int lane, int nwaves) {
  constexpr int NI = (ROWS * COLS * 4 + 63) / 64;  // 64-lane copies (16 B per lane)
  const char *base = (const char *)(src + b.plane * (int64_t)s.H * s.W * kHeadDim);
  for (int ins = wave; ins < NI; ins += nwaves) {
    const int slot = ins * 64 + lane;
    const int pix = slot >> 2, pch = slot & 3;
    const int row = pix / COLS, col = pix - row * COLS;
    if (pix < ROWS * COLS) {
      const int lch = pch ^ ((col >> 1) & 3);
      const unsigned p = pixel_of(s, b, min(r0 + row, r1), min(c0 + col, c1));
      __builtin_amdgcn_global_load_lds(
          (const void *)(base + (size_t)p * (kHeadDim * sizeof(T)) + lch * 16),
          (lds_void *)(buf + ins * 1024), 16, 0, 0);
    }
  }
}

// 16-byte operand of pixel (row, col) of a staged halo: channels 8g..8g+7.
template <typename T, int COLS>
__device__ __forceinline__ typename Mma<T>::vec halo_vec(const char *buf, int row, int col, int g) {
  const u32x4 *p = (const u32x4 *)(buf + (row * COLS + col) * 64 + 16 * (g ^ ((col >> 1) & 3)));
  return __builtin_bit_cast(typename Mma<T>::vec, *p);
}

// Transposed operand (16 channels x 32 pixels) of pixel rows r0, r0+1 of a
// staged halo: lane (g, l) supplies 4 channels of column tc (= first column
// + 4g + l/4); cb selects channels 0..15 or 16..31.
template <typename T, int COLS>
__device__ __forceinline__ typename Mma<T>::vec halo_tr(const char *buf, int r0, int tc, int ql,
                                                       int cb) {
  const int qd = ql & 3, vs = (tc >> 1) & 3;
  const char *p = buf + tc * 64 + 8 * (qd & 1) + 16 * (((qd >> 1) | (2 * cb)) ^ vs);
  const u32x2 a = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + r0 * COLS * 64)));
  const u32x2 c = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + (r0 + 1) * COLS * 64)));
  return __builtin_bit_cast(typename Mma<T>::vec, u32x4{a[0], a[1], c[0], c[1]});
}

// 16-bit B operand (rows 2j, 2j+1 of a tile) split into a rounded head and
// the rounded remainder: hi + lo equals x to about 16 significant bits.  The
// fp32 values are pinned first: otherwise the compiler may fold the product
// that made them into mixed-precision FMAs for one of the two roundings
// only (fp16), and hi + lo then misses x by a 16-bit ulp.
template <typename T>
__device__ __forceinline__ void split_operand(f32x4 s0, f32x4 s1, typename Mma<T>::vec &hi,
                                              typename Mma<T>::vec &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    asm volatile("" : "+v"(s0[i]), "+v"(s1[i]));
    const T h0 = static_cast<T>(s0[i]), h1 = static_cast<T>(s1[i]);
    hi[i] = h0;
    hi[4 + i] = h1;
    lo[i] = static_cast<T>(s0[i] - static_cast<float>(h0));
    lo[4 + i] = static_cast<T>(s1[i] - static_cast<float>(h1));
  }
}

// acc (+)= A . (hi + lo)
template <typename T>
__device__ __forceinline__ f32x4 mma2(typename Mma<T>::vec a, typename Mma<T>::vec hi,
                                      typename Mma<T>::vec lo, f32x4 acc) {
  acc = Mma<T>::run(a, hi, acc);
  return Mma<T>::run(a, lo, acc);
}

// Writes channels 4g..4g+3 (o0) and 16+4g..16+4g+3 (o1), times scale, of
// the pixel whose data starts at dst.
template <typename T>
__device__ __forceinline__ void store_channels(T *dst, int g, const f32x4 &o0, const f32x4 &o1,
                                               float scale) {
  typedef __attribute__((ext_vector_type(4))) T vec4;
  vec4 r0, r1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r0[i] = static_cast<T>(o0[i] * scale);
    r1[i] = static_cast<T>(o1[i] * scale);
  }
  *(u32x2 *)(dst + 4 * g) = __builtin_bit_cast(u32x2, r0);
  *(u32x2 *)(dst + 16 + 4 * g) = __builtin_bit_cast(u32x2, r1);
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::vec load_operand(const T *pixel, int g) {
  return __builtin_bit_cast(typename Mma<T>::vec, *(const u32x4 *)(pixel + 8 * g));
}

// Bias table of head h, times sqrt(D) (accumulator units of the score MFMA).
template <typename T, int NT>
__device__ __forceinline__ void load_bias(const T *__restrict__ rpb, int h, float *tab, int tid,
                                          int nthreads) {
  for (int e = tid; e < NT; e += nthreads)
    tab[e] = rpb != nullptr ? Elem<T>::to_f(rpb[(int64_t)h * NT + e]) * kSqrtD : 0.f;
}

// ---------------------------------------------------------------------------
// Query kernel.
template <typename T, int KS>
__global__ __launch_bounds__(BG<KS>::THREADS) void bwd_query_mfma(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, const T *__restrict__ dout, T *__restrict__ dq,
    float *__restrict__ lse, float *__restrict__ dqdot, float *__restrict__ bias_part, Shape s,
    int nby, int nbx) {
  using G = BG<KS>;
  constexpr int NB = G::NB, SIDE = G::SIDE, NT = G::NT, HC = G::HC;
  constexpr int HALO = G::HR * HC * 64;  // bytes per staged tensor
  // K then V halo; afterwards the waves' parking space for dS (bias gradient)
  __shared__ __attribute__((aligned(16))) char halo[2 * HALO];
  __shared__ float btab[NT];
  __shared__ float dtab[G::WAVES][NT];
  constexpr int PARK = G::TX * KS * 16;  // floats per wave: [query column][window row][16]
  static_assert(G::WAVES * PARK * 4 <= 2 * HALO, "dS parking exceeds the halo buffers");
  char *const kbuf = halo, *const vbuf = halo + HALO;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const Block b = block_at(id, s, nby, nbx, G::RY, G::RX);
  const bool bias = bias_part != nullptr;
  if (!b.ok) {
    if (bias)
      for (int e = tid; e < NT; e += G::THREADS) bias_part[(int64_t)id * NT + e] = 0.f;
    return;
  }
  const int Ly = b.Ly, Lx = b.Lx;
  const int y1 = min(b.y0 + G::RY, Ly) - 1, x1 = min(b.x0 + G::RX, Lx) - 1;
  const int hy0 = window_start(b.y0, Ly, KS), hy1 = window_start(y1, Ly, KS) + KS - 1;
  const int hx0 = window_start(b.x0, Lx, KS), hx1 = window_start(x1, Lx, KS) + KS - 1;
  stage_halo<T, G::HR, HC>(k, s, b, hy0, hy1, hx0, hx1, kbuf, wave, lane, G::WAVES);
  stage_halo<T, G::HR, HC>(v, s, b, hy0, hy1, hx0, hx1, vbuf, wave, lane, G::WAVES);
  load_bias<T, NT>(rpb, b.h, btab, tid, G::THREADS);
  if (bias)
    for (int e = lane; e < NT; e += 64) dtab[wave][e] = 0.f;
  __syncthreads();  // also completes the LDS copies

  const int64_t pofs = b.plane * (int64_t)s.H * s.W * kHeadDim;
  const int tci0 = b.y0 + (wave / G::NTX) * G::TY, tcj0 = b.x0 + (wave % G::NTX) * G::TX;
  const bool tile_ok = tci0 < Ly && tcj0 < Lx;
  const int qy = ql / G::TX, qx = ql % G::TX;
  const int ci = min(tci0 + qy, Ly - 1), cj = min(tcj0 + qx, Lx - 1);
  const int Y0 = window_start(min(tci0, Ly - 1), Ly, KS), X0 = window_start(min(tcj0, Lx - 1), Lx, KS);
  const int sy = window_start(ci, Ly, KS), sx = window_start(cj, Lx, KS);
  f32x4 dp[NB];  // dP, then dS
  if (tile_ok) {
    const bool qok = tci0 + qy < Ly && tcj0 + qx < Lx;
    const unsigned qpix = pixel_of(s, b, ci, cj);
    const typename Mma<T>::vec qv = load_operand(q + pofs + (size_t)qpix * kHeadDim, g);
    const typename Mma<T>::vec gv = load_operand(dout + pofs + (size_t)qpix * kHeadDim, g);
    const int lr0 = Y0 - hy0, lc0 = X0 - hx0;
    float capx[4];
    int colp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int xx = X0 + 4 * g + i;
      capx[i] = (unsigned)(xx - sx) < (unsigned)KS ? INFINITY : -INFINITY;
      colp[i] = clampi(xx - cj + KS - 1, 0, SIDE - 1);
    }
    f32x4 sc[NB];
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int yy = Y0 + a;
      const float capy = (unsigned)(yy - sy) < (unsigned)KS ? INFINITY : -INFINITY;
      const int rowp = clampi(yy - ci + KS - 1, 0, SIDE - 1) * SIDE;
      f32x4 cin;
#pragma unroll
      for (int i = 0; i < 4; ++i) cin[i] = fminf(fminf(btab[rowp + colp[i]], capx[i]), capy);
      sc[a] = Mma<T>::run(halo_vec<T, HC>(kbuf, lr0 + a, lc0 + ql, g), qv, cin);
      dp[a] = Mma<T>::run(halo_vec<T, HC>(vbuf, lr0 + a, lc0 + ql, g), gv, zero);
    }
    // softmax over the window (masked entries are -inf), in log2 units of z
    const float c2 = kLog2e * kInvSqrtD;
    float mx = -INFINITY;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[a][i]);
    mx = group_max(mx);
    const float mc = mx * c2;
    float l = 0.f;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[a][i] = __builtin_amdgcn_exp2f(fmaf(sc[a][i], c2, -mc));
        l += sc[a][i];
      }
    l = group_sum(l);
    const float inv = 1.0f / l;
    float dqd = 0.f;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[a][i] *= inv;
        dqd = fmaf(sc[a][i], dp[a][i], dqd);
      }
    dqd = group_sum(dqd);
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[a][i] = sc[a][i] * (dp[a][i] - dqd);  // dS
    // dq^T = K^T . dS^T over pairs of key rows
    f32x4 o0 = zero, o1 = zero;
    const int tc = lc0 + 4 * g + (ql >> 2);
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) {
      typename Mma<T>::vec hi, lo;
      split_operand<T>(dp[2 * j], dp[2 * j + 1], hi, lo);
      o0 = mma2<T>(halo_tr<T, HC>(kbuf, lr0 + 2 * j, tc, ql, 0), hi, lo, o0);
      o1 = mma2<T>(halo_tr<T, HC>(kbuf, lr0 + 2 * j, tc, ql, 1), hi, lo, o1);
    }
    if (qok) {
      store_channels<T>(dq + pofs + (size_t)qpix * kHeadDim, g, o0, o1, kInvSqrtD);
      if (g == 0) {
        const int64_t qi = pofs / kHeadDim + qpix;
        lse[qi] = mc + log2f(l);
        dqdot[qi] = dqd;
      }
    }
  }
  if (!bias) return;
  // Bias gradient of the tile.  Once every wave is done with the K/V halo,
  // each wave parks its dS rows in its own slice of that LDS, one query row
  // of the tile at a time ([query column][window row][16 halo columns]), and
  // lane l sums window slot l over that row's queries, in column order, into
  // the wave's table (plain read-add-write: the lanes' entries are distinct).
  __syncthreads();
  if (tile_ok) {
    float *park = (float *)halo + wave * PARK;
    float *wt = dtab[wave];
    for (int h = 0; h < G::TY; ++h) {
      const int qi = tci0 + h;
      if (qi >= Ly) break;
      if (qy == h) {
#pragma unroll
        for (int a = 0; a < NB; ++a) {
          const int wa = a + Y0 - sy;
          if ((unsigned)wa < (unsigned)KS) *(f32x4 *)(park + (qx * KS + wa) * 16 + 4 * g) = dp[a];
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int syq = window_start(qi, Ly, KS);
      for (int s0 = 0; s0 < KS * KS; s0 += 64) {
        const int slot = s0 + lane;
        if (slot < KS * KS) {
          const int wa = slot / KS, wc = slot - wa * KS;
          const int erow = (wa + syq - qi + KS - 1) * SIDE;
          float run = 0.f;
          int re = -1;  // table entry the running sum belongs to
          for (int x = 0; x < G::TX; ++x) {
            const int qj = tcj0 + x;
            if (qj >= Lx) break;
            const int sxq = window_start(qj, Lx, KS);
            const float val = park[(x * KS + wa) * 16 + wc + sxq - X0];
            const int e = erow + wc + sxq - qj + KS - 1;
            if (e != re) {
              if (re >= 0) wt[re] += run;
              run = val;
              re = e;
            } else {
              run += val;
            }
          }
          if (re >= 0) wt[re] += run;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  for (int e = tid; e < NT; e += G::THREADS) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < G::WAVES; ++w) t += dtab[w][e];
    bias_part[(int64_t)id * NT + e] = t;
  }
}

// ---------------------------------------------------------------------------
// Key kernel.
template <typename T, int KS>
__global__ __launch_bounds__(BG<KS>::THREADS) void bwd_key_mfma(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, const T *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ dqdot, T *__restrict__ dk, T *__restrict__ dv, Shape s, int nby,
    int nbx) {
  using G = BG<KS>;
  constexpr int SIDE = G::SIDE, NT = G::NT, QR = G::QR, QC = G::QC;
  __shared__ __attribute__((aligned(16))) char qbuf[QR * QC * 64], gbuf[QR * QC * 64];
  __shared__ f32x2 lbuf[QR * QC];  // (log-sum-exp, Dq) of the halo queries
  __shared__ float btab[NT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const Block b = block_at(id, s, nby, nbx, G::RY, G::RX);
  if (!b.ok) return;
  const int Ly = b.Ly, Lx = b.Lx;
  const int y1 = min(b.y0 + G::RY, Ly) - 1, x1 = min(b.x0 + G::RX, Lx) - 1;
  const int hq0 = inv_lo(b.y0, KS), hq1 = inv_hi(y1, Ly, KS);
  const int hc0 = inv_lo(b.x0, KS), hc1 = inv_hi(x1, Lx, KS);
  stage_halo<T, QR, QC>(q, s, b, hq0, hq1, hc0, hc1, qbuf, wave, lane, G::WAVES);
  stage_halo<T, QR, QC>(dout, s, b, hq0, hq1, hc0, hc1, gbuf, wave, lane, G::WAVES);
  const int64_t pofs = b.plane * (int64_t)s.H * s.W * kHeadDim;
  const int64_t qbase = pofs / kHeadDim;
  for (int p = tid; p < QR * QC; p += G::THREADS) {
    const int row = p / QC, col = p - row * QC;
    const int64_t qi = qbase + pixel_of(s, b, min(hq0 + row, hq1), min(hc0 + col, hc1));
    lbuf[p] = f32x2{lse[qi], dqdot[qi]};
  }
  load_bias<T, NT>(rpb, b.h, btab, tid, G::THREADS);
  __syncthreads();  // also completes the LDS copies

  const int t0 = b.y0 + (wave / G::NTX) * G::TY, tx0 = b.x0 + (wave % G::NTX) * G::TX;
  if (t0 >= Ly || tx0 >= Lx) return;
  const int kyl = t0 + ql / G::TX, kxl = tx0 + ql % G::TX;
  const bool kok = kyl < Ly && kxl < Lx;
  const int ky = min(kyl, Ly - 1), kx = min(kxl, Lx - 1);
  const unsigned kpix = pixel_of(s, b, ky, kx);
  const typename Mma<T>::vec kv = load_operand(k + pofs + (size_t)kpix * kHeadDim, g);
  const typename Mma<T>::vec vv = load_operand(v + pofs + (size_t)kpix * kHeadDim, g);
  const int rlo = inv_lo(t0, KS), rhi = inv_hi(min(t0 + G::TY, Ly) - 1, Ly, KS);
  const int clo = inv_lo(tx0, KS), chi = inv_hi(min(tx0 + G::TX, Lx) - 1, Lx, KS);
  const float c2 = kLog2e * kInvSqrtD;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 k0 = zero, k1 = zero, v0 = zero, v1 = zero;
  for (int c0 = clo; c0 <= chi; c0 += 16) {
    // this lane's 4 query columns c0 + 4g + i: window test, bias column and
    // LDS column (clamped: columns past the halo are masked)
    float capx[4];
    int colp[4], lcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qc = c0 + 4 * g + i;
      const bool in = qc < Lx && (unsigned)(kx - window_start(min(qc, Lx - 1), Lx, KS)) < (unsigned)KS;
      capx[i] = in ? INFINITY : -INFINITY;
      colp[i] = clampi(kx - qc + KS - 1, 0, SIDE - 1);
      lcol[i] = min(qc - hc0, QC - 1);
    }
    const int acol = min(c0 + ql - hc0, QC - 1);
    const int tc = min(c0 + 4 * g + (ql >> 2) - hc0, QC - 1);
    for (int r = rlo; r <= rhi; r += 2) {
      f32x4 P[2], dS[2];
      const int lrow0 = r - hq0;  // r + 1 - hq0 <= QR - 1: the staged rows cover the pair
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qr = r + u, lrow = lrow0 + u;
        const int syq = window_start(min(qr, Ly - 1), Ly, KS);
        const float capy = qr < Ly && (unsigned)(ky - syq) < (unsigned)KS ? INFINITY : -INFINITY;
        const int rowp = clampi(ky - qr + KS - 1, 0, SIDE - 1) * SIDE;
        f32x4 cin;
#pragma unroll
        for (int i = 0; i < 4; ++i) cin[i] = fminf(fminf(btab[rowp + colp[i]], capx[i]), capy);
        const f32x4 sv = Mma<T>::run(halo_vec<T, QC>(qbuf, lrow, acol, g), kv, cin);
        const f32x4 dpv = Mma<T>::run(halo_vec<T, QC>(gbuf, lrow, acol, g), vv, zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2 ld = lbuf[lrow * QC + lcol[i]];
          P[u][i] = __builtin_amdgcn_exp2f(fmaf(sv[i], c2, -ld[0]));
          dS[u][i] = P[u][i] * (dpv[i] - ld[1]);
        }
      }
      typename Mma<T>::vec phi, plo, shi, slo;
      split_operand<T>(P[0], P[1], phi, plo);
      split_operand<T>(dS[0], dS[1], shi, slo);
      v0 = mma2<T>(halo_tr<T, QC>(gbuf, lrow0, tc, ql, 0), phi, plo, v0);
      v1 = mma2<T>(halo_tr<T, QC>(gbuf, lrow0, tc, ql, 1), phi, plo, v1);
      k0 = mma2<T>(halo_tr<T, QC>(qbuf, lrow0, tc, ql, 0), shi, slo, k0);
      k1 = mma2<T>(halo_tr<T, QC>(qbuf, lrow0, tc, ql, 1), shi, slo, k1);
    }
  }
  if (kok) {
    store_channels<T>(dk + pofs + (size_t)kpix * kHeadDim, g, k0, k1, kInvSqrtD);
    store_channels<T>(dv + pofs + (size_t)kpix * kHeadDim, g, v0, v1, 1.0f);
  }
}

// drpb[h][e] = sum over the blocks of head h's planes of their tables: each
// thread a fixed strided subset, then a fixed tree.
constexpr int kSumThreads = 256;
__global__ __launch_bounds__(kSumThreads) void bwd_bias_sum(const float *__restrict__ part,
                                                           float *__restrict__ drpb, int B,
                                                           int heads, int bpp, int nt) {
  __shared__ float red[kSumThreads];
  const int e = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int n = B * bpp;
  float acc = 0.f;
  for (int j = t; j < n; j += kSumThreads) {
    const int bb = j / bpp, blk = j - bb * bpp;
    acc += part[(((int64_t)bb * heads + h) * bpp + blk) * nt + e];
  }
  red[t] = acc;
  __syncthreads();
#pragma unroll
  for (int w = kSumThreads / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) drpb[h * nt + e] = red[0];
}

struct Grid {
  int nby, nbx;
  int64_t bpp, nblocks;
};

template <int KS>
Grid grid_of(const Shape &s) {
  using G = BG<KS>;
  Grid r;
  r.nby = (class_len(s.H, 0, s.dil) + G::RY - 1) / G::RY;
  r.nbx = (class_len(s.W, 0, s.dil) + G::RX - 1) / G::RX;
  r.bpp = (int64_t)s.dil * s.dil * r.nby * r.nbx;
  r.nblocks = (int64_t)s.B * s.heads * r.bpp;
  return r;
}

template <typename T, int KS>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *rpb,
                    const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                    const Shape &s, hipStream_t st) {
  using G = BG<KS>;
  const Grid gr = grid_of<KS>(s);
  if (gr.nblocks > INT_MAX) return hipErrorInvalidConfiguration;
  float *lse = (float *)ws;
  float *dqdot = lse + s.n_query;
  float *part = drpb != nullptr ? dqdot + s.n_query : nullptr;
  bwd_query_mfma<T, KS><<<dim3((unsigned)gr.nblocks), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (const T *)dout, (T *)dq, lse,
      dqdot, part, s, gr.nby, gr.nbx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_key_mfma<T, KS><<<dim3((unsigned)gr.nblocks), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (const T *)dout, lse, dqdot,
      (T *)dk, (T *)dv, s, gr.nby, gr.nbx);
  e = hipGetLastError();
  if (e != hipSuccess || drpb == nullptr) return e;
  bwd_bias_sum<<<dim3(G::NT, s.heads), kSumThreads, 0, st>>>(part, drpb, s.B, s.heads,
                                                             (int)gr.bpp, G::NT);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const void *q, const void *k, const void *v, const void *rpb,
                        const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                        const Shape &s, hipStream_t st) {
  switch (s.ks) {
    case 3: return launch_t<T, 3>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 5: return launch_t<T, 5>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 7: return launch_t<T, 7>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 9: return launch_t<T, 9>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 11: return launch_t<T, 11>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
    case 13: return launch_t<T, 13>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
  }
  return hipErrorInvalidValue;
}

template <int KS>
int64_t blocks_of(const Shape &s) {
  return grid_of<KS>(s).nblocks;
}

}  // namespace

bool backward_mfma_supported(const Shape &s, na2d_dtype_t dt) {
  return (dt == NA2D_DTYPE_BF16 || dt == NA2D_DTYPE_F16) && s.ks >= 3 && s.ks <= kMaxKernel &&
         (int64_t)s.H * s.W < kMaxPlanePixels;
}

size_t backward_mfma_workspace_bytes(const Shape &s, bool with_bias) {
  size_t n = (size_t)s.n_query * 2 * sizeof(float);
  if (!with_bias) return n;
  int64_t nb = 0;
  switch (s.ks) {
    case 3: nb = blocks_of<3>(s); break;
    case 5: nb = blocks_of<5>(s); break;
    case 7: nb = blocks_of<7>(s); break;
    case 9: nb = blocks_of<9>(s); break;
    case 11: nb = blocks_of<11>(s); break;
    case 13: nb = blocks_of<13>(s); break;
    default: return n;
  }
  const size_t side = 2 * s.ks - 1;
  return n + (size_t)nb * side * side * sizeof(float);
}

hipError_t launch_backward_mfma(const void *q, const void *k, const void *v, const void *rpb,
                                const void *dout, void *dq, void *dk, void *dv, float *drpb,
                                void *ws, const Shape &s, na2d_dtype_t dt, hipStream_t st) {
  if (dt == NA2D_DTYPE_BF16)
    return launch_dtype<__bf16>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
  if (dt == NA2D_DTYPE_F16)
    return launch_dtype<_Float16>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
  return hipErrorInvalidValue;
}

}  // namespace na2d
