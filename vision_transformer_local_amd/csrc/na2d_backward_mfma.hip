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
//   * The bias gradient: after the tile's products, each wave parks its dS
//     rows (by query, in window coordinates) in the freed halo LDS and every
//     lane sums one window slot over the tile's queries in a fixed order into
//     the wave's own table (distinct lanes, distinct entries: no atomics);
//     the block sums its waves' tables in wave order, and a last kernel sums
//     the blocks of each head in a fixed tree.  The pass is deterministic.
//   * Each wave's Q/dout (query kernel) or K/V (key kernel) operands are
//     loaded while the block's halo copy is in flight.
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

// Block height: 16 rows, or 8 when the residue classes are at most 8 rows
// long (large dilations), so that no wave of a block idles.
template <int KS, int RYV = 16> struct BG {
  static constexpr int TY = KS <= 9 ? 2 : 4, TX = 16 / TY;  // tile: TY x TX pixels
  static constexpr int RY = RYV, RX = 8;                      // block: RY x RX pixels
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
  // Bias tables (times sqrt(D)) laid out so that a lane reads its entries at
  // one base plus immediate offsets, margins included (no clamping):
  //   query kernel, interior tiles: [a - qy + TY-1][c - qx + TX-1] with the
  //     window mask baked in (-inf outside); edge tiles: [key - query row +
  //     k-1 + TY-1][key - query column + k-1 + TX-1], zero margins;
  //   key kernel: the same two kinds indexed by query - key (+ k-1 and the
  //     margins TY-1, TX-1).
  static constexpr int IH = NB + TY - 1, IW = 16 + TX - 1;
  static constexpr int EH = NB + KS + TY - 2, EW = TX + KS + 14;
  static constexpr int FH = 2 * TY + 2 * KS - 2, FW = 2 * TX + 2 * KS + 12;
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

// Divisors of the block numbering, fixed per launch.
struct BlockDivs {
  FastDiv nbx, nby, dil, heads;
};

__device__ __forceinline__ Block block_at(int id, const Shape &s, const BlockDivs &dv, int RY,
                                          int RX) {
  Block b;
  uint32_t u = (uint32_t)id, t = fast_div(u, dv.nbx);
  const int bx = (int)(u - t * dv.nbx.div);
  u = t;
  t = fast_div(u, dv.nby);
  const int by = (int)(u - t * dv.nby.div);
  u = t;
  t = fast_div(u, dv.dil);
  b.rx = (int)(u - t * dv.dil.div);
  u = t;
  t = fast_div(u, dv.dil);
  b.ry = (int)(u - t * dv.dil.div);
  b.plane = t;
  b.h = (int)(t - fast_div(t, dv.heads) * dv.heads.div);
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

// x, made opaque to the optimiser where it is defined.  Values that are later
// split by split_operand go through this: otherwise the compiler may fold the
// product that made x into mixed-precision FMAs for one of the two roundings
// only (fp16), and hi + lo then misses x by a 16-bit ulp.  Pinning at the
// definition (rather than inside the split) costs no copies when x stays live.
__device__ __forceinline__ float pinned(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// 16-bit B operand (rows 2j, 2j+1 of a tile) split into a rounded head and
// the rounded remainder: hi + lo equals x to about 16 significant bits.  Two
// values at a time: one packed conversion gives both heads, whose fp32 values
// come back exactly from the packed bits, and one packed conversion the two
// remainders.  The inputs must come from pinned().
template <typename T>
__device__ __forceinline__ void split_operand(f32x4 s0, f32x4 s1, typename Mma<T>::vec &hi,
                                              typename Mma<T>::vec &lo) {
  typedef __attribute__((ext_vector_type(2))) T t2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 &src = j < 2 ? s0 : s1;
    const int e = 2 * (j & 1), o = 4 * (j >> 1) + e;  // source element, operand slot
    const f32x2 x = {src[e], src[e + 1]};
    const t2 h = __builtin_convertvector(x, t2);
    const t2 l = __builtin_convertvector(x - __builtin_convertvector(h, f32x2), t2);
    hi[o] = h[0];
    hi[o + 1] = h[1];
    lo[o] = l[0];
    lo[o + 1] = l[1];
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

// Fills an H x W table: entry (u, w) holds sqrt(D) * rpb[h][ry][rx] for the
// bias index (ry, rx) = map(u, w) when that lies in the (2k-1)^2 table, else
// `outside` (0 for margins, -inf for a baked-in window mask); `inside`
// additionally restricts the valid entries.
template <typename T, int KS, typename Map>
__device__ __forceinline__ void fill_table(const T *__restrict__ rpb, int h, float *tab, int H,
                                           int W, int tid, int nthreads, float outside,
                                           Map map) {
  constexpr int SIDE = 2 * KS - 1;
  for (int e = tid; e < H * W; e += nthreads) {
    const int u = e / W, w = e - u * W;
    int by, bx;
    const bool in = map(u, w, by, bx);
    float x = outside;
    if (in && (unsigned)by < (unsigned)SIDE && (unsigned)bx < (unsigned)SIDE)
      x = rpb != nullptr ? Elem<T>::to_f(rpb[((int64_t)h * SIDE + by) * SIDE + bx]) * kSqrtD : 0.f;
    tab[e] = x;
  }
}

// ---------------------------------------------------------------------------
// Query kernel.
template <typename T, int KS, int RY>
__global__ __launch_bounds__((BG<KS, RY>::THREADS)) void bwd_query_mfma(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, const T *__restrict__ dout, T *__restrict__ dq,
    float *__restrict__ lse, float *__restrict__ dqdot, float *__restrict__ bias_part, Shape s,
    BlockDivs dv) {
  using G = BG<KS, RY>;
  constexpr int NB = G::NB, SIDE = G::SIDE, NT = G::NT, HC = G::HC, TY = G::TY, TX = G::TX;
  constexpr int R = KS / 2;
  constexpr int HALO = G::HR * HC * 64;  // bytes per staged tensor
  // K then V halo
  __shared__ __attribute__((aligned(16))) char halo[2 * HALO];
  __shared__ float tabI[G::IH * G::IW], tabE[G::EH * G::EW];
  __shared__ float dtab[G::WAVES][NT];
  // each wave's parking space for dS (bias gradient): apart from the halo
  // for 16-row blocks, so that no wave waits for the others before parking;
  // in the halo, once every wave is done with it, for 8-row blocks (measured
  // faster there: DiNAT 56 d8 170 vs 184 us)
  constexpr int PARK = TX * KS * 16;  // floats per wave: [query column][window row][16]
  constexpr bool OWN_PARKING = RY == 16;
  static_assert(OWN_PARKING || G::WAVES * PARK * 4 <= 2 * HALO, "dS parking exceeds the halo");
  __shared__ __attribute__((aligned(16))) float parking[OWN_PARKING ? G::WAVES * PARK : 1];
  char *const kbuf = halo, *const vbuf = halo + HALO;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const Block b = block_at(id, s, dv, G::RY, G::RX);
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
  // this wave's tile; its Q / dout operands load while the halo copy runs
  const int64_t pofs = b.plane * (int64_t)s.H * s.W * kHeadDim;
  const int tci0 = b.y0 + (wave / G::NTX) * TY, tcj0 = b.x0 + (wave % G::NTX) * TX;
  const bool tile_ok = tci0 < Ly && tcj0 < Lx;
  // every query of the tile has an unclamped window (and the tile is whole)
  const bool tile_inner = tci0 >= R && tci0 + TY - 1 + R <= Ly - 1 && tcj0 >= R &&
                          tcj0 + TX - 1 + R <= Lx - 1;
  const int qy = ql / TX, qx = ql % TX;
  const int ci = min(tci0 + qy, Ly - 1), cj = min(tcj0 + qx, Lx - 1);
  const unsigned qpix = pixel_of(s, b, ci, cj);
  const typename Mma<T>::vec qv = load_operand(q + pofs + (size_t)qpix * kHeadDim, g);
  const typename Mma<T>::vec gv = load_operand(dout + pofs + (size_t)qpix * kHeadDim, g);
  fill_table<T, KS>(rpb, b.h, tabI, G::IH, G::IW, tid, G::THREADS, -INFINITY,
                    [](int u, int w, int &by, int &bx) {
                      const int oy = u - (TY - 1), ox = w - (TX - 1);  // window slot
                      by = oy + R;
                      bx = ox + R;
                      return (unsigned)oy < (unsigned)KS && (unsigned)ox < (unsigned)KS;
                    });
  fill_table<T, KS>(rpb, b.h, tabE, G::EH, G::EW, tid, G::THREADS, 0.f,
                    [](int u, int w, int &by, int &bx) {
                      by = u - (TY - 1);
                      bx = w - (TX - 1);
                      return true;
                    });
  if (bias)
    for (int e = lane; e < NT; e += 64) dtab[wave][e] = 0.f;
  __syncthreads();  // also completes the LDS copies

  const int Y0 = window_start(min(tci0, Ly - 1), Ly, KS);
  const int X0 = window_start(min(tcj0, Lx - 1), Lx, KS);
  const int sy = window_start(ci, Ly, KS), sx = window_start(cj, Lx, KS);
  f32x4 dp[NB];  // dP, then dS
  if (tile_ok) {
    const bool qok = tci0 + qy < Ly && tcj0 + qx < Lx;
    const int lr0 = Y0 - hy0, lc0 = X0 - hx0;
    f32x4 sc[NB];
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bool inner = tile_inner;
    const char *kb = kbuf + (lr0 * HC + lc0 + ql) * 64 + 16 * (g ^ (((lc0 + ql) >> 1) & 3));
    const char *vb = vbuf + (kb - kbuf);
    if (inner) {
      const float *tb = tabI + (TY - 1 - qy) * G::IW + (4 * g - qx + TX - 1);
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        f32x4 cin;
#pragma unroll
        for (int i = 0; i < 4; ++i) cin[i] = tb[a * G::IW + i];
        sc[a] = Mma<T>::run(*(const typename Mma<T>::vec *)(kb + a * HC * 64), qv, cin);
        dp[a] = Mma<T>::run(*(const typename Mma<T>::vec *)(vb + a * HC * 64), gv, zero);
      }
    } else {
      // +inf inside the query's window, -inf outside: one min per bound
      float capx[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        capx[i] = (unsigned)(X0 + 4 * g + i - sx) < (unsigned)KS ? INFINITY : -INFINITY;
      int be = (Y0 - ci + KS - 1 + TY - 1) * G::EW + (X0 + 4 * g - cj + KS - 1 + TX - 1);
      asm volatile("" : "+v"(be));  // one base register; the reads use immediate offsets
      const float *tb = tabE + be;
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const float capy = (unsigned)(Y0 + a - sy) < (unsigned)KS ? INFINITY : -INFINITY;
        f32x4 cin;
#pragma unroll
        for (int i = 0; i < 4; ++i) cin[i] = fminf(fminf(tb[a * G::EW + i], capx[i]), capy);
        sc[a] = Mma<T>::run(*(const typename Mma<T>::vec *)(kb + a * HC * 64), qv, cin);
        dp[a] = Mma<T>::run(*(const typename Mma<T>::vec *)(vb + a * HC * 64), gv, zero);
      }
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
    float l = 0.f, pd = 0.f;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[a][i] = __builtin_amdgcn_exp2f(fmaf(sc[a][i], c2, -mc));  // unnormalised p
        l += sc[a][i];
        pd = fmaf(sc[a][i], dp[a][i], pd);
      }
    l = group_sum(l);
    pd = group_sum(pd);
    const float inv = __builtin_amdgcn_rcpf(l);  // l >= 1 (the maximum contributes 1)
    const float dqd = pd * inv;                   // Dq = sum P dP
    const float ninvd = -inv * dqd;
    // dS = P (dP - Dq) = p (inv dP - inv Dq)
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[a][i] = pinned(sc[a][i] * fmaf(dp[a][i], inv, ninvd));
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
  // Bias gradient of the tile.  Each wave parks its dS rows in its own LDS
  // slice, one query row of the tile at a time ([query column][window row]
  // [16 halo columns]), and lane l sums window slot l over that row's
  // queries, in column order, into the wave's table (plain read-add-write:
  // the lanes' entries are distinct).
  if constexpr (!OWN_PARKING) __syncthreads();  // every wave is done with the halo
  if (tile_ok) {
    float *park = (OWN_PARKING ? parking : (float *)halo) + wave * PARK;
    float *wt = dtab[wave];
    constexpr int NS = (KS * KS + 63) / 64;  // window slots per lane
    int pslot[NS], eslot[NS];                // slot's parking / table offsets
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int slot = min(u * 64 + lane, KS * KS - 1);
      const int wa = slot / KS, wc = slot - wa * KS;
      pslot[u] = wa * 16 + wc;
      eslot[u] = wa * SIDE + wc;
    }
    for (int h = 0; h < TY; ++h) {
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
      if (tile_inner) {
        // every query of the row has an unclamped window: query column x's
        // slot sits x columns further in the parking, and every query's
        // slot maps to the same table entry (offset R, R from the slot)
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          if (u * 64 + lane < KS * KS) {
            float run = 0.f;
#pragma unroll
            for (int x = 0; x < TX; ++x) run += park[x * (KS * 16 + 1) + pslot[u]];
            wt[eslot[u] + R * SIDE + R] += run;
          }
        }
        __builtin_amdgcn_wave_barrier();
        continue;
      }
      // the row's queries in column order; the table offset of a slot
      // depends on the query only through its window start (uniform), so
      // consecutive queries with the same start share one running sum
      const int rowcls = (window_start(qi, Ly, KS) - qi + KS - 1) * SIDE;
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const bool active = u * 64 + lane < KS * KS;
        float run = 0.f;
        int rc = -1;  // table offset (uniform) of the running sum
#pragma unroll
        for (int x = 0; x < TX; ++x) {
          const int qj = tcj0 + x;
          if (qj >= Lx) break;
          const int sxq = window_start(qj, Lx, KS);
          const int cls = rowcls + sxq - qj + KS - 1;
          const float val = park[x * KS * 16 + (sxq - X0) + pslot[u]];
          if (cls != rc) {
            if (rc >= 0 && active) wt[eslot[u] + rc] += run;
            run = val;
            rc = cls;
          } else {
            run += val;
          }
        }
        if (active) wt[eslot[u] + rc] += run;
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
template <typename T, int KS, int RY>
__global__ __launch_bounds__((BG<KS, RY>::THREADS)) void bwd_key_mfma(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, const T *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ dqdot, T *__restrict__ dk, T *__restrict__ dv, Shape s,
    BlockDivs dvs) {
  using G = BG<KS, RY>;
  constexpr int QR = G::QR, QC = G::QC, TY = G::TY, TX = G::TX, FW = G::FW;
  constexpr int R = KS / 2;
  __shared__ __attribute__((aligned(16))) char qbuf[QR * QC * 64], gbuf[QR * QC * 64];
  __shared__ f32x2 lbuf[QR * QC];  // (log-sum-exp, Dq) of the halo queries
  __shared__ float tabI[G::FH * FW], tabE[G::FH * FW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int id = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const Block b = block_at(id, s, dvs, G::RY, G::RX);
  if (!b.ok) return;
  const int Ly = b.Ly, Lx = b.Lx;
  const int y1 = min(b.y0 + G::RY, Ly) - 1, x1 = min(b.x0 + G::RX, Lx) - 1;
  const int hq0 = inv_lo(b.y0, KS), hq1 = inv_hi(y1, Ly, KS);
  const int hc0 = inv_lo(b.x0, KS), hc1 = inv_hi(x1, Lx, KS);
  stage_halo<T, QR, QC>(q, s, b, hq0, hq1, hc0, hc1, qbuf, wave, lane, G::WAVES);
  stage_halo<T, QR, QC>(dout, s, b, hq0, hq1, hc0, hc1, gbuf, wave, lane, G::WAVES);
  const int64_t pofs = b.plane * (int64_t)s.H * s.W * kHeadDim;
  const int64_t qbase = pofs / kHeadDim;
  // this wave's key tile; its K / V operands load while the halo copy runs
  const int t0 = b.y0 + (wave / G::NTX) * TY, tx0 = b.x0 + (wave % G::NTX) * TX;
  const int kyl = t0 + ql / TX, kxl = tx0 + ql % TX;
  const bool kok = kyl < Ly && kxl < Lx;
  const int ky = min(kyl, Ly - 1), kx = min(kxl, Lx - 1);
  const unsigned kpix = pixel_of(s, b, ky, kx);
  const typename Mma<T>::vec kv = load_operand(k + pofs + (size_t)kpix * kHeadDim, g);
  const typename Mma<T>::vec vv = load_operand(v + pofs + (size_t)kpix * kHeadDim, g);
  for (int p = tid; p < QR * QC; p += G::THREADS) {
    const int row = p / QC, col = p - row * QC;
    const int64_t qi = qbase + pixel_of(s, b, min(hq0 + row, hq1), min(hc0 + col, hc1));
    lbuf[p] = f32x2{lse[qi], dqdot[qi]};
  }
  // entry (u, w): query - key offset (u - (TY-1) - (k-1), w - (TX-1) - (k-1))
  fill_table<T, KS>(rpb, b.h, tabI, G::FH, FW, tid, G::THREADS, -INFINITY,
                    [](int u, int w, int &by, int &bx) {
                      const int oy = u - (TY - 1) - (KS - 1), ox = w - (TX - 1) - (KS - 1);
                      by = KS - 1 - oy;
                      bx = KS - 1 - ox;
                      return oy >= -R && oy <= R && ox >= -R && ox <= R;
                    });
  fill_table<T, KS>(rpb, b.h, tabE, G::FH, FW, tid, G::THREADS, 0.f,
                    [](int u, int w, int &by, int &bx) {
                      by = KS - 1 - (u - (TY - 1) - (KS - 1));
                      bx = KS - 1 - (w - (TX - 1) - (KS - 1));
                      return true;
                    });
  __syncthreads();  // also completes the LDS copies
  if (t0 >= Ly || tx0 >= Lx) return;
  const int t1 = min(t0 + TY, Ly) - 1, tx1 = min(tx0 + TX, Lx) - 1;
  const int rlo = inv_lo(t0, KS), rhi = inv_hi(t1, Ly, KS);
  const int clo = inv_lo(tx0, KS), chi = inv_hi(tx1, Lx, KS);
  // every query reaching the tile has an unclamped window (and the tile is
  // whole): the window mask is the table's
  const bool inner = t0 + TY - 1 < Ly && tx0 + TX - 1 < Lx && rlo >= R && rhi <= Ly - 1 - R &&
                     clo >= R && chi <= Lx - 1 - R;
  const float c2 = kLog2e * kInvSqrtD;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 k0 = zero, k1 = zero, v0 = zero, v1 = zero;
  // one row pair (r, r+1) of one 16-column chunk starting at c0
  auto pair = [&](const float *tb, int r, int acol, int tc, const int (&lcol)[4],
                  const float (&capx)[4], bool edge) {
    f32x4 P[2], dS[2];
    const int lrow0 = r - hq0;  // r + 1 - hq0 <= QR - 1: the staged rows cover the pair
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qr = r + u, lrow = lrow0 + u;
      f32x4 cin;
      if (edge) {
        const int syq = window_start(min(qr, Ly - 1), Ly, KS);
        const float capy = qr < Ly && (unsigned)(ky - syq) < (unsigned)KS ? INFINITY : -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) cin[i] = fminf(fminf(tb[u * FW + i], capx[i]), capy);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cin[i] = tb[u * FW + i];
      }
      const f32x4 sv = Mma<T>::run(halo_vec<T, QC>(qbuf, lrow, acol, g), kv, cin);
      const f32x4 dpv = Mma<T>::run(halo_vec<T, QC>(gbuf, lrow, acol, g), vv, zero);
      const f32x2 *lr = lbuf + lrow * QC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 ld = lr[lcol[i]];
        P[u][i] = pinned(__builtin_amdgcn_exp2f(fmaf(sv[i], c2, -ld[0])));
        dS[u][i] = pinned(P[u][i] * (dpv[i] - ld[1]));
      }
    }
    typename Mma<T>::vec phi, plo, shi, slo;
    split_operand<T>(P[0], P[1], phi, plo);
    split_operand<T>(dS[0], dS[1], shi, slo);
    v0 = mma2<T>(halo_tr<T, QC>(gbuf, lrow0, tc, ql, 0), phi, plo, v0);
    v1 = mma2<T>(halo_tr<T, QC>(gbuf, lrow0, tc, ql, 1), phi, plo, v1);
    k0 = mma2<T>(halo_tr<T, QC>(qbuf, lrow0, tc, ql, 0), shi, slo, k0);
    k1 = mma2<T>(halo_tr<T, QC>(qbuf, lrow0, tc, ql, 1), shi, slo, k1);
  };
  for (int c0 = clo; c0 <= chi; c0 += 16) {
    // this lane's 4 query columns c0 + 4g + i: window test and LDS column
    // (clamped: columns past the halo are masked)
    float capx[4];
    int lcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qc = c0 + 4 * g + i;
      const bool in =
          qc < Lx && (unsigned)(kx - window_start(min(qc, Lx - 1), Lx, KS)) < (unsigned)KS;
      capx[i] = in ? INFINITY : -INFINITY;
      lcol[i] = min(qc - hc0, QC - 1);
    }
    const int acol = min(c0 + ql - hc0, QC - 1);
    const int tc = min(c0 + 4 * g + (ql >> 2) - hc0, QC - 1);
    // table entry of (query row r, column c0 + 4g) against this lane's key
    int bt = (rlo - ky + KS - 1 + TY - 1) * FW + (c0 + 4 * g - kx + KS - 1 + TX - 1);
    asm volatile("" : "+v"(bt));
    if (inner) {
      const float *tb = tabI + bt;
#pragma unroll
      for (int j = 0; j < (TY + KS - 1) / 2; ++j)
        pair(tb + 2 * j * FW, rlo + 2 * j, acol, tc, lcol, capx, false);
    } else {
      const float *tb = tabE + bt;
      for (int r = rlo; r <= rhi; r += 2, tb += 2 * FW) pair(tb, r, acol, tc, lcol, capx, true);
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
  BlockDivs divs;
};

template <int KS, int RY>
Grid grid_of(const Shape &s) {
  using G = BG<KS, RY>;
  Grid r;
  r.nby = (class_len(s.H, 0, s.dil) + G::RY - 1) / G::RY;
  r.nbx = (class_len(s.W, 0, s.dil) + G::RX - 1) / G::RX;
  r.bpp = (int64_t)s.dil * s.dil * r.nby * r.nbx;
  r.nblocks = (int64_t)s.B * s.heads * r.bpp;
  r.divs = BlockDivs{make_fastdiv((uint32_t)r.nbx), make_fastdiv((uint32_t)r.nby),
                     make_fastdiv((uint32_t)s.dil), make_fastdiv((uint32_t)s.heads)};
  return r;
}

// Short residue classes take 8-row blocks (k <= 9; longer windows need
// longer classes).
inline bool short_classes(const Shape &s, int ks) {
  return ks <= 9 && class_len(s.H, 0, s.dil) <= 8;
}

template <typename T, int KS, int RY>
hipError_t launch_rt(const void *q, const void *k, const void *v, const void *rpb,
                     const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                     const Shape &s, hipStream_t st) {
  using G = BG<KS, RY>;
  const Grid gr = grid_of<KS, RY>(s);
  if (gr.nblocks > INT_MAX) return hipErrorInvalidConfiguration;
  float *lse = (float *)ws;
  float *dqdot = lse + s.n_query;
  float *part = drpb != nullptr ? dqdot + s.n_query : nullptr;
  bwd_query_mfma<T, KS, RY><<<dim3((unsigned)gr.nblocks), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (const T *)dout, (T *)dq, lse,
      dqdot, part, s, gr.divs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_key_mfma<T, KS, RY><<<dim3((unsigned)gr.nblocks), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (const T *)dout, lse, dqdot,
      (T *)dk, (T *)dv, s, gr.divs);
  e = hipGetLastError();
  if (e != hipSuccess || drpb == nullptr) return e;
  bwd_bias_sum<<<dim3(G::NT, s.heads), kSumThreads, 0, st>>>(part, drpb, s.B, s.heads,
                                                             (int)gr.bpp, G::NT);
  return hipGetLastError();
}

template <typename T, int KS>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *rpb,
                    const void *dout, void *dq, void *dk, void *dv, float *drpb, void *ws,
                    const Shape &s, hipStream_t st) {
  if constexpr (KS <= 9)
    if (short_classes(s, KS))
      return launch_rt<T, KS, 8>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
  return launch_rt<T, KS, 16>(q, k, v, rpb, dout, dq, dk, dv, drpb, ws, s, st);
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
  if constexpr (KS <= 9)
    if (short_classes(s, KS)) return grid_of<KS, 8>(s).nblocks;
  return grid_of<KS, 16>(s).nblocks;
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
