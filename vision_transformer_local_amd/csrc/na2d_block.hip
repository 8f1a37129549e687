// na2d_block.hip -- the attention block of a NAT / DiNAT layer in one kernel:
// q/k/v projection with bias, per-head 2D neighborhood attention with the
// relative-position bias, output projection with bias (DiNAT walk-through
// blog, "What is DiNAT": the module projects the channels-last features to
// queries, keys and values with bias and runs natten2dqkrpb -> softmax ->
// natten2dav per head; the heads' outputs then pass the block's output
// projection, the usual close of an attention block).  This kernel covers C = 64
// channels in 2 heads of 32, k in {3, 5, 7}, no dilation, maps of at least
// k x k (no padding); other blocks take the three-launch path.
//
// Per block of 16 x 8 queries of one image (four waves, each with two 2 x 8
// query tiles), with both heads:
//   * x is read straight into MFMA operands (lane (g, i) holds 8 channels of
//     pixel i), never staged: the halo rows of the block for the key/value
//     projection (loaded once per head, so that they are not live across the
//     attention), the block's own pixels for the query projection (fetched
//     for the next block during the current one's second head).
//   * Q^T = Wq . x^T: lane (g, i) ends with channels 16c + 4g..+3 of query i
//     for the four 16-channel blocks c.  For head h the lane's two blocks
//     2h, 2h+1 form the 8-element operand of the score product as they are:
//     k-position 8g + j stands for head channel pi(8g + j) = 16*(j/4) + 4g +
//     j%4.  A dot product does not care about the order of its terms, so the
//     keys are stored in the same order pi and Q never passes through LDS.
//   * Per head: K^T and V^T of the halo (up to RY + k - 1 rows x 16 columns,
//     the tile's key block; columns past the map repeat its last column, and
//     the one row past the block's halo that a bottom-clamped tile reads
//     repeats the last map row -- finite values that only ever meet masked
//     scores) are projected into LDS, K in order pi, V in channel
//     order, 16-byte pieces XOR-swizzled by column; then each wave runs the
//     attention of its two query tiles against them as the general matrix-core
//     kernel does (scores transposed, bias and mask as the accumulator input,
//     V^T read with ds_read_b64_tr_b16, softmax denominator from a product with
//     ones over the 16-bit weights).
//   * The two heads' outputs, rounded to the data type, are again in order pi
//     per head and feed the output projection directly: Wo sits in LDS with
//     its input channels permuted to pi.  y rows are written once.
// The weights (q, k, v, out: 32 KB) live in LDS for the life of a persistent
// workgroup; one head's K and V halo (44 KB) plus the bias table leave room
// for two workgroups per compute unit, 2 waves per SIMD with 256 registers
// each.  Each weight operand read from LDS serves two query tiles (the query
// and output projections) or about six halo rows (key/value projection).
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kC = 64;  // channels: 2 heads of 32

template <int KS, int RY> struct BlockGeom {
  static constexpr int R = KS / 2;
  static constexpr int TY = 2, TX = 8;          // query tile (16 queries)
  static constexpr int TPW = 2;                 // tiles per wave (stacked vertically)
  static constexpr int RX = TX;                 // block columns: one tile column
  static constexpr int WAVES = RY / (TY * TPW), THREADS = WAVES * 64;
  static constexpr int NB = TY + KS - 1;        // key rows of a tile
  static constexpr int HR = RY + KS - 1;        // staged key rows
  static constexpr int HC = 16;                 // staged key columns
  static constexpr int RPW = (HR + WAVES - 1) / WAVES;  // halo rows per wave (at most)
  static constexpr int SIDE = 2 * KS - 1;
  // bias table: interior part (mask baked in), then the plain table with
  // zero margins, as in the general kernel
  static constexpr int IU = NB + TY - 1, IW = 16 + TX, NINT = IU * IW;
  static constexpr int MARGIN = TY * SIDE + 32;
  static constexpr int BOFF = NINT + MARGIN;
  static constexpr int NTAB = NINT + SIDE * SIDE + 2 * MARGIN;
  static constexpr int TPT = (NTAB + THREADS - 1) / THREADS;  // table entries per thread
  static constexpr int WMAT = kC * kC * 2;      // bytes of one weight matrix
  static constexpr int KVB = HR * HC * 64;      // bytes of one head's K (or V) halo
  static constexpr int LDS = 4 * WMAT + 2 * KVB + NTAB * 4 + 4 * kC * 4;
  static_assert(TX + KS - 1 <= HC, "key columns do not cover the tile");
  static_assert(NB % 2 == 0, "PV consumes key rows in pairs");
  static_assert(RY % (TY * TPW) == 0, "blocks hold whole waves of tiles");
  static_assert(LDS <= 80 * 1024, "two workgroups per compute unit");
};

// Entry e of the bias table (times sqrt(D), -inf outside the window in the
// interior part): index into the head's rpb, -1 for a zero margin, -2 for -inf.
template <int KS, int RY>
__device__ __forceinline__ int table_entry(int e) {
  using G = BlockGeom<KS, RY>;
  if (e >= G::NINT) {
    const int t = e - G::BOFF;
    return (t >= 0 && t < G::SIDE * G::SIDE) ? t : -1;
  }
  // interior entry (u, w): key row - first query row's window row, key column
  // offset within the query's window
  const int u = e / G::IW - (G::TY - 1), w = e % G::IW - G::TX;
  return ((unsigned)u < (unsigned)KS && (unsigned)w < (unsigned)KS)
             ? (u + G::R) * G::SIDE + w + G::R
             : -2;
}

// LDS offset of 16-byte piece c (0..7) of row r of a 64 x 64 weight matrix:
// pieces XOR-swizzled by row, so that the 16 rows of an operand read spread
// over all banks.
__device__ __forceinline__ int wpiece(int r, int c) { return r * 128 + 16 * (c ^ (r & 7)); }

// A lane reads piece 4kk + g of row r0 + ql of an operand (r0 a multiple of
// 8, so that r & 7 = ql & 7): wpiece(r0 + ql, 4kk + g) = r0 * 128 + wl[kk]
// with the two per-lane offsets below (wl[1] = wl[0] ^ 64).  Operand reads
// then cost one register each plus an immediate offset.
struct WeightLane {
  int wl0, wl1;
};

__device__ __forceinline__ WeightLane weight_lane(int ql, int g) {
  const int wl0 = ql * 128 + 16 * (g ^ (ql & 3)) + 64 * ((ql >> 2) & 1);
  return WeightLane{wl0, wl0 ^ 64};
}

// Where a block sits: image, first query row / column, their ends, and the
// first row / column of the key halo (the window start of the first query).
struct BlockPos {
  int64_t img;  // element offset of the image in x and y
  int y0, y1, x0, x1, hy0, hx0;
  int hrows;    // staged halo rows any live tile reads (rows past them are not projected)
};

template <int KS, int RY>
__device__ __forceinline__ BlockPos block_pos(int id, int H, int W, const FastDiv &fnbx,
                                              const FastDiv &fnby) {
  BlockPos p;
  const int t = (int)fast_div((uint32_t)id, fnbx), bx = id - t * (int)fnbx.div;
  const int b = (int)fast_div((uint32_t)t, fnby), by = t - b * (int)fnby.div;
  p.img = (int64_t)b * H * W * kC;
  p.y0 = by * RY;
  p.y1 = min(p.y0 + RY, H);
  p.x0 = bx * BlockGeom<KS, RY>::RX;
  p.x1 = min(p.x0 + BlockGeom<KS, RY>::RX, W);
  p.hy0 = window_start(p.y0, H, KS);
  p.hx0 = window_start(p.x0, W, KS);
  // the block's real halo rows, plus the one past them that a tile with a
  // bottom-clamped window reads as its (masked) last key row
  p.hrows = min(BlockGeom<KS, RY>::HR, window_start(p.y1 - 1, H, KS) + KS - p.hy0 + 1);
  return p;
}

// The x operands of a block for this lane: its wave's halo rows (pixel
// (hy0 + r, hx0 + ql), clamped into the map) and its query (clamped into the
// block), channels 8g..8g+7 and 32+8g..32+8g+7.
template <typename T, int KS, int RY> struct XOps {
  u32x4 halo[BlockGeom<KS, RY>::RPW][2];
  u32x4 query[BlockGeom<KS, RY>::TPW][2];
};

// First query row of tile t of this wave.
template <int KS, int RY>
__device__ __forceinline__ int tile_row(const BlockPos &p, int wave, int t) {
  using G = BlockGeom<KS, RY>;
  return p.y0 + (wave * G::TPW + t) * G::TY;
}

template <typename T, int KS, int RY>
__device__ __forceinline__ void load_halo(const T *__restrict__ x, const BlockPos &p, int H,
                                          int W, int wave, int ql, int g, XOps<T, KS, RY> &o) {
  using G = BlockGeom<KS, RY>;
  const int hc = min(p.hx0 + ql, W - 1);
#pragma unroll
  for (int j = 0; j < G::RPW; ++j) {
    const int r = wave + j * G::WAVES;
    if (r < p.hrows) {
      const int hr = min(p.hy0 + r, H - 1);
      const u32x4 *src = (const u32x4 *)(x + p.img + ((int64_t)hr * W + hc) * kC) + g;
      o.halo[j][0] = src[0];
      o.halo[j][1] = src[4];
    }
  }
}

template <typename T, int KS, int RY>
__device__ __forceinline__ void load_query(const T *__restrict__ x, const BlockPos &p, int W,
                                           int wave, int ql, int g, XOps<T, KS, RY> &o) {
  using G = BlockGeom<KS, RY>;
  const int qc = min(p.x0 + ql % G::TX, p.x1 - 1);
#pragma unroll
  for (int t = 0; t < G::TPW; ++t) {
    const int qr = min(tile_row<KS, RY>(p, wave, t) + ql / G::TX, p.y1 - 1);
    const u32x4 *src = (const u32x4 *)(x + p.img + ((int64_t)qr * W + qc) * kC) + g;
    o.query[t][0] = src[0];
    o.query[t][1] = src[4];
  }
}

template <typename T>
__device__ __forceinline__ u32x2 pack4(const f32x4 &a) {
  typedef __attribute__((ext_vector_type(4))) T vec4;
  vec4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = static_cast<T>(a[i]);
  return __builtin_bit_cast(u32x2, r);
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::vec join(u32x2 a, u32x2 b) {
  return __builtin_bit_cast(typename Mma<T>::vec, u32x4{a[0], a[1], b[0], b[1]});
}

// One head's attention for this wave's TPW query tiles (2 x 8 queries each,
// the first starting at row tci0, the next TY rows further): for each, out^T
// of the head, rounded, as the output projection's operand (channels in order
// pi).  One interior-or-edge decision covers all the wave's tiles, so that
// their independent products and softmax steps share straight-line code the
// compiler can interleave.
template <typename T, int KS, int RY>
__device__ __forceinline__ void attend(const char *kbuf, const char *vbuf, const float *tab,
                                       const typename Mma<T>::vec (&qv)[BlockGeom<KS, RY>::TPW],
                                       const BlockPos &p, int H, int W, int tci0, int lane,
                                       u32x4 (&out)[BlockGeom<KS, RY>::TPW]) {
  using G = BlockGeom<KS, RY>;
  using vec = typename Mma<T>::vec;
  constexpr int TY = G::TY, TX = G::TX, NB = G::NB, SIDE = G::SIDE, R = G::R, TPW = G::TPW;
  const int ql = lane & 15, g = lane >> 4;
  const int qy = ql / TX, qx = ql % TX;
  int Y0[TPW], lrow0[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    Y0[t] = window_start(tci0 + t * TY, H, KS);
    lrow0[t] = Y0[t] - p.hy0;  // the tile's key block starts at staged column 0
  }

  // S^T rows: key (Y0 + a, hx0 + 4g + i) against query ql, i = 0..3
  const int kofs = ql * 64 + 16 * (g ^ ((ql >> 1) & 3));
  f32x4 sc[TPW][NB];
  const bool inner = tci0 >= R && tci0 + TPW * TY - 1 + R <= H - 1 && p.x0 >= R &&
                     p.x0 + TX - 1 + R <= W - 1;
  if (inner) {
    const float *tb = tab + (TY - 1 - qy) * G::IW + (TX + 4 * g - qx);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const u32x4 *kb = (const u32x4 *)(kbuf + lrow0[t] * G::HC * 64 + kofs);
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        f32x4 cin;
#pragma unroll
        for (int i = 0; i < 4; ++i) cin[i] = tb[a * G::IW + i];
        sc[t][a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * G::HC * 4]), qv[t], cin);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const u32x4 *kb = (const u32x4 *)(kbuf + lrow0[t] * G::HC * 64 + kofs);
      // key rows TY-1..k-1 of the key block lie inside every query row's window
      const int ci = min(tci0 + t * TY + qy, p.y1 - 1), cj = min(p.x0 + qx, p.x1 - 1);
      const int sy = window_start(ci, H, KS), sx = window_start(cj, W, KS);
      const int rowrel = Y0[t] - sy, colrel = p.hx0 + 4 * g - sx;
      int bidx = G::BOFF + (Y0[t] - ci + KS - 1) * SIDE + (p.hx0 + 4 * g - cj + KS - 1);
      asm volatile("" : "+v"(bidx));  // one base register; the reads use immediate offsets
      const float *bb = tab + bidx;
      float ccap[4];  // +inf inside the window's columns, -inf outside
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ccap[i] = (unsigned)(colrel + i) < (unsigned)KS ? INFINITY : -INFINITY;
        asm volatile("" : "+v"(ccap[i]));
      }
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const bool rtest = !(a >= TY - 1 && a <= KS - 1);
        float rcap = (unsigned)(rowrel + a) < (unsigned)KS ? INFINITY : -INFINITY;
        if (rtest) asm volatile("" : "+v"(rcap));
        f32x4 cin;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cin[i] = rtest ? fminf(fminf(bb[a * SIDE + i], ccap[i]), rcap)
                         : fminf(bb[a * SIDE + i], ccap[i]);
        sc[t][a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * G::HC * 4]), qv[t], cin);
      }
    }
  }

  // softmax numerators exp((S - max) / sqrt(D)); the 4 lane groups hold
  // disjoint keys of the same query
  const float c2 = kLog2e / kSqrtD;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][a][i]);
    const float mc = group_max(mx) * c2;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][a][i] = __builtin_amdgcn_exp2f(fmaf(sc[t][a][i], c2, -mc));
  }

  // out^T = V^T . P^T over pairs of key rows; lane (g, 4k + qd) is the source
  // of channels 4qd..4qd+3 (and 16+4qd..) of key column hx0 + 4g + k
  const int vcol = 4 * g + (ql >> 2), qd = ql & 3, vs = (vcol >> 1) & 3;
  const int vofs = vcol * 64 + 8 * (qd & 1);
  const int va0 = vofs + 16 * ((qd >> 1) ^ vs), va1 = vofs + 16 * (((qd >> 1) | 2) ^ vs);
  vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);
  constexpr int RB = G::HC * 64;  // bytes per staged row
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const char *vrow = vbuf + lrow0[t] * RB;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, o2 = o0;
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) {
      vec pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<T>(sc[t][2 * j][i]);
        pb[4 + i] = static_cast<T>(sc[t][2 * j + 1][i]);
      }
      const char *r0 = vrow + (2 * j) * RB, *r1 = vrow + (2 * j + 1) * RB;
      const u32x2 a0 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(r0 + va0)));
      const u32x2 a1 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(r1 + va0)));
      const u32x2 b0 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(r0 + va1)));
      const u32x2 b1 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(r1 + va1)));
      o0 = Mma<T>::run(join<T>(a0, a1), pb, o0);
      o1 = Mma<T>::run(join<T>(b0, b1), pb, o1);
      o2 = Mma<T>::run(ones, pb, o2);
    }
    const float inv = __builtin_amdgcn_rcpf(o2[0]);
    const u32x2 w0 = pack4<T>(o0 * inv), w1 = pack4<T>(o1 * inv);
    out[t] = u32x4{w0[0], w0[1], w1[0], w1[1]};
  }
}

// Two workgroups of 4 waves per compute unit: 2 waves per SIMD (at most 256
// registers each).
template <typename T, int KS, int RY>
__global__ __launch_bounds__((BlockGeom<KS, RY>::THREADS), 2) void block_fused_kernel(
    const T *__restrict__ x, const T *__restrict__ w_qkv, const T *__restrict__ b_qkv,
    const T *__restrict__ rpb, const T *__restrict__ w_out, const T *__restrict__ b_out,
    T *__restrict__ y, int H, int W, FastDiv fnbx, FastDiv fnby, int nblocks) {
  using G = BlockGeom<KS, RY>;
  using vec = typename Mma<T>::vec;
  // weights: Wq, Wk, Wv as [out][in], Wo as [out][in in order pi per head]
  __shared__ __attribute__((aligned(16))) char wts[4 * G::WMAT];
  __shared__ __attribute__((aligned(16))) char kbuf[G::KVB], vbuf[G::KVB];
  __shared__ __attribute__((aligned(16))) float tab[G::NTAB];
  __shared__ __attribute__((aligned(16))) float bias[4 * kC];  // bq, bk, bv, bo

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int wg = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int b0 = (int)((int64_t)nblocks * wg / gridDim.x);
  const int b1 = (int)((int64_t)nblocks * (wg + 1) / gridDim.x);
  if (b0 >= b1) return;

  // ---- once per workgroup: weights, biases, raw bias-table values ----
  XOps<T, KS, RY> xo;
  BlockPos pos = block_pos<KS, RY>(b0, H, W, fnbx, fnby);
  load_query<T, KS, RY>(x, pos, W, wave, ql, g, xo);
  for (int e = tid; e < 4 * kC * 8; e += G::THREADS) {
    const int mat = e >> 9, r = (e >> 3) & 63, c = e & 7;
    u32x4 val;
    if (mat < 3) {
      val = *(const u32x4 *)(w_qkv + (mat * kC + r) * kC + 8 * c);
    } else {
      // piece c = 4h + gg holds input channels 32h + 4gg.. and 32h + 16 + 4gg..
      const T *src = w_out + r * kC + 32 * (c >> 2) + 4 * (c & 3);
      const u32x2 lo = *(const u32x2 *)src, hi = *(const u32x2 *)(src + 16);
      val = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    *(u32x4 *)(wts + mat * G::WMAT + wpiece(r, c)) = val;
  }
  for (int e = tid; e < 4 * kC; e += G::THREADS) {
    float bv = 0.f;
    if (e < 3 * kC) {
      if (b_qkv != nullptr) bv = Elem<T>::to_f(b_qkv[e]);
    } else if (b_out != nullptr) {
      bv = Elem<T>::to_f(b_out[e - 3 * kC]);
    }
    bias[e] = bv;
  }
  float traw[2][G::TPT];  // this thread's table entries (times sqrt(D)) for both heads
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int it = 0; it < G::TPT; ++it) {
      const int idx = table_entry<KS, RY>(min(tid + it * G::THREADS, G::NTAB - 1));
      float v = idx == -2 ? -INFINITY : 0.f;
      if (idx >= 0 && rpb != nullptr)
        v = Elem<T>::to_f(rpb[h * G::SIDE * G::SIDE + idx]) * kSqrtD;
      traw[h][it] = v;
    }
  const char *wq = wts, *wk = wts + G::WMAT, *wv = wts + 2 * G::WMAT, *wo = wts + 3 * G::WMAT;
  const WeightLane wl = weight_lane(ql, g);
  for (int bi = b0; bi < b1; ++bi) {
    const BlockPos p = pos;
    // the key halo rows of this wave: loaded per head, so that they are not
    // live across the attention (the second read hits L2)
    load_halo<T, KS, RY>(x, p, H, W, wave, ql, g, xo);
    __syncthreads();  // weights and biases written (first block); previous block done

    // ---- query projection: Q^T for 64 channels of this lane's queries ----
    vec qop[G::TPW][2];
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {  // channel blocks 2hc, 2hc + 1: head hc
      f32x4 acc[G::TPW][2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int c = 2 * hc + c2;
        const f32x4 b4 = *(const f32x4 *)(bias + 16 * c + 4 * g);
        const vec a0 = *(const vec *)(wq + 16 * c * 128 + wl.wl0);
        const vec a1 = *(const vec *)(wq + 16 * c * 128 + wl.wl1);
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) {
          acc[t][c2] = Mma<T>::run(a0, __builtin_bit_cast(vec, xo.query[t][0]), b4);
          acc[t][c2] = Mma<T>::run(a1, __builtin_bit_cast(vec, xo.query[t][1]), acc[t][c2]);
        }
      }
#pragma unroll
      for (int t = 0; t < G::TPW; ++t)
        qop[t][hc] = join<T>(pack4<T>(acc[t][0]), pack4<T>(acc[t][1]));
    }

    u32x4 ctx[G::TPW][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) {
        load_halo<T, KS, RY>(x, p, H, W, wave, ql, g, xo);
        __syncthreads();  // head 0's attention has read kbuf, vbuf, tab
      }
      // bias table of head h
#pragma unroll
      for (int it = 0; it < G::TPT; ++it) {
        const int e = tid + it * G::THREADS;
        if (e < G::NTAB) tab[e] = traw[h][it];
      }
      // K^T, V^T of head h for this wave's halo rows
      {
        const int swz = (ql >> 1) & 3;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          // the weights of one 16-channel block of K and of V at a time
          asm volatile("" ::: "memory");
          vec ak[2], av[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int off = (32 * h + 16 * c) * 128 + (kk ? wl.wl1 : wl.wl0);
            ak[kk] = *(const vec *)(wk + off);
            av[kk] = *(const vec *)(wv + off);
          }
          const f32x4 kb0 = *(const f32x4 *)(bias + kC + 32 * h + 16 * c + 4 * g);
          const f32x4 vb0 = *(const f32x4 *)(bias + 2 * kC + 32 * h + 16 * c + 4 * g);
#pragma unroll
          for (int j = 0; j < G::RPW; ++j) {
            const int r = wave + j * G::WAVES;
            if (r < p.hrows) {
              f32x4 ka = kb0, va = vb0;
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) {
                const vec xb = __builtin_bit_cast(vec, xo.halo[j][kk]);
                ka = Mma<T>::run(ak[kk], xb, ka);
                va = Mma<T>::run(av[kk], xb, va);
              }
              char *kp = kbuf + (r * G::HC + ql) * 64;
              char *vp = vbuf + (r * G::HC + ql) * 64;
              // K: piece g holds channels 4g.. (c = 0) and 16+4g.. (c = 1)
              *(u32x2 *)(kp + 16 * (g ^ swz) + 8 * c) = pack4<T>(ka);
              // V: channels 16c + 4g.. sit in piece 2c + g/2, half g&1
              *(u32x2 *)(vp + 16 * ((2 * c + (g >> 1)) ^ swz) + 8 * (g & 1)) = pack4<T>(va);
            }
          }
        }
      }
      if (h == 1) {
        // the query operands are consumed: fetch the next block's during head
        // 1's attention and the output projection
        if (bi + 1 < b1) {
          pos = block_pos<KS, RY>(bi + 1, H, W, fnbx, fnby);
          load_query<T, KS, RY>(x, pos, W, wave, ql, g, xo);
        }
      }
      __syncthreads();  // K, V and table of head h complete
      const int tci0 = tile_row<KS, RY>(p, wave, 0);
      if (tci0 < p.y1) {  // waves whose tiles lie past the map's last row idle
        vec qh[G::TPW];
        u32x4 ch[G::TPW];
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) qh[t] = qop[t][h];
        attend<T, KS, RY>(kbuf, vbuf, tab, qh, p, H, W, tci0, lane, ch);
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) ctx[t][h] = ch[t];
      }
    }

    // ---- output projection of this wave's queries ----
    // (whole-wave products: every lane supplies its weight row, also lanes
    // whose own query lies outside a ragged block and stores nothing)
    {
      const int qc = p.x0 + ql % G::TX;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 b4 = *(const f32x4 *)(bias + 3 * kC + 16 * c + 4 * g);
        const vec a0 = *(const vec *)(wo + 16 * c * 128 + wl.wl0);
        const vec a1 = *(const vec *)(wo + 16 * c * 128 + wl.wl1);
#pragma unroll
        for (int t = 0; t < G::TPW; ++t) {
          const int tci0 = tile_row<KS, RY>(p, wave, t);
          if (tci0 < p.y1) {
            f32x4 acc = Mma<T>::run(a0, __builtin_bit_cast(vec, ctx[t][0]), b4);
            acc = Mma<T>::run(a1, __builtin_bit_cast(vec, ctx[t][1]), acc);
            const int qr = tci0 + ql / G::TX;
            if (qr < p.y1 && qc < p.x1)
              *(u32x2 *)(y + p.img + ((int64_t)qr * W + qc) * kC + 16 * c + 4 * g) =
                  pack4<T>(acc);
          }
        }
      }
    }
  }
}

template <typename T, int KS, int RY>
hipError_t launch_rt(const void *x, const void *w_qkv, const void *b_qkv, const void *rpb,
                     const void *w_out, const void *b_out, void *y, int B, int H, int W,
                     hipStream_t st) {
  using G = BlockGeom<KS, RY>;
  const int nby = (H + RY - 1) / RY, nbx = (W + G::RX - 1) / G::RX;
  const int64_t nblocks = (int64_t)B * nby * nbx;
  if (nblocks > INT_MAX) return hipErrorInvalidConfiguration;
  const int64_t slots = 2 * (int64_t)device_compute_units();  // two workgroups per CU
  const int64_t grid = nblocks < slots ? nblocks : slots;
  block_fused_kernel<T, KS, RY><<<dim3((unsigned)grid), G::THREADS, 0, st>>>(
      (const T *)x, (const T *)w_qkv, (const T *)b_qkv, (const T *)rpb, (const T *)w_out,
      (const T *)b_out, (T *)y, H, W, make_fastdiv((uint32_t)nbx), make_fastdiv((uint32_t)nby),
      (int)nblocks);
  return hipGetLastError();
}

template <typename T, int KS>
hipError_t launch_ks(const void *x, const void *w_qkv, const void *b_qkv, const void *rpb,
                     const void *w_out, const void *b_out, void *y, int B, int H, int W,
                     hipStream_t st) {
  return launch_rt<T, KS, 16>(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W, st);
}

template <typename T>
hipError_t launch_dtype(const void *x, const void *w_qkv, const void *b_qkv, const void *rpb,
                        const void *w_out, const void *b_out, void *y, int B, int H, int W,
                        int ks, hipStream_t st) {
  switch (ks) {
    case 3: return launch_ks<T, 3>(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W, st);
    case 5: return launch_ks<T, 5>(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W, st);
    default: return launch_ks<T, 7>(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W, st);
  }
}

}  // namespace

bool block_fused_supported(int H, int W, int C, int heads, int ks, int dil, na2d_dtype_t dt) {
  return (dt == NA2D_DTYPE_BF16 || dt == NA2D_DTYPE_F16) && C == kC && heads == 2 &&
         (ks == 3 || ks == 5 || ks == 7) && dil == 1 && H >= ks && W >= ks &&
         (int64_t)H * W <= kMaxPlanePixels;
}

hipError_t launch_block_fused(const void *x, const void *w_qkv, const void *b_qkv,
                              const void *rpb, const void *w_out, const void *b_out, void *y,
                              int B, int H, int W, int ks, na2d_dtype_t dt, hipStream_t st) {
  if (dt == NA2D_DTYPE_BF16)
    return launch_dtype<__bf16>(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W, ks, st);
  return launch_dtype<_Float16>(x, w_qkv, b_qkv, rpb, w_out, b_out, y, B, H, W, ks, st);
}

}  // namespace na2d
