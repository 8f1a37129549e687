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
//   * A block is an RY x RX rectangle of queries of one class of one (batch,
//     head) plane.  Its halo -- the union of its queries' clamped windows, at
//     most (RY+k-1) x (RX+k-1) sub-grid pixels -- is copied to LDS by the
//     direct global->LDS path (global_load_lds_dwordx4): K and V both as
//     [row][column] 64-byte pixels, 16-byte chunks XOR-swizzled by column
//     against bank conflicts.  Rows/columns past the halo hold clamped real
//     pixels, so every LDS read is in bounds and finite without clamping.
//   * Workgroups are persistent, one wave per 16-query tile of a block.  A
//     workgroup walks a contiguous run of blocks (neighbouring blocks share
//     halo rows in the same L2) with two LDS buffers: while it computes block
//     i from one buffer, the DMA fills the other with block i+1.
//   * Per tile (TY x TX queries): the keys are NB = TY + k - 1 halo rows x 16
//     columns.  Scores are produced transposed, S^T = K . Q^T (one
//     v_mfma_f32_16x16x32 per key row), so each lane holds scores of ONE
//     query: the softmax max needs two lane swaps and the 16-bit
//     probabilities are already the B operand of out^T = V^T . P^T.  The V^T
//     operand is read from row-major V with ds_read_b64_tr_b16: a 16-lane
//     group reads 4 pixels x 16 channels and each lane receives one channel
//     of those 4 pixels.  A product against an all-ones matrix yields the
//     softmax denominator over exactly the 16-bit weights used.
//   * The relative-position bias (times sqrt(D)) and the window mask (-inf
//     outside the query's clamped window) enter as the accumulator input of
//     the score MFMA; for tiles whose windows are all unclamped it is a fixed
//     per-lane pattern read from a small padded table.
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Block and tile geometry per kernel size.  A tile's 16 key columns cover
// its TX queries' windows: TX + k - 1 <= 16.
template <int KS> struct Geometry {
  static constexpr int TY = KS <= 9 ? 2 : 4;                   // tile rows
  static constexpr int TX = 16 / TY;                           // tile columns
  static constexpr int RY = KS <= 7 ? 28 : (KS == 9 ? 20 : (KS == 11 ? 16 : 12));
  static constexpr int RX = 8;
  static constexpr int NTY = RY / TY, NTX = RX / TX;
  static constexpr int NTILE = NTY * NTX;  // one wave per tile
  static constexpr int THREADS = NTILE * 64;
  static constexpr int NB = TY + KS - 1;                       // key rows per tile
  static constexpr int HRM = RY + KS - 1;                      // halo rows (max)
  static constexpr int ROWS = HRM + TY;                        // staged rows
  static constexpr int HCM = RX + KS - 1 > 16 ? RX + KS - 1 : 16;  // staged columns
  static constexpr int PIX = ROWS * HCM;                       // staged pixels
  static constexpr int SIDE = 2 * KS - 1;
  static constexpr int MARGIN = TY * SIDE + 32;  // keeps masked bias reads in bounds
  // LDS tables, one set per buffer.  First the interior accumulator table:
  // entry (u, w), u = key row - query row within the tile's key block
  // (-(TY-1)..NB-1), w = key column - query column (-TX..15), at
  // (u + TY-1) * IW + w + TX, holds bias * sqrt(D) inside the k x k window and
  // -inf outside.  Then the bias table (times sqrt(D)) with zero margins; its
  // entry (0, 0) sits at BOFF.  The interior table starts at offset 0 so that
  // a lane's reads of it fit the immediate offsets of one base address.
  static constexpr int IU = NB + TY - 1, IW = 16 + TX;
  static constexpr int NINT = IU * IW;
  static constexpr int BOFF = NINT + MARGIN;
  static constexpr int NTAB = NINT + SIDE * SIDE + 2 * MARGIN;
  static_assert(TX + KS - 1 <= 16, "key columns do not cover the tile");
  static_assert(NB % 2 == 0, "PV consumes key rows in pairs");
  static_assert(RY % TY == 0 && RX % TX == 0, "blocks hold whole tiles");
  static_assert((2 * PIX * 128 + 2 * NTAB * 4) <= 160 * 1024, "LDS");
};

// Per-block coordinates (all workgroup-uniform).
struct Block {
  int64_t plane;
  int h, Ly, Lx, rc0, rc1, cc0, cc1, hy0, hx0, HR, cmax;
  int org;  // in-plane pixel index of the class origin (ry, rx)
  bool valid;
};

// Block ids enumerate (plane, ry, by, bx, rx) with rx fastest.  A workgroup
// visits consecutive ids, so it keeps the mixed-radix digits and steps them.
struct BlockCursor {
  int64_t plane;
  int h, ry, by, bx, rx;
};

__device__ __forceinline__ BlockCursor cursor_at(uint32_t id, int dil, const FastDiv &fdil,
                                                 const FastDiv &fnbx, const FastDiv &fnby,
                                                 const FastDiv &fheads) {
  BlockCursor c;
  uint32_t t = fast_div(id, fdil);
  c.rx = id - t * dil;
  id = t;
  t = fast_div(id, fnbx);
  c.bx = id - t * fnbx.div;
  id = t;
  t = fast_div(id, fnby);
  c.by = id - t * fnby.div;
  id = t;
  t = fast_div(id, fdil);
  c.ry = id - t * dil;
  c.plane = t;
  c.h = (int)(t - fast_div(t, fheads) * fheads.div);
  return c;
}

__device__ __forceinline__ void cursor_step(BlockCursor &c, int dil, int nbx, int nby, int heads) {
  if (++c.rx < dil) return;
  c.rx = 0;
  if (++c.bx < nbx) return;
  c.bx = 0;
  if (++c.by < nby) return;
  c.by = 0;
  if (++c.ry < dil) return;
  c.ry = 0;
  ++c.plane;
  if (++c.h == heads) c.h = 0;
}

template <int KS>
__device__ __forceinline__ Block block_of(const BlockCursor &c, const Shape &s,
                                          const FastDiv &fdil) {
  using G = Geometry<KS>;
  Block b;
  b.plane = c.plane;
  b.h = c.h;
  b.org = c.ry * s.W + c.rx;
  // class_len(n, r, d) = (n - r + d - 1) / d
  b.Ly = fast_div((uint32_t)(s.H - c.ry + s.dil - 1), fdil);
  b.Lx = fast_div((uint32_t)(s.W - c.rx + s.dil - 1), fdil);
  b.rc0 = c.by * G::RY;
  b.cc0 = c.bx * G::RX;
  b.valid = b.rc0 < b.Ly && b.cc0 < b.Lx;
  b.rc1 = min(b.rc0 + G::RY, b.Ly);
  b.cc1 = min(b.cc0 + G::RX, b.Lx);
  b.hy0 = window_start(b.rc0, b.Ly, KS);
  b.HR = window_start(b.rc1 - 1, b.Ly, KS) + KS - b.hy0;
  b.hx0 = window_start(b.cc0, b.Lx, KS);
  b.cmax = b.Lx - 1 - b.hx0;
  return b;
}

// Copy a block's K and V halo into one LDS buffer with the direct
// global->LDS path: 16 bytes per lane, lane i of an instruction lands at
// base + 16*i, so each instruction fills 64 consecutive 16-byte slots.  Slot
// (pixel, p) of the buffer holds logical chunk p ^ swz(column) of the pixel.
template <typename T, int KS>
__device__ __forceinline__ void stage_block(const T *__restrict__ k, const T *__restrict__ v,
                                            const Block &b, const Shape &s, int64_t pstride,
                                            char *kbuf, char *vbuf, int wave, int lane) {
  using G = Geometry<KS>;
  constexpr int NI = (G::PIX * 4 + 63) / 64;  // instructions per tensor (last one partial)
  constexpr int NW = G::NTILE;
  constexpr unsigned PB = kHeadDim * sizeof(T);  // bytes per pixel
  // halo origin, as a byte offset within the plane (planes are < 2^24 pixels)
  const unsigned org = (unsigned)(b.org + b.hy0 * s.dil * s.W + b.hx0 * s.dil) * PB;
  const char *kb0 = (const char *)(k + b.plane * pstride) + org;
  const char *vb0 = (const char *)(v + b.plane * pstride) + org;
  const unsigned rowb = (unsigned)s.dil * (unsigned)s.W * PB;
  const unsigned colb = (unsigned)s.dil * PB;
  if constexpr (G::HCM == 16) {
    // one instruction = one staged row of one tensor: the column / chunk part
    // of the address is fixed per lane, the row part is uniform and shared by
    // the K and V copies of the row
    const int col = lane >> 2, lch = (lane & 3) ^ ((col >> 1) & 3);
    const unsigned coff = (unsigned)min(col, b.cmax) * colb + lch * 16;
#pragma unroll
    for (int j = 0; j < (G::ROWS + NW - 1) / NW; ++j) {
      const int row = wave + j * NW;
      if (row < G::ROWS) {
        const unsigned roff = (unsigned)min(row, b.HR - 1) * rowb;
        __builtin_amdgcn_global_load_lds((const void *)(kb0 + (roff + coff)),
                                         (lds_void *)(kbuf + row * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(vb0 + (roff + coff)),
                                         (lds_void *)(vbuf + row * 1024), 16, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < (2 * NI + NW - 1) / NW; ++j) {
      const int ins = wave + j * NW;
      if (ins < 2 * NI) {
        const bool isv = ins >= NI;
        const int slot = (isv ? ins - NI : ins) * 64 + lane;
        const int pix = slot >> 2, pch = slot & 3;
        const int row = pix / G::HCM, col = pix - row * G::HCM;
        const int lch = pch ^ ((col >> 1) & 3);
        const unsigned off = (unsigned)min(row, b.HR - 1) * rowb +
                             (unsigned)min(col, b.cmax) * colb + lch * 16;
        char *dst = (isv ? vbuf : kbuf) + (slot - lane) * 16;
        if (pix < G::PIX)
          __builtin_amdgcn_global_load_lds((const void *)((isv ? vb0 : kb0) + off),
                                           (lds_void *)dst, 16, 0, 0);
      }
    }
  }
}

// Table entries (interior table, then bias table with zero margins) this
// thread writes: entry index into rpb, or -1 for a zero margin, -2 for -inf.
template <int KS>
__device__ __forceinline__ int table_index(int e) {
  using G = Geometry<KS>;
  constexpr int R = KS / 2;
  if (e >= G::NINT) {
    const int t = e - G::BOFF;
    return (t >= 0 && t < G::SIDE * G::SIDE) ? t : -1;
  }
  const int u = e / G::IW - (G::TY - 1), w = e % G::IW - G::TX;
  return ((unsigned)u < (unsigned)KS && (unsigned)w < (unsigned)KS) ? (u + R) * G::SIDE + w + R
                                                                    : -2;
}

template <int KS> struct TableRegs {
  static constexpr int N = (Geometry<KS>::NTAB + Geometry<KS>::THREADS - 1) / Geometry<KS>::THREADS;
};

// Raw rpb values of this thread's entries for head h (loads are unconditional
// -- margin entries read entry 0 -- so they never need an early wait).
template <typename T, int KS>
__device__ __forceinline__ void load_tables(const T *__restrict__ rpb, int h, int tid,
                                            T (&reg)[TableRegs<KS>::N]) {
  using G = Geometry<KS>;
  if (rpb == nullptr) return;
#pragma unroll
  for (int it = 0; it < TableRegs<KS>::N; ++it) {
    const int e = min(tid + it * G::THREADS, G::NTAB - 1);
    const int idx = max(table_index<KS>(e), 0);
    reg[it] = rpb[(int64_t)h * G::SIDE * G::SIDE + idx];
  }
}

template <typename T, int KS>
__device__ __forceinline__ void store_tables(float *tab, int tid, bool has_rpb,
                                             const T (&reg)[TableRegs<KS>::N]) {
  using G = Geometry<KS>;
#pragma unroll
  for (int it = 0; it < TableRegs<KS>::N; ++it) {
    const int e = tid + it * G::THREADS;
    if (e < G::NTAB) {
      const int idx = table_index<KS>(e);
      float x = idx == -2 ? -INFINITY : 0.f;
      if (idx >= 0 && has_rpb) x = Elem<T>::to_f(reg[it]) * kSqrtD;
      tab[e] = x;
    }
  }
}

// In-plane pixel index of this lane's query in block b: block row lr, block
// column lc, clamped into a ragged block (such lanes recompute a real query
// and store nothing).  Planes hold fewer than 2^24 pixels, so 24-bit
// multiplies suffice.
__device__ __forceinline__ int query_pixel(const Block &b, const Shape &s, int lr, int lc) {
  const int ci = b.rc0 + min(lr, b.rc1 - 1 - b.rc0);
  const int cj = b.cc0 + min(lc, b.cc1 - 1 - b.cc0);
  return b.org + (int)__umul24((unsigned)ci, (unsigned)(s.dil * s.W)) +
         (int)__umul24((unsigned)cj, (unsigned)s.dil);
}

// The 16-byte Q slice (channels 8g..8g+7) of the query at pixel pix.
template <typename T>
__device__ __forceinline__ u32x4 load_q(const T *__restrict__ q, const Block &b, int64_t pstride,
                                        int pix, int g) {
  const char *qp = (const char *)(q + b.plane * pstride);
  return *(const u32x4 *)(qp + ((unsigned)pix * (unsigned)(kHeadDim * sizeof(T)) + g * 16u));
}

// One 16-query tile of block b (this wave's), from one LDS buffer.
// One 16-query tile of block b (this wave's), from one LDS buffer; the
// query of this lane sits at in-plane pixel pix.
template <typename T, int KS>
__device__ __forceinline__ void compute_tile(T *__restrict__ out, const Block &b, const Shape &s,
                                             int64_t pstride, int pix, const char *kbuf,
                                             const char *vbuf, const float *tab, u32x4 qraw,
                                             int wave, int lane) {
  using G = Geometry<KS>;
  using vec = typename Mma<T>::vec;
  constexpr int TY = G::TY, TX = G::TX, NB = G::NB, SIDE = G::SIDE, HCM = G::HCM;
  constexpr int R = KS / 2;
  const int ql = lane & 15, g = lane >> 4;
  const int qy = ql / TX, qx = ql % TX;
  const int ty = wave / G::NTX, tx = wave % G::NTX;
  const int tci0 = b.rc0 + ty * TY, tcj0 = b.cc0 + tx * TX;
  if (tci0 >= b.rc1 || tcj0 >= b.cc1) return;  // tile outside a ragged block
  const int Y0 = window_start(tci0, b.Ly, KS), X0 = window_start(tcj0, b.Lx, KS);
  const int lrow0 = Y0 - b.hy0, lcol0 = X0 - b.hx0;
  const vec qv = __builtin_bit_cast(vec, qraw);
  const float c2 = kLog2e / kSqrtD;  // exp(S - Smax) = exp2((acc - accmax) * c2)

  // S^T rows: key (Y0 + a, X0 + 4g + i) against query ql, i = 0..3.
  const int kcol = lcol0 + ql;
  const u32x4 *kb =
      (const u32x4 *)(kbuf + (lrow0 * HCM + kcol) * 64) + (g ^ ((kcol >> 1) & 3));
  f32x4 sc[NB];
  const bool interior = tci0 - R >= 0 && tci0 + TY - 1 + R <= b.Ly - 1 && tcj0 - R >= 0 &&
                        tcj0 + TX - 1 + R <= b.Lx - 1;
  if (interior) {
    const float *tb = tab + (TY - 1 - qy) * G::IW + (TX + 4 * g - qx);
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      f32x4 c;
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = tb[a * G::IW + i];
      sc[a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * HCM * 4]), qv, c);
    }
  } else {
    // The query's window starts sy, sx lie TY-1 resp. TX-1 at most past the
    // tile's Y0, X0, so key rows TY-1..k-1 of the key block are inside every
    // lane's row window: only the first and last TY-1 rows need a row test.
    const int ci = min(tci0 + qy, b.rc1 - 1), cj = min(tcj0 + qx, b.cc1 - 1);
    const int sy = window_start(ci, b.Ly, KS), sx = window_start(cj, b.Lx, KS);
    const int rowrel = Y0 - sy, colrel = X0 + 4 * g - sx;
    int bidx = G::BOFF + (Y0 - ci + KS - 1) * SIDE + (X0 + 4 * g - cj + KS - 1);
    asm volatile("" : "+v"(bidx));  // one base register; the reads use immediate offsets
    const float *bb = tab + bidx;
    // +inf inside the window, -inf outside; hidden from the optimiser so that
    // each entry costs one min and the table reads stay unconditional
    float ccap[4];
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
      f32x4 c;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c[i] = rtest ? fminf(fminf(bb[a * SIDE + i], ccap[i]), rcap)
                     : fminf(bb[a * SIDE + i], ccap[i]);
      sc[a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * HCM * 4]), qv, c);
    }
  }

  // softmax over the query's k*k keys: the 4 lane groups hold disjoint keys
  float mx = -INFINITY;
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[a][i]);
  mx = group_max(mx);
  const float mc = mx * c2;
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[a][i] = __builtin_amdgcn_exp2f(fmaf(sc[a][i], c2, -mc));

  // out^T = V^T . P^T over pairs of key rows (32 keys per MFMA).  As a source
  // of the transposing read, lane (g, 4k + qd) reads channels 4qd..4qd+3
  // (+16 for the second channel block) of key column X0 + 4g + k.
  const int vcol = lcol0 + 4 * g + (ql >> 2), qd = ql & 3, vs = (vcol >> 1) & 3;
  const char *vrow = vbuf + (lrow0 * HCM + vcol) * 64 + 8 * (qd & 1);
  const char *va0 = vrow + 16 * ((qd >> 1) ^ vs);
  const char *va1 = vrow + 16 * (((qd >> 1) | 2) ^ vs);
  vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f}, o2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NB / 2; ++j) {
    vec pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = static_cast<T>(sc[2 * j][i]);
      pb[4 + i] = static_cast<T>(sc[2 * j + 1][i]);
    }
    constexpr int RB = HCM * 64;  // bytes per staged row
    const u32x2 a0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va0 + (2 * j) * RB)));
    const u32x2 a1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va0 + (2 * j + 1) * RB)));
    const u32x2 b0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va1 + (2 * j) * RB)));
    const u32x2 b1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va1 + (2 * j + 1) * RB)));
    const u32x4 w0 = {a0[0], a0[1], a1[0], a1[1]};
    const u32x4 w1 = {b0[0], b0[1], b1[0], b1[1]};
    o0 = Mma<T>::run(__builtin_bit_cast(vec, w0), pb, o0);
    o1 = Mma<T>::run(__builtin_bit_cast(vec, w1), pb, o1);
    o2 = Mma<T>::run(ones, pb, o2);
  }

  // lane holds channels 4g..4g+3 (o0) and 16+4g..16+4g+3 (o1) of query ql
  if (tci0 + qy < b.rc1 && tcj0 + qx < b.cc1) {
    const float inv = __builtin_amdgcn_rcpf(o2[0]);
    typedef __attribute__((ext_vector_type(4))) T vec4;
    vec4 r0, r1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r0[i] = static_cast<T>(o0[i] * inv);
      r1[i] = static_cast<T>(o1[i] * inv);
    }
    char *o = (char *)(out + b.plane * pstride) +
              ((unsigned)pix * (unsigned)(kHeadDim * sizeof(T)) + g * 8u);
    *(u32x2 *)o = __builtin_bit_cast(u32x2, r0);
    *(u32x2 *)(o + 16 * sizeof(T)) = __builtin_bit_cast(u32x2, r1);
  }
}

template <typename T, int KS>
__global__ __launch_bounds__(Geometry<KS>::THREADS) void fused_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, Shape s, FastDiv fdil, FastDiv fnbx,
    FastDiv fnby, FastDiv fheads, int nblocks) {
  using G = Geometry<KS>;
  __shared__ __attribute__((aligned(16))) char kbuf0[G::PIX * 64], vbuf0[G::PIX * 64];
  __shared__ __attribute__((aligned(16))) char kbuf1[G::PIX * 64], vbuf1[G::PIX * 64];
  __shared__ float tab0[G::NTAB], tab1[G::NTAB];

  // wave index is uniform within a wave: keep it (and all that derives from
  // it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  // this workgroup's contiguous run of blocks
  const int wg = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int b0 = (int)((int64_t)nblocks * wg / gridDim.x);
  const int b1 = (int)((int64_t)nblocks * (wg + 1) / gridDim.x);
  if (b0 >= b1) return;
  const bool has_rpb = rpb != nullptr;
  const int64_t pstride = (int64_t)s.H * s.W * kHeadDim;  // elements per plane
  // this lane's query position within a block
  const int lr = (wave / G::NTX) * G::TY + ql / G::TX, lc = (wave % G::NTX) * G::TX + ql % G::TX;

  // Prefetch order for block n+1 while block n computes: its Q slice (and,
  // when the head changes, its bias-table values) first, then the K/V DMA;
  // nothing consumes them before the end-of-block barrier, so the loads
  // overlap the whole compute of block n.
  T treg[TableRegs<KS>::N];
  BlockCursor cc = cursor_at(b0, s.dil, fdil, fnbx, fnby, fheads);
  Block cur = block_of<KS>(cc, s, fdil);
  int pcur = query_pixel(cur, s, lr, lc);
  u32x4 qcur = load_q<T>(q, cur, pstride, pcur, g);
  load_tables<T, KS>(rpb, cur.h, tid, treg);
  if (cur.valid) stage_block<T, KS>(k, v, cur, s, pstride, kbuf0, vbuf0, wave, lane);
  store_tables<T, KS>(tab0, tid, has_rpb, treg);
  int tab_h0 = cur.h, tab_h1 = -1;  // head whose tables each buffer holds
  __syncthreads();
  const int nbx = fnbx.div, nby = fnby.div;

  // Two blocks per iteration so that each buffer is a fixed LDS array.
  for (int bi = b0; bi < b1; bi += 2) {
    {  // block bi from buffer 0; block bi+1 into buffer 1
      const bool more = bi + 1 < b1;
      if (more) cursor_step(cc, s.dil, nbx, nby, s.heads);
      const Block nxt = block_of<KS>(cc, s, fdil);
      const int pnxt = query_pixel(nxt, s, lr, lc);
      const u32x4 qnxt = load_q<T>(q, nxt, pstride, pnxt, g);
      const bool newtab = more && nxt.h != tab_h1;
      if (newtab) load_tables<T, KS>(rpb, nxt.h, tid, treg);
      if (more && nxt.valid) stage_block<T, KS>(k, v, nxt, s, pstride, kbuf1, vbuf1, wave, lane);
      if (cur.valid)
        compute_tile<T, KS>(out, cur, s, pstride, pcur, kbuf0, vbuf0, tab0, qcur, wave, lane);
      if (!more) break;
      if (newtab) {
        store_tables<T, KS>(tab1, tid, has_rpb, treg);
        tab_h1 = nxt.h;
      }
      __syncthreads();  // also waits for the DMA (workgroup fence)
      cur = nxt;
      pcur = pnxt;
      qcur = qnxt;
    }
    {  // block bi+1 from buffer 1; block bi+2 into buffer 0
      const bool more = bi + 2 < b1;
      if (more) cursor_step(cc, s.dil, nbx, nby, s.heads);
      const Block nxt = block_of<KS>(cc, s, fdil);
      const int pnxt = query_pixel(nxt, s, lr, lc);
      const u32x4 qnxt = load_q<T>(q, nxt, pstride, pnxt, g);
      const bool newtab = more && nxt.h != tab_h0;
      if (newtab) load_tables<T, KS>(rpb, nxt.h, tid, treg);
      if (more && nxt.valid) stage_block<T, KS>(k, v, nxt, s, pstride, kbuf0, vbuf0, wave, lane);
      if (cur.valid)
        compute_tile<T, KS>(out, cur, s, pstride, pcur, kbuf1, vbuf1, tab1, qcur, wave, lane);
      if (!more) break;
      if (newtab) {
        store_tables<T, KS>(tab0, tid, has_rpb, treg);
        tab_h0 = nxt.h;
      }
      __syncthreads();
      cur = nxt;
      pcur = pnxt;
      qcur = qnxt;
    }
  }
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <typename T, int KS>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *rpb, void *out,
                    const Shape &s, hipStream_t st) {
  using G = Geometry<KS>;
  const int Lymax = class_len(s.H, 0, s.dil), Lxmax = class_len(s.W, 0, s.dil);
  const int nby = (Lymax + G::RY - 1) / G::RY, nbx = (Lxmax + G::RX - 1) / G::RX;
  const int64_t nblocks = (int64_t)s.B * s.heads * s.dil * s.dil * nby * nbx;
  if (nblocks > INT_MAX) return hipErrorInvalidConfiguration;
  // one persistent workgroup per compute unit (its LDS holds two blocks)
  const int64_t grid = nblocks < device_cus() ? nblocks : device_cus();
  fused_mfma_kernel<T, KS><<<dim3((unsigned)grid), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (T *)out, s,
      make_fastdiv((uint32_t)s.dil), make_fastdiv((uint32_t)nbx), make_fastdiv((uint32_t)nby),
      make_fastdiv((uint32_t)s.heads), (int)nblocks);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, hipStream_t st, bool *supported) {
  // in-plane offsets are 32-bit and pixel products 24-bit
  if ((int64_t)s.H * s.W >= kMaxPlanePixels) {
    *supported = false;
    return hipSuccess;
  }
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
  hipError_t e = launch_dense_mfma(q, k, v, rpb, out, s, dt, st, supported);
  if (*supported) return e;
  *supported = true;
  if (dt == NA2D_DTYPE_BF16) return launch_dtype<__bf16>(q, k, v, rpb, out, s, st, supported);
  if (dt == NA2D_DTYPE_F16) return launch_dtype<_Float16>(q, k, v, rpb, out, s, st, supported);
  *supported = false;
  return hipSuccess;
}

}  // namespace na2d
