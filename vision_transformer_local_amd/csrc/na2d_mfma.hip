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
constexpr int default_rows(int ks) { return ks <= 7 ? 32 : (ks == 9 ? 24 : 16); }

template <int KS, int RYV = default_rows(KS)> struct Geometry {
  static constexpr int TY = KS <= 9 ? 2 : 4;                   // tile rows
  static constexpr int TX = 16 / TY;                           // tile columns
  // Block rows: the waves (one per tile) come in multiples of 4, so that
  // they spread evenly over the 4 SIMDs, or 14 waves for k <= 7 where that
  // tiles the map with fewer blocks; at most what the two LDS buffers allow.
  static constexpr int RY = RYV;
  static constexpr int RX = 8;
  static constexpr int NTY = RY / TY, NTX = RX / TX;
  static constexpr int NTILE = NTY * NTX;  // one wave per tile
  static constexpr int THREADS = NTILE * 64;
  static constexpr int NB = TY + KS - 1;                       // key rows per tile
  static constexpr int HRM = RY + KS - 1;                      // halo rows (max)
  static constexpr int HCM = RX + KS - 1 > 16 ? RX + KS - 1 : 16;  // staged columns
  // A tile reads 16 key columns from its first one, at most RX - TX past the
  // block's: with HCM < RX - TX + 16 the last reads run into the next staged
  // row, so one more row keeps them inside the buffer (they only ever meet
  // masked keys).
  static constexpr int ROWS = HRM + (RX - TX + 16 > HCM ? 1 : 0);  // staged rows
  static constexpr int PIX = ROWS * HCM;                       // staged pixels
  static constexpr int SIDE = 2 * KS - 1;
  static constexpr int MARGIN = TY * SIDE + 32;  // keeps masked bias reads in bounds
  // LDS tables, one set per buffer.  First the interior accumulator table:
  // entry (u, w), u = key row - query row within the tile's key block
  // (-(TY-1)..NB-1), w = key column - query column (-TX..15), at
  // (u + TY-1) * IW + w + TX, holds bias * sqrt(D) inside the k x k window and
  // -inf outside.  Then the bias table (times sqrt(D)) with zero margins; its
  // entry (0, 0) sits at BOFF.  The interior table starts at offset 0 so that
  // a lane's reads of it fit the immediate offsets of one base address.  The
  // row pitch IW (at least 16 + TX) is chosen for the LDS banks: the lanes of
  // a read span TX + 4 consecutive entries in each of TY table rows, and a
  // pitch of 16 (TY = 2) or 8 (TY = 4) banks mod 32 keeps those row ranges
  // on distinct banks (TY = 2) or overlapping in one bank (TY = 4).
  static constexpr int IU = NB + TY - 1, IW = TY == 2 ? 48 : 40;
  static constexpr int NINT = IU * IW;
  static constexpr int BOFF = NINT + MARGIN;
  static constexpr int NTAB = NINT + SIDE * SIDE + 2 * MARGIN;
  static_assert(TX + KS - 1 <= 16, "key columns do not cover the tile");
  static_assert(IW >= 16 + TX, "interior table rows hold the tile's key columns");
  static_assert(NB % 2 == 0, "PV consumes key rows in pairs");
  static_assert(RY % TY == 0 && RX % TX == 0, "blocks hold whole tiles");
  static_assert(THREADS <= 1024, "one workgroup");
  static_assert((2 * PIX * 128 + 2 * NTAB * 4) <= 160 * 1024, "LDS");
};

// Block ids enumerate (batch, head, ry, by, bx, rx) with rx fastest.  A
// workgroup keeps the mixed-radix digits and steps them.  Without dilation it
// visits a contiguous run of ids.  With dilation d the workgroups form crews
// of d (consecutive workgroup numbers, so one XCD): member rx of a crew keeps
// column class rx and the crew walks a contiguous run of the other digits in
// step.  The classes rx and rx + 1 share every 128-byte line (their 64-byte
// pixels alternate along a row), so the crew's members request each line
// within the same block time and the second request finds it in L2; and
// the next block column of a class, whose halo overlaps this one's, is the
// member's next block.  (With channels-last maps the heads of a pixel share
// its lines; making the head the fastest digit was tried and lost the halo
// reuse between neighbouring blocks: 2.6x the L2 misses.)
struct BlockCursor {
  int b, h, ry, by, bx, rx;
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
  const uint32_t bq = fast_div(t, fheads);
  c.b = (int)bq;
  c.h = (int)(t - bq * fheads.div);
  return c;
}

// Steps to the next id (with fixrx, to the next id of the same column class
// rx); true when the row part (batch, head, ry, by) changed.
__device__ __forceinline__ bool cursor_step(BlockCursor &c, int dil, int nbx, int nby, int heads,
                                            bool fixrx) {
  if (!fixrx) {
    if (++c.rx < dil) return false;
    c.rx = 0;
  }
  if (++c.bx < nbx) return false;
  c.bx = 0;
  if (++c.by < nby) return true;
  c.by = 0;
  if (++c.ry < dil) return true;
  c.ry = 0;
  if (++c.h == heads) {
    c.h = 0;
    ++c.b;
  }
  return true;
}

// A block splits into a row part, which depends on (plane, ry, by) only and
// is recomputed when those change, and a column part, which depends on
// (rx, bx).  Both include what this wave's tile and this lane's query need.
// Byte offsets within a plane fit 32 bits.
struct RowPart {
  int64_t pofs;    // byte offset of the (batch, head) plane of q, k, v
  int64_t opofs;   // the same for out
  int h, Ly, rc0, rc1, hy0, HR;
  int tci0, Y0;    // first query row of this wave's tile; first key row of its key block
  unsigned hrow;   // byte offset of the first halo row: (ry + hy0*d) * row stride
  int ry;
  int ok, inner;   // block row exists; the tile's windows are unclamped in y
};

struct ColPart {
  int Lx, cc0, cc1, hx0, cmax;
  int tcj0, X0;
  unsigned hcol;   // byte offset of the first halo column: (rx + hx0*d) * column stride
  int rx;
  int ok, inner;
};

template <typename T, int KS, int RY>
__device__ __forceinline__ RowPart row_part(const BlockCursor &c, const Shape &s,
                                            const FastDiv &fdil, const ByteStrides &si,
                                            const ByteStrides &so, int ty, int lr) {
  using G = Geometry<KS, RY>;
  constexpr int R = KS / 2;
  RowPart r;
  r.pofs = c.b * si.b + c.h * si.h;
  r.opofs = c.b * so.b + c.h * so.h;
  r.h = c.h;
  // class_len(n, r, d) = (n - r + d - 1) / d
  r.Ly = fast_div((uint32_t)(s.H - c.ry + s.dil - 1), fdil);
  r.rc0 = c.by * G::RY;
  r.ok = r.rc0 < r.Ly;
  r.rc1 = min(r.rc0 + G::RY, r.Ly);
  r.hy0 = window_start(r.rc0, r.Ly, KS);
  r.HR = window_start(r.rc1 - 1, r.Ly, KS) + KS - r.hy0;
  r.tci0 = r.rc0 + ty * G::TY;
  r.Y0 = window_start(r.tci0, r.Ly, KS);
  r.inner = r.tci0 >= R && r.tci0 + G::TY - 1 + R <= r.Ly - 1;
  r.hrow = (unsigned)(c.ry + r.hy0 * s.dil) * si.y;
  r.ry = c.ry;
  return r;
}

template <typename T, int KS>
__device__ __forceinline__ ColPart col_part(const BlockCursor &c, const Shape &s,
                                            const FastDiv &fdil, const ByteStrides &si, int tx,
                                            int lc) {
  using G = Geometry<KS>;
  constexpr int R = KS / 2;
  ColPart q;
  q.Lx = fast_div((uint32_t)(s.W - c.rx + s.dil - 1), fdil);
  q.cc0 = c.bx * G::RX;
  q.ok = q.cc0 < q.Lx;
  q.cc1 = min(q.cc0 + G::RX, q.Lx);
  q.hx0 = window_start(q.cc0, q.Lx, KS);
  q.cmax = q.Lx - 1 - q.hx0;
  q.tcj0 = q.cc0 + tx * G::TX;
  q.X0 = window_start(q.tcj0, q.Lx, KS);
  q.inner = q.tcj0 >= R && q.tcj0 + G::TX - 1 + R <= q.Lx - 1;
  q.hcol = (unsigned)(c.rx + q.hx0 * s.dil) * si.x;
  q.rx = c.rx;
  return q;
}

// In-plane byte offsets of this lane's query (block row lr, block column
// lc) in q and in out, clamped into a ragged block: such lanes recompute a
// real query and store nothing.
struct QueryOffs {
  unsigned q, o;
};

__device__ __forceinline__ QueryOffs query_offsets(const RowPart &r, const ColPart &c,
                                                   const Shape &s, const ByteStrides &si,
                                                   const ByteStrides &so, int lr, int lc) {
  const int ci = r.rc0 + min(lr, r.rc1 - 1 - r.rc0);
  const int cj = c.cc0 + min(lc, c.cc1 - 1 - c.cc0);
  const unsigned row = r.ry + __umul24((unsigned)ci, (unsigned)s.dil);
  const unsigned col = c.rx + __umul24((unsigned)cj, (unsigned)s.dil);
  // row < 2^24 pixels and strides < 2^24 bytes (checked on the host)
  return QueryOffs{(unsigned)__umul24(row, si.y) + (unsigned)__umul24(col, si.x),
                   (unsigned)__umul24(row, so.y) + (unsigned)__umul24(col, so.x)};
}

// Copy a block's K and V halo into one LDS buffer with the direct
// global->LDS path: 16 bytes per lane, lane i of an instruction lands at
// base + 16*i, so each instruction fills 64 consecutive 16-byte slots.  Slot
// (pixel, p) of the buffer holds logical chunk p ^ swz(column) of the pixel.
template <typename T, int KS, int RY, bool WITH_V = true>
__device__ __forceinline__ void stage_block(const T *__restrict__ k, const T *__restrict__ v,
                                            const RowPart &r, const ColPart &c, const Shape &s,
                                            const ByteStrides &si, char *kbuf, char *vbuf,
                                            int wave, int lane) {
  using G = Geometry<KS, RY>;
  constexpr int NI = (G::PIX * 4 + 63) / 64;  // instructions per tensor (last one partial)
  constexpr int NW = G::NTILE;
  const unsigned org = r.hrow + c.hcol;  // halo origin within the plane
  const char *kb0 = ((const char *)k + r.pofs) + org;
  const char *vb0 = ((const char *)v + r.pofs) + org;
  const unsigned rowb = (unsigned)s.dil * si.y;
  const unsigned colb = (unsigned)s.dil * si.x;
  if constexpr (G::HCM == 16) {
    // one instruction = one staged row of one tensor: the column / chunk part
    // of the address is fixed per lane, the row part is uniform and shared by
    // the K and V copies of the row
    const int col = lane >> 2, lch = (lane & 3) ^ ((col >> 1) & 3);
    unsigned coff = (unsigned)min(col, c.cmax) * colb + lch * 16;
    asm volatile("" : "+v"(coff));  // keep the row part a scalar base, not refactored
#pragma unroll
    for (int j = 0; j < (G::ROWS + NW - 1) / NW; ++j) {
      const int row = wave + j * NW;
      if (row < G::ROWS) {
        const unsigned roff = (unsigned)min(row, r.HR - 1) * rowb;
        __builtin_amdgcn_global_load_lds((const void *)((kb0 + roff) + coff),
                                         (lds_void *)(kbuf + row * 1024), 16, 0, 0);
        if constexpr (WITH_V)
          __builtin_amdgcn_global_load_lds((const void *)((vb0 + roff) + coff),
                                           (lds_void *)(vbuf + row * 1024), 16, 0, 0);
      }
    }
  } else {
    constexpr int NT = WITH_V ? 2 * NI : NI;  // copies (K, then V)
#pragma unroll
    for (int j = 0; j < (NT + NW - 1) / NW; ++j) {
      const int ins = wave + j * NW;
      if (ins < NT) {
        const bool isv = ins >= NI;
        const int slot = (isv ? ins - NI : ins) * 64 + lane;
        const int pix = slot >> 2, pch = slot & 3;
        const int row = pix / G::HCM, col = pix - row * G::HCM;
        const int lch = pch ^ ((col >> 1) & 3);
        const unsigned off = (unsigned)min(row, r.HR - 1) * rowb +
                             (unsigned)min(col, c.cmax) * colb + lch * 16;
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

template <int KS, int RY> struct TableRegs {
  static constexpr int N =
      (Geometry<KS, RY>::NTAB + Geometry<KS, RY>::THREADS - 1) / Geometry<KS, RY>::THREADS;
};

// Raw rpb values of this thread's entries for head h (loads are unconditional
// -- margin entries read entry 0 -- so they never need an early wait).
template <typename T, int KS, int RY>
__device__ __forceinline__ void load_tables(const T *__restrict__ rpb, int h, int tid,
                                            T (&reg)[TableRegs<KS, RY>::N]) {
  using G = Geometry<KS, RY>;
  if (rpb == nullptr) return;
#pragma unroll
  for (int it = 0; it < TableRegs<KS, RY>::N; ++it) {
    const int e = min(tid + it * G::THREADS, G::NTAB - 1);
    const int idx = max(table_index<KS>(e), 0);
    reg[it] = rpb[(int64_t)h * G::SIDE * G::SIDE + idx];
  }
}

template <typename T, int KS, int RY>
__device__ __forceinline__ void store_tables(float *tab, int tid, bool has_rpb,
                                             const T (&reg)[TableRegs<KS, RY>::N]) {
  using G = Geometry<KS, RY>;
#pragma unroll
  for (int it = 0; it < TableRegs<KS, RY>::N; ++it) {
    const int e = tid + it * G::THREADS;
    if (e < G::NTAB) {
      const int idx = table_index<KS>(e);
      float x = idx == -2 ? -INFINITY : 0.f;
      if (idx >= 0 && has_rpb) x = Elem<T>::to_f(reg[it]) * kSqrtD;
      tab[e] = x;
    }
  }
}

// The 16-byte Q slice (channels 8g..8g+7) of the query at in-plane byte
// offset off.
// Without dilation Q is read once and out written once, in whole cache
// lines: both then bypass cache retention (non-temporal), leaving the caches
// to the K/V halo rows that neighbouring blocks share.  With dilation the
// classes rx and rx + 1, visited one after the other, share the lines.
template <typename T, bool STREAM>
__device__ __forceinline__ u32x4 load_q(const T *__restrict__ q, int64_t pofs, unsigned off,
                                        int g) {
  const u32x4 *p = (const u32x4 *)(((const char *)q + pofs) + (off + g * 16u));
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  return *p;
}

// A lane's share of a tile's output: channels 4g..4g+3 and 16+4g..16+4g+3
// of its query, rounded; ok is false for queries outside a ragged block;
// lse: the query's log-sum-exp (when requested).
struct TileOut {
  u32x4 val;
  bool ok;
  float lse;
};

// Unnormalised softmax weights over the query's k*k keys, in place (the 4
// lane groups hold disjoint keys; the denominator comes from the PV step).
// Returns the reference mc the weights are taken against.
template <int KS>
__device__ __forceinline__ float softmax_weights(f32x4 (&sc)[Geometry<KS>::NB]) {
  constexpr int NB = Geometry<KS>::NB;
  const float c2 = kLog2e / kSqrtD;  // exp(S - Smax) = exp2((acc - accmax) * c2)
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
  return mc;
}

// 16-bit P^T operand of key rows 2j and 2j+1.
template <typename T>
__device__ __forceinline__ typename Mma<T>::vec p_operand(const f32x4 &s0, const f32x4 &s1) {
  typename Mma<T>::vec pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pb[i] = static_cast<T>(s0[i]);
    pb[4 + i] = static_cast<T>(s1[i]);
  }
  return pb;
}

// Accumulators of one tile's PV product: channels 4g.. (o0) and 16+4g..
// (o1) of query ql, and the softmax denominator (o2, a product with ones).
struct PVAcc {
  f32x4 o0, o1, o2;
};

template <typename T>
__device__ __forceinline__ void pv_step(PVAcc &acc, typename Mma<T>::vec w0,
                                        typename Mma<T>::vec w1, typename Mma<T>::vec p) {
  typename Mma<T>::vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);
  acc.o0 = Mma<T>::run(w0, p, acc.o0);
  acc.o1 = Mma<T>::run(w1, p, acc.o1);
  acc.o2 = Mma<T>::run(ones, p, acc.o2);
}

template <typename T>
__device__ __forceinline__ TileOut finish(const PVAcc &acc, bool ok, float lse) {
  const float inv = __builtin_amdgcn_rcpf(acc.o2[0]);
  typedef __attribute__((ext_vector_type(4))) T vec4;
  vec4 r0, r1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r0[i] = static_cast<T>(acc.o0[i] * inv);
    r1[i] = static_cast<T>(acc.o1[i] * inv);
  }
  const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
  return TileOut{{w0[0], w0[1], w1[0], w1[1]}, ok, lse};
}

// What a launch of the general kernel computes.
enum Mode { kForward = 0, kForwardLse = 1, kScores = 2 };

constexpr float kInvSqrtD = 0.17677669529663687f;  // 1 / sqrt(32)

// One 16-query tile of a block (this wave's), from one LDS buffer.
// kForwardLse: also the query's log-sum-exp.  kScores: only the scores
// q.k / sqrt(D) + bias of the window, written to scores ([.., k*k] fp32,
// dense query order; qbase = the plane's first query) through this wave's
// LDS area stage (16 k*k floats); nothing is returned.
template <typename T, int KS, int MODE>
__device__ __forceinline__ TileOut compute_tile(const RowPart &r, const ColPart &c,
                                                const char *kbuf, const char *vbuf,
                                                const float *tab, u32x4 qraw, int lane,
                                                float *stage = nullptr,
                                                float *__restrict__ scores = nullptr,
                                                int64_t qbase = 0, int W = 0, int dil = 1) {
  constexpr bool LSE = MODE == kForwardLse;
  using G = Geometry<KS>;
  using vec = typename Mma<T>::vec;
  constexpr int TY = G::TY, TX = G::TX, NB = G::NB, SIDE = G::SIDE, HCM = G::HCM;
  const int ql = lane & 15, g = lane >> 4;
  const int qy = ql / TX, qx = ql % TX;
  const int tci0 = r.tci0, tcj0 = c.tcj0;
  if (tci0 >= r.rc1 || tcj0 >= c.cc1) return TileOut{{0u, 0u, 0u, 0u}, false, 0.f};  // outside
  const int Y0 = r.Y0, X0 = c.X0;
  const int lrow0 = Y0 - r.hy0, lcol0 = X0 - c.hx0;
  const vec qv = __builtin_bit_cast(vec, qraw);

  // S^T rows: key (Y0 + a, X0 + 4g + i) against query ql, i = 0..3.
  const int kcol = lcol0 + ql;
  const u32x4 *kb =
      (const u32x4 *)(kbuf + (lrow0 * HCM + kcol) * 64) + (g ^ ((kcol >> 1) & 3));
  f32x4 sc[NB];
  if (r.inner && c.inner) {
    const float *tb = tab + (TY - 1 - qy) * G::IW + (TX + 4 * g - qx);
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      f32x4 cin;
#pragma unroll
      for (int i = 0; i < 4; ++i) cin[i] = tb[a * G::IW + i];
      sc[a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * HCM * 4]), qv, cin);
    }
  } else {
    // The query's window starts sy, sx lie TY-1 resp. TX-1 at most past the
    // tile's Y0, X0, so key rows TY-1..k-1 of the key block are inside every
    // lane's row window: only the first and last TY-1 rows need a row test.
    const int ci = min(tci0 + qy, r.rc1 - 1), cj = min(tcj0 + qx, c.cc1 - 1);
    const int sy = window_start(ci, r.Ly, KS), sx = window_start(cj, c.Lx, KS);
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
      f32x4 cin;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cin[i] = rtest ? fminf(fminf(bb[a * SIDE + i], ccap[i]), rcap)
                       : fminf(bb[a * SIDE + i], ccap[i]);
      sc[a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * HCM * 4]), qv, cin);
    }
  }

  if constexpr (MODE == kScores) {
    // the in-window entries to the wave's LDS rows (one per query), then
    // the 16 rows out with consecutive lanes on consecutive floats
    constexpr int KK = KS * KS;
    const int ci = min(tci0 + qy, r.rc1 - 1), cj = min(tcj0 + qx, c.cc1 - 1);
    const int sy = window_start(ci, r.Ly, KS), sx = window_start(cj, c.Lx, KS);
    float *row = stage + ql * KK;
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int wa = Y0 + a - sy;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int wc = X0 + 4 * g + i - sx;
        if ((unsigned)wa < (unsigned)KS && (unsigned)wc < (unsigned)KS)
          row[wa * KS + wc] = sc[a][i] * kInvSqrtD;
      }
    }
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < 16 * KK; e += 64) {
      const int qq = e / KK, slot = e - qq * KK;
      const int qci = tci0 + qq / TX, qcj = tcj0 + qq % TX;
      if (qci < r.rc1 && qcj < c.cc1)
        scores[(qbase + (int64_t)(r.ry + qci * dil) * W + c.rx + qcj * dil) * KK + slot] = stage[e];
    }
    __builtin_amdgcn_wave_barrier();
    return TileOut{{0u, 0u, 0u, 0u}, false, 0.f};
  }

  const float mc = softmax_weights<KS>(sc);
  float lse = 0.f;
  if constexpr (LSE) {  // the fp32 weights' sum (not the 16-bit one the output is divided by)
    float l = 0.f;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) l += sc[a][i];
    lse = window_lse(mc, group_sum(l));
  }

  // out^T = V^T . P^T over pairs of key rows (32 keys per MFMA).  As a source
  // of the transposing read, lane (g, 4k + qd) reads channels 4qd..4qd+3
  // (+16 for the second channel block) of key column X0 + 4g + k.
  const int vcol = lcol0 + 4 * g + (ql >> 2), qd = ql & 3, vs = (vcol >> 1) & 3;
  const char *vrow = vbuf + (lrow0 * G::HCM + vcol) * 64 + 8 * (qd & 1);
  const char *va0 = vrow + 16 * ((qd >> 1) ^ vs);
  const char *va1 = vrow + 16 * (((qd >> 1) | 2) ^ vs);
  PVAcc acc{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < NB / 2; ++j) {
    const vec pb = p_operand<T>(sc[2 * j], sc[2 * j + 1]);
    constexpr int RB = G::HCM * 64;  // bytes per staged row
    const u32x2 a0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va0 + (2 * j) * RB)));
    const u32x2 a1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va0 + (2 * j + 1) * RB)));
    const u32x2 b0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va1 + (2 * j) * RB)));
    const u32x2 b1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(va1 + (2 * j + 1) * RB)));
    pv_step<T>(acc, __builtin_bit_cast(vec, u32x4{a0[0], a0[1], a1[0], a1[1]}),
               __builtin_bit_cast(vec, u32x4{b0[0], b0[1], b1[0], b1[1]}), pb);
  }
  return finish<T>(acc, tci0 + qy < r.rc1 && tcj0 + qx < c.cc1, lse);
}

// Writes a lane's TileOut to the query at in-plane byte offset off of out.
template <typename T, bool STREAM>
__device__ __forceinline__ void store_out(T *__restrict__ out, int64_t pofs, unsigned off, int g,
                                          const TileOut &t) {
  if (t.ok) {
    u32x2 *o = (u32x2 *)(((char *)out + pofs) + (off + g * 8u));
    if constexpr (STREAM) {
      __builtin_nontemporal_store(u32x2{t.val[0], t.val[1]}, o);
      __builtin_nontemporal_store(u32x2{t.val[2], t.val[3]}, o + 2 * sizeof(T));
    } else {
      o[0] = u32x2{t.val[0], t.val[1]};
      o[2 * sizeof(T)] = u32x2{t.val[2], t.val[3]};
    }
  }
}

// Writes a query's log-sum-exp (one lane of its 4): with dense q its index in
// [B, heads, H, W] order is its q byte offset over the pixel's D channels.
template <typename T>
__device__ __forceinline__ void store_lse(float *__restrict__ lse, int64_t pofs, unsigned off,
                                          int g, const TileOut &t) {
  if (g == 0 && t.ok) lse[(pofs + off) / (kHeadDim * sizeof(T))] = t.lse;
}

// STREAM: Q and out accesses are non-temporal (dense maps without dilation).
// MODE (dense q only beyond kForward): kForwardLse also writes each query's
// log-sum-exp to lse; kScores writes only the scores, to lse as a [.., k*k]
// tensor (no V staged, no out).
template <typename T, int KS, int RY, bool STREAM, int MODE>
__global__ __launch_bounds__((Geometry<KS, RY>::THREADS)) void fused_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, Shape s, ByteStrides si, ByteStrides so,
    FastDiv fdil, FastDiv fnbx, FastDiv fnby, FastDiv fheads, int nblocks,
    float *__restrict__ lse) {
  using G = Geometry<KS, RY>;
  constexpr bool LSE = MODE == kForwardLse, SCORES = MODE == kScores;
  // kScores: each wave's score rows go through the free V buffers, half of
  // the waves in each
  constexpr int HALF = (G::NTILE + 1) / 2;
  static_assert(!SCORES || HALF * 16 * KS * KS * 4 <= G::PIX * 64, "score staging exceeds LDS");
  __shared__ __attribute__((aligned(16))) char kbuf0[G::PIX * 64], vbuf0[G::PIX * 64];
  __shared__ __attribute__((aligned(16))) char kbuf1[G::PIX * 64], vbuf1[G::PIX * 64];
  __shared__ float tab0[G::NTAB], tab1[G::NTAB];

  // wave index is uniform within a wave: keep it (and all that derives from
  // it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  // this workgroup's blocks: a contiguous run of ids, or, in a crew of d
  // (the launch makes the grid a multiple of d when d > 1), every d-th id of
  // the crew's run of d * count ids, from the member's own class
  const int wg = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int ngrid = (int)gridDim.x;
  const bool crew = s.dil > 1 && ngrid % s.dil == 0;
  int first, count;
  if (crew) {
    const int nsets = ngrid / s.dil, set = (int)fast_div((uint32_t)wg, fdil);
    const int units = nblocks / s.dil;  // blocks per column class digit
    const int p0 = (int)((int64_t)units * set / nsets);
    const int p1 = (int)((int64_t)units * (set + 1) / nsets);
    first = p0 * s.dil + (wg - set * s.dil);
    count = p1 - p0;
  } else {
    first = (int)((int64_t)nblocks * wg / ngrid);
    count = (int)((int64_t)nblocks * (wg + 1) / ngrid) - first;
  }
  if (count <= 0) return;
  const bool has_rpb = rpb != nullptr;
  // this wave's tile and this lane's query position within a block
  const int ty = wave / G::NTX, tx = wave % G::NTX;
  const int lr = ty * G::TY + ql / G::TX, lc = tx * G::TX + ql % G::TX;
  const int nbx = fnbx.div, nby = fnby.div;

  // Prefetch order for block n+1 while block n computes: its Q slice (and,
  // when the head changes, its bias-table values) first, then the K/V DMA;
  // nothing consumes them before the end-of-block barrier, so the loads
  // overlap the whole compute of block n.
  T treg[TableRegs<KS, RY>::N];
  BlockCursor cc = cursor_at((uint32_t)first, s.dil, fdil, fnbx, fnby, fheads);
  RowPart rcur = row_part<T, KS, RY>(cc, s, fdil, si, so, ty, lr);
  ColPart ccur = col_part<T, KS>(cc, s, fdil, si, tx, lc);
  QueryOffs pcur = query_offsets(rcur, ccur, s, si, so, lr, lc);
  u32x4 qcur = load_q<T, STREAM>(q, rcur.pofs, pcur.q, g);
  load_tables<T, KS, RY>(rpb, rcur.h, tid, treg);
  if (rcur.ok && ccur.ok)
    stage_block<T, KS, RY, !SCORES>(k, v, rcur, ccur, s, si, kbuf0, vbuf0, wave, lane);
  store_tables<T, KS, RY>(tab0, tid, has_rpb, treg);
  float *const stage =
      SCORES ? (float *)(wave < HALF ? vbuf0 : vbuf1) + (wave % HALF) * 16 * KS * KS : nullptr;
  int tab_h0 = rcur.h, tab_h1 = -1;  // head whose tables each buffer holds
  __syncthreads();

  TileOut res;
  // One block: compute the current one from buffer (kc, vc, tc) while block
  // n+1 is staged into (kn, vn, tn).  Called with fixed arrays, so that the
  // compiler can tell the DMA target from the buffer being read.
  auto step = [&](const char *kc, const char *vc, const float *tc, char *kn, char *vn, float *tn,
                  int &tab_hn, bool more) {
    RowPart rnxt = rcur;
    if (more && cursor_step(cc, s.dil, nbx, nby, s.heads, crew))
      rnxt = row_part<T, KS, RY>(cc, s, fdil, si, so, ty, lr);
    const ColPart cnxt = col_part<T, KS>(cc, s, fdil, si, tx, lc);
    const QueryOffs pnxt = query_offsets(rnxt, cnxt, s, si, so, lr, lc);
    const u32x4 qnxt = load_q<T, STREAM>(q, rnxt.pofs, pnxt.q, g);
    const bool newtab = more && rnxt.h != tab_hn;
    if (newtab) load_tables<T, KS, RY>(rpb, rnxt.h, tid, treg);
    if (more && rnxt.ok && cnxt.ok)
      stage_block<T, KS, RY, !SCORES>(k, v, rnxt, cnxt, s, si, kn, vn, wave, lane);
    res = TileOut{{0u, 0u, 0u, 0u}, false, 0.f};
    if (rcur.ok && ccur.ok)
      res = compute_tile<T, KS, MODE>(rcur, ccur, kc, vc, tc, qcur, lane, stage, lse,
                                      rcur.pofs / (kHeadDim * (int64_t)sizeof(T)), s.W, s.dil);
    if (!more) return;
    if (newtab) {
      store_tables<T, KS, RY>(tn, tid, has_rpb, treg);
      tab_hn = rnxt.h;
    }
    __syncthreads();  // also waits for the DMA (workgroup fence)
    // the block's results leave after the barrier, so that its wait covers
    // the next block's loads but not these stores
    // (STREAM runs dense maps only: out has q's strides)
    if constexpr (STREAM) store_out<T, STREAM>(out, rcur.pofs, pcur.q, g, res);
    else if constexpr (!SCORES) store_out<T, STREAM>(out, rcur.opofs, pcur.o, g, res);
    if constexpr (LSE) store_lse<T>(lse, rcur.pofs, pcur.q, g, res);
    rcur = rnxt;
    ccur = cnxt;
    pcur = pnxt;
    qcur = qnxt;
  };
  // Two blocks per iteration so that each buffer is a fixed LDS array.
  for (int bi = 0; bi < count; bi += 2) {
    const bool more0 = bi + 1 < count;
    step(kbuf0, vbuf0, tab0, kbuf1, vbuf1, tab1, tab_h1, more0);
    if (!more0) break;
    step(kbuf1, vbuf1, tab1, kbuf0, vbuf0, tab0, tab_h0, bi + 2 < count);
  }
  // the last block
  if constexpr (STREAM) store_out<T, STREAM>(out, rcur.pofs, pcur.q, g, res);
  else if constexpr (!SCORES) store_out<T, STREAM>(out, rcur.opofs, pcur.o, g, res);
  if constexpr (LSE) store_lse<T>(lse, rcur.pofs, pcur.q, g, res);
}

// Host-side view of a launch's layout: strides in bytes, whether q, k, v and
// out are all dense [B, heads, H, W, D], the optional log-sum-exp output
// (dense maps only), and the score output of a scores-only launch.
struct Layout {
  ByteStrides in, out;
  bool planar;
  float *lse;
  float *scores;
};

template <typename T, int KS, int RY>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *rpb, void *out,
                    const Shape &s, const Layout &lay, hipStream_t st) {
  using G = Geometry<KS, RY>;
  const int Lymax = class_len(s.H, 0, s.dil), Lxmax = class_len(s.W, 0, s.dil);
  const int nby = (Lymax + G::RY - 1) / G::RY, nbx = (Lxmax + G::RX - 1) / G::RX;
  const int64_t nblocks = (int64_t)s.B * s.heads * s.dil * s.dil * nby * nbx;
  if (nblocks > INT_MAX) return hipErrorInvalidConfiguration;
  // one persistent workgroup per compute unit (its LDS holds two blocks);
  // with dilation a multiple of d (crews of d workgroups, one per column
  // class; nblocks is a multiple of d)
  int64_t grid = nblocks < device_compute_units() ? nblocks : device_compute_units();
  if (s.dil > 1 && grid >= s.dil) grid -= grid % s.dil;
  // Non-temporal Q/out only when each line belongs to one block: dense maps
  // without dilation (channels-last maps interleave the heads' channels).
  auto kernel = s.dil == 1 && lay.planar
                    ? (lay.lse ? fused_mfma_kernel<T, KS, RY, true, kForwardLse>
                               : fused_mfma_kernel<T, KS, RY, true, kForward>)
                    : (lay.lse ? fused_mfma_kernel<T, KS, RY, false, kForwardLse>
                               : fused_mfma_kernel<T, KS, RY, false, kForward>);
  float *extra = lay.lse;
  if (lay.scores != nullptr) {
    if constexpr (KS <= 9) {
      kernel = fused_mfma_kernel<T, KS, RY, false, kScores>;
      extra = lay.scores;
    } else {
      return hipErrorInvalidValue;  // no scores-only variant (its LDS rows do not fit)
    }
  }
  kernel<<<dim3((unsigned)grid), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (T *)out, s, lay.in, lay.out,
      make_fastdiv((uint32_t)s.dil), make_fastdiv((uint32_t)nbx), make_fastdiv((uint32_t)nby),
      make_fastdiv((uint32_t)s.heads), (int)nblocks, extra);
  return hipGetLastError();
}

// k <= 7: blocks of 32 rows (16 waves) or 28 rows (14 waves), whichever
// covers the tallest residue class with fewer blocks (28 on a tie: less work
// per block for the same count).
template <typename T, int KS>
hipError_t launch_small(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, const Layout &lay, hipStream_t st) {
  const int L = class_len(s.H, 0, s.dil);
  if ((L + 27) / 28 <= (L + 31) / 32) return launch_t<T, KS, 28>(q, k, v, rpb, out, s, lay, st);
  return launch_t<T, KS, 32>(q, k, v, rpb, out, s, lay, st);
}

template <typename T>
hipError_t launch_dtype(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, const Layout &lay, hipStream_t st, bool *supported) {
  switch (s.ks) {
    case 1: return launch_small<T, 1>(q, k, v, rpb, out, s, lay, st);
    case 3: return launch_small<T, 3>(q, k, v, rpb, out, s, lay, st);
    case 5: return launch_small<T, 5>(q, k, v, rpb, out, s, lay, st);
    case 7: return launch_small<T, 7>(q, k, v, rpb, out, s, lay, st);
    case 9: return launch_t<T, 9, default_rows(9)>(q, k, v, rpb, out, s, lay, st);
    case 11: return launch_t<T, 11, default_rows(11)>(q, k, v, rpb, out, s, lay, st);
    case 13: return launch_t<T, 13, default_rows(13)>(q, k, v, rpb, out, s, lay, st);
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_fused_mfma(const void *q, const void *k, const void *v, const void *rpb,
                             void *out, const Shape &s, const Strides &in,
                             const Strides &out_st, const Pad &pad, na2d_dtype_t dt,
                             hipStream_t st, bool *supported, float *lse, bool stream) {
  *supported = true;
  if (dt != NA2D_DTYPE_BF16 && dt != NA2D_DTYPE_F16) {
    *supported = false;
    return hipSuccess;
  }
  Layout lay;
  lay.planar = is_planar(in, s) && is_planar(out_st, s);
  lay.lse = lse;
  lay.scores = nullptr;
  if (lse != nullptr && !is_planar(in, s)) {  // its index comes from q's dense offsets
    *supported = false;
    return hipSuccess;
  }
  const int64_t elem = 2;
  if (!mfma::byte_strides(in, s, elem, &lay.in) || !mfma::byte_strides(out_st, s, elem, &lay.out)) {
    *supported = false;
    return hipSuccess;
  }
  hipError_t e =
      launch_dense_mfma(q, k, v, rpb, out, s, lay.in, lay.out, pad, dt, st, supported, lse);
  if (*supported) return e;
  // the general kernels run unpadded maps only
  if (pad.Hp > s.H || pad.Wp > s.W) {
    *supported = false;
    return hipSuccess;
  }
  *supported = true;
  if (stream && stream_mfma_supported(s, dt))
    return launch_stream_mfma(q, k, v, rpb, out, lse, s, lay.in, lay.out, dt, st);
  if (dt == NA2D_DTYPE_BF16)
    return launch_dtype<__bf16>(q, k, v, rpb, out, s, lay, st, supported);
  return launch_dtype<_Float16>(q, k, v, rpb, out, s, lay, st, supported);
}

hipError_t launch_scores_mfma(const void *q, const void *k, const void *rpb, float *attn,
                              const Shape &s, na2d_dtype_t dt, hipStream_t st, bool *supported) {
  *supported = false;
  if ((dt != NA2D_DTYPE_BF16 && dt != NA2D_DTYPE_F16) || s.ks > 9) return hipSuccess;
  Layout lay;
  const Strides pl = planar_strides(s);
  if (!mfma::byte_strides(pl, s, 2, &lay.in)) return hipSuccess;
  lay.out = lay.in;
  lay.planar = true;
  lay.lse = nullptr;
  lay.scores = attn;
  *supported = true;
  if (dt == NA2D_DTYPE_BF16)
    return launch_dtype<__bf16>(q, k, nullptr, rpb, nullptr, s, lay, st, supported);
  return launch_dtype<_Float16>(q, k, nullptr, rpb, nullptr, s, lay, st, supported);
}

}  // namespace na2d
