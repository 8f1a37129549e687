// na2d_stream.hip -- row-streaming fused forward of 2D (dilated) Neighborhood
// Attention on the CDNA4 matrix cores: bf16 / fp16 inputs, fp32
// accumulation, D = 32, kernel sizes 3, 5, 7, maps (or, with dilation d,
// residue classes) of any width: up to 56 columns in one workgroup of 1 to 7
// waves, wider ones in strips of 56 columns.
//
// The operator is the one the DiNAT module composes from natten2dqkrpb,
// softmax(dim=-1) and natten2dav (DiNAT walk-through blog, "What is DiNAT");
// the window is the query-centred k x k neighbourhood shifted inward at the
// borders (NAT repository README, introduction).
//
// Why streaming.  Every key/value pixel is read by the k x k queries around
// it.  A kernel that stages a separate halo per query block moves each pixel
// into LDS about twice and, with all compute units staging their next block
// at the same moment, leaves HBM idle between bursts.  Here a workgroup owns
// a run of query rows of one (batch, head) plane, over the map's full width,
// and walks down it four query rows per step.  Each key and value row is
// fetched from HBM once, into registers, two steps before it is needed, then
// written into a 16-row LDS ring; a step waits only for its own rows, so the
// loads of later steps stay in flight while it computes.
//
// Work per step (4 query rows x 8*NTX columns): one wave per 8-column tile
// column, for both of its 2 x 8 query tiles (rows R, R+1 and R+2, R+3).
// A tile's keys are NB = k + 1 rows x 16 columns of the ring; the two tiles
// of a wave share k - 1 of their key rows (and the operand reads of those).
// S^T = K . Q^T on v_mfma_f32_16x16x32 (one per key row), the bias times
// sqrt(D) and the -inf window mask as the accumulator input, softmax in
// registers (max by lane swaps, exp2), out^T = V^T . P^T with V^T read by
// ds_read_b64_tr_b16, the denominator from a product with ones.
//
// Memory layout of the ring (per tensor, 16 rows, SCW staged columns):
//   K: [row][column][64 bytes], the four 16-byte chunks of a pixel permuted
//      by kswz(column) so that the 8 pixels one pass of a K read serves
//      (8 lanes x 16 bytes: 128 bytes, the width of the LDS banks) fall on
//      distinct banks;
//   V: two planes (channels 0-15 and 16-31), [row][column][32 bytes]: a pass
//      of the transposing read (16 lanes x 8 bytes) covers 4 consecutive
//      pixels, 128 contiguous bytes, and the second channel block sits at a
//      fixed offset.
// Ring row y & 15 holds pixel row y.
//
// Dilation.  With dilation d the pixels (ry + d*i, rx + d*j) of one residue
// class form an ordinary map on which the operator is plain neighborhood
// attention (DiNAT walk-through blog, "What is DiNAT": the window samples
// every d-th pixel).  When d divides H and W every class is (H/d) x (W/d);
// the kernel then runs on the classes as on maps of that size, with the
// row and column strides multiplied by d.  Units are numbered with rx
// fastest, so the classes rx and rx + 1, whose pixels share 128-byte lines,
// run at the same time on one XCD and the second read of each line hits L2.
#include "na2d_mfma_common.h"

#include <limits.h>

#include <algorithm>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16-byte chunk permutation of the K ring (see the header comment).
__device__ __forceinline__ int kswz(int c) { return (c >> 1) & 3; }

// STRIPS: the map is wider than 8 * NTX columns and each unit covers one
// strip of 8 * NTX query columns (its staged key columns reach k - 1 past
// it); one more wave then shares the loads (and repeats the last tile
// column's compute on the otherwise idle fourth SIMD, storing nothing), so
// that each lane stages as many pieces as without strips.
template <int KS, int NTX, bool STRIPS = false> struct StreamGeo {
  static constexpr int R = KS / 2;
  static constexpr int TX = 8;                    // tile: 2 rows x 8 columns
  static constexpr int NB = KS + 1;               // key rows per tile
  static constexpr int NS = NB + 2;               // key rows of a wave's two tiles
  static constexpr int WAVES = NTX + (STRIPS ? 1 : 0);
  static constexpr int THREADS = 64 * WAVES;      // one wave per tile column
  static constexpr int CW = 8 * NTX;              // query columns
  // staged columns: at most CW (the map, at most CW wide) or, with strips,
  // CW + k - 1; a tile's reads of the 16 key columns from its first one are
  // clamped to the last staged column (columns past it are only ever masked)
  static constexpr int NK = STRIPS ? CW + KS - 1 : CW;
  // ring row pitch in columns: NK where several workgroups share a compute
  // unit (NTX < 5) and LDS is the limit; 8 * (NTX + 1) otherwise, as it
  // measured a little faster than 8 * NTX at NTX = 7
  static constexpr int SCW = (STRIPS || NTX < 5) ? NK : CW + 8;
  static constexpr int RING = 16;                 // staged rows
  static constexpr int KROW = SCW * 64;           // bytes per K ring row
  static constexpr int VROW = SCW * 32;           // bytes per V ring row (one channel half)
  static constexpr int KRING = RING * KROW;
  static constexpr int VHALF = RING * VROW + 64;  // second half after a bank offset
  static constexpr int VOFF = KRING;              // V ring after the K ring
  static constexpr int SIDE = 2 * KS - 1;
  static constexpr int MARGIN = 2 * SIDE + 32;    // keeps masked bias reads in bounds
  static constexpr int NTAB = SIDE * SIDE + 2 * MARGIN;
  static constexpr int TABOFF = VOFF + 2 * VHALF; // bias table (times sqrt(D)), zero margins
  static constexpr int LDS = TABOFF + NTAB * 4;
  // 16-byte pieces per lane and tensor for one group of 4 rows
  static constexpr int NP = (16 * NK + THREADS - 1) / THREADS;
  static_assert(NB % 2 == 0 && NB <= 8, "tile key rows");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(VHALF < (1 << 16), "the second V half is a 16-bit immediate offset");
};

// One unit of work: a residue class of a (batch, head) plane (the plane
// itself without dilation) and a run of its query rows.
// Units alternate direction: an even one walks down its rows, an odd one up
// (it sees the map flipped upside down: row y of the unit is memory row
// H - 1 - y, and the bias table's rows are reversed).  The two units that
// share a boundary then read the key/value rows around it at the same time
// (both at their last steps, or both at their first), so the second read
// finds them in the cache, and the first and last units of a plane start at
// the map's edge, where the windows of the first query rows overlap most.
struct Unit {
  int64_t pin, pout;     // byte offsets of the class origin in q/k/v and in out
  int64_t lpix;          // pixel index of the class origin in [B, heads, H, W]
  int h, q0, q1, nsteps; // query rows [q0, q1) in the unit's own row order
  int strip;             // query columns [strip * CW, strip * CW + CW) of the map
  bool flip;
};

// s: the class map (H/d x W/d, dilation 1); si, so: strides within a class
// (row and column strides of the map times d); pixel strides of the map
// for the class origins, and the map's size for the log-sum-exp index.
struct StreamArgs {
  Shape s;
  ByteStrides si, so;
  int dil, Hm, Wm;         // dilation; the map's rows and columns
  int oyi, oxi, oyo, oxo;  // map row / column strides of q, k, v and of out (bytes)
  int seg, nseg;           // query rows per unit, units per class and strip
  int nstrip;              // column strips per class
  int nunits;
  FastDiv fseg, fheads, fdil, fstrip;
};

__device__ __forceinline__ Unit unit_at(int u, const StreamArgs &a) {
  Unit t;
  // u = (((((b * heads + h) * d + ry) * d + rx) * nstrip + strip) * nseg + sg
  const uint32_t cs = fast_div((uint32_t)u, a.fseg);
  const int sg = u - (int)cs * a.nseg;
  const uint32_t cls = fast_div(cs, a.fstrip);
  t.strip = (int)(cs - cls * a.nstrip);
  const uint32_t t1 = fast_div(cls, a.fdil);
  const int rx = (int)(cls - t1 * a.dil);
  const uint32_t bh = fast_div(t1, a.fdil);
  const int ry = (int)(t1 - bh * a.dil);
  const uint32_t b = fast_div(bh, a.fheads);
  t.h = (int)(bh - b * a.s.heads);
  t.pin = (int64_t)b * a.si.b + (int64_t)t.h * a.si.h + (int64_t)ry * a.oyi +
          (int64_t)rx * a.oxi;
  t.pout = (int64_t)b * a.so.b + (int64_t)t.h * a.so.h + (int64_t)ry * a.oyo +
           (int64_t)rx * a.oxo;
  t.lpix = (int64_t)bh * a.Hm * a.Wm + (int64_t)ry * a.Wm + rx;
  const int r0 = sg * a.seg, r1 = min(r0 + a.seg, a.s.H);
  t.flip = (sg & 1) != 0;
  t.q0 = t.flip ? a.s.H - r1 : r0;
  t.q1 = t.flip ? a.s.H - r0 : r1;
  t.nsteps = (t.q1 - t.q0 + 3) >> 2;
  return t;
}

// A lane's share of one group of 4 key/value rows: NP pieces of K and the
// same NP pieces of V (16 bytes each, at the same in-plane offset).
template <int NP> struct Piece {
  uint32_t goff[NP];     // in-plane byte offset at the group's first row = row 0
  uint32_t klds[NP];     // K ring offset at ring row 0
  uint32_t vlds[NP];     // V ring offset at ring row 0
  int row[NP];           // row within the group
};

template <int NP> struct Regs {
  u32x4 k[NP], v[NP];
};

// Cache policy of the buffer loads and stores: non-temporal (every byte is
// read or written once); and the fourth word of a buffer resource (raw
// dword access, no format conversion).
constexpr int kNonTemporal = 2;
constexpr int kRsrcWord3 = 0x00020000;

// LSE: also write each query's log-sum-exp to lse, [B, heads, H, W] (dense
// q only).  STREAM: query loads and output / lse stores are non-temporal
// (without dilation each line belongs to one unit); with dilation the
// classes rx and rx + 1 share every line of q and out, so those accesses stay
// cached and the second class finds the line in L2.
template <typename T, int KS, int NTX, bool LSE, bool STREAM, bool STRIPS>
__global__ __launch_bounds__((StreamGeo<KS, NTX, STRIPS>::THREADS)) void stream_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, float *__restrict__ lse, StreamArgs A) {
  constexpr int kQO = STREAM ? kNonTemporal : 0;  // cache policy of q, out and lse
  using G = StreamGeo<KS, NTX, STRIPS>;
  using vec = typename Mma<T>::vec;
  constexpr int NB = G::NB, NS = G::NS, NP = G::NP, SIDE = G::SIDE, R = G::R;
  __shared__ __attribute__((aligned(16))) char lds[G::LDS];
  float *const tab = (float *)(lds + G::TABOFF);

  const int tid = threadIdx.x, lane = tid & 63;
  const int tx = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's tile column
  const int ql = lane & 15, g = lane >> 4, qy = ql >> 3, qx = ql & 7;
  const int H = A.s.H, W = A.s.W;
  const bool has_rpb = rpb != nullptr;
  const float c2 = kLog2e / kSqrtD;

  // ---- per-lane constants of a column strip (the whole map without
  // strips): set by set_strip when a unit's strip differs from the last one.
  // This lane's pieces of a 4-row group: (row, staged column, chunk); lanes
  // beyond the group's 16 * nk pieces repeat one (same data, same place).
  // Every load, LDS write and store below is unconditional, so that the
  // count of memory operations in flight is the same on every path and the
  // compiler's waits before a use cover exactly the operation it needs.
  Piece<NP> pc;
  // this wave's tiles: query columns C .. C+7; first key column X0; this
  // lane's query column cq (clamped) and its window's first column sx; the
  // K read of key (row a, column X0 + ql), chunk g, and the V^T read of
  // column X0 + 4g + ql/4, channels 4*(ql%4) .. + 3 of each channel half, at
  // ring columns counted from the strip's first staged column
  int C = 0, X0 = 0, cq = 0, sx = 0;
  uint32_t klane = 0, vlane = 0;
  // Query slices and outputs move through memory in "pixel order": lane L
  // holds 16-byte chunk L%4 of the tile's query L/4 (row L/32, column
  // (L/4)%8), so that each 16-lane quarter of a wave touches 4 whole 64-byte
  // pixels.  Lane shuffles (ds_bpermute) convert to and from the
  // matrix-core layout, where lane (g, ql) holds chunk g of query ql.
  const int lp = lane >> 2, lc = lane & 3;
  const int lpy = lp >> 3, lpx = lp & 7;
  bool lcol_ok = false;
  uint32_t qcol = 0, ocol = 0;
  // Window caps of this lane's key columns X0 + 4g + i: +inf inside its
  // query's window, -inf outside (hidden from the optimiser so that each
  // masked entry costs one min).
  float ccap[4];
  auto set_strip = [&](int strip) {
    const int c0 = strip * G::CW, c1 = min(c0 + G::CW, W);
    const int xs0 = window_start(c0, W, KS);
    const int nk = window_start(c1 - 1, W, KS) + KS - xs0;  // staged columns
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      int f = tid + j * G::THREADS;
      f = f < 16 * nk ? f : f % (16 * nk);
      const int p = f & 3, cx = f >> 2;            // chunk; row * nk + staged column
      int rr = 0;
#pragma unroll
      for (int m = 1; m < 4; ++m) rr += cx >= m * nk;
      const int lx = cx - rr * nk;
      pc.row[j] = rr;
      pc.goff[j] = (uint32_t)rr * A.si.y + (uint32_t)(xs0 + lx) * A.si.x + p * 16;
      pc.klds[j] = (uint32_t)(lx * 64 + ((p ^ kswz(lx)) * 16));
      pc.vlds[j] = (uint32_t)(G::VOFF + (p >> 1) * G::VHALF + lx * 32 + (p & 1) * 16);
    }
    C = c0 + 8 * min(tx, NTX - 1);
    X0 = window_start(min(C, W - 1), W, KS);
    cq = min(C + qx, W - 1);
    sx = window_start(cq, W, KS);
    const int kx = min(X0 - xs0 + ql, nk - 1);
    klane = (uint32_t)(kx * 64 + ((g ^ kswz(kx)) * 16));
    vlane = (uint32_t)(G::VOFF + min(X0 - xs0 + 4 * g + (ql >> 2), nk - 1) * 32 + (ql & 3) * 8);
    lcol_ok = tx < NTX && C + lpx < c1;
    qcol = (uint32_t)min(C + lpx, W - 1) * A.si.x + lc * 16;
    ocol = (uint32_t)(C + lpx) * A.so.x + lc * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ccap[i] = (unsigned)(X0 + 4 * g + i - sx) < (unsigned)KS ? INFINITY : -INFINITY;
      asm volatile("" : "+v"(ccap[i]));
    }
  };
  const int qsrc = (4 * ql + g) * 4;
  // out: the lane holding chunk lc of query lp after the pair swap below
  const int osrc = (16 * ((lc >> 1) + 2 * (lc & 1)) + lp) * 4;
  auto shuffle = [](u32x4 x, int src) -> u32x4 {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)x[i]);
    return r;
  };
  const int inspan = (int)((uint32_t)(H - 1) * A.si.y + (uint32_t)(W - 1) * A.si.x + 64);
  const int outspan = (int)((uint32_t)(H - 1) * A.so.y + (uint32_t)(W - 1) * A.so.x + 64);

  // The accumulator inputs of this wave's tiles on steps whose query rows
  // are all unclamped: bias * sqrt(D) inside the window, -inf outside, for
  // key row a (of the tile's NB) and key columns X0 + 4g .. + 3 of this
  // lane's query.  Rebuilt from the LDS table when the head changes.
  f32x4 cin[NB];
  auto build_cin = [&]() {
    const int colrel = X0 + 4 * g - sx;          // key column - window start (i = 0)
    const int dx0 = X0 + 4 * g - cq + KS - 1;    // table column (i = 0)
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int rowrel = a - qy;                 // key row - window start
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = (unsigned)rowrel < (unsigned)KS && (unsigned)(colrel + i) < (unsigned)KS;
        const int e = G::MARGIN + (rowrel - R + KS - 1) * SIDE + dx0 + i;
        cin[a][i] = in ? tab[in ? e : G::MARGIN] : -INFINITY;
      }
    }
  };

  // Softmax weights of one tile's scores, as the 16-bit P^T operands of its
  // NB / 2 key-row pairs; returns the log-sum-exp of the lane's query (LSE
  // only: from the fp32 weights' sum, not the 16-bit one the output is
  // divided by).
  auto weights = [&](f32x4 (&sc)[NB], vec (&pbs)[NB / 2]) -> float {
    // the maximum as a tree (short dependency chains)
    float m[NB];
#pragma unroll
    for (int a = 0; a < NB; ++a) m[a] = fmaxf(fmaxf(sc[a][0], sc[a][1]), fmaxf(sc[a][2], sc[a][3]));
#pragma unroll
    for (int w = 1; w < NB; w *= 2)
#pragma unroll
      for (int a = 0; a + w < NB; a += 2 * w) m[a] = fmaxf(m[a], m[a + w]);
    const float mx = group_max(m[0]);
    const float mc = mx * c2;
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < NB / 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pa = __builtin_amdgcn_exp2f(fmaf(sc[2 * j][i], c2, -mc));
        const float pb = __builtin_amdgcn_exp2f(fmaf(sc[2 * j + 1][i], c2, -mc));
        pbs[j][i] = static_cast<T>(pa);
        pbs[j][4 + i] = static_cast<T>(pb);
        if constexpr (LSE) l += pa + pb;
      }
    if constexpr (LSE) return window_lse(mc, group_sum(l));
    return 0.f;
  };
  // V^T operands (channels 0-15 and 16-31) of the key-row pair at ring rows
  // y, y + 1.
  auto v_pair = [&](int y, vec &va, vec &vb) {
    const uint32_t r0 = vlane + (uint32_t)(y & (G::RING - 1)) * G::VROW;
    const uint32_t r1 = vlane + (uint32_t)((y + 1) & (G::RING - 1)) * G::VROW;
    const u32x2 a0 = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + r0)));
    const u32x2 a1 = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + r1)));
    const u32x2 b0 = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + r0 + G::VHALF)));
    const u32x2 b1 = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds + r1 + G::VHALF)));
    va = __builtin_bit_cast(vec, u32x4{a0[0], a0[1], a1[0], a1[1]});
    vb = __builtin_bit_cast(vec, u32x4{b0[0], b0[1], b1[0], b1[1]});
  };
  auto k_row = [&](int y) -> vec {
    return __builtin_bit_cast(
        vec, *(const u32x4 *)(lds + klane + (uint32_t)(y & (G::RING - 1)) * G::KROW));
  };
  vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);
  // The rounded output of a tile in pixel order (see above).
  auto finish = [&](const f32x4 &o0, const f32x4 &o1, const f32x4 &o2) -> u32x4 {
    const float inv = __builtin_amdgcn_rcpf(o2[0]);
    typedef __attribute__((ext_vector_type(4))) T vec4;
    vec4 w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = static_cast<T>(o0[i] * inv);
      w1[i] = static_cast<T>(o1[i] * inv);
    }
    // Lane group g holds channels 4g..4g+3 (w0) and 16+4g..16+4g+3 (w1). One
    // swap between the groups of a pair (g even with g + 1) gives each lane
    // 16 contiguous bytes: group g even channels 4g..4g+7 (chunk g/2), group
    // g odd channels 16+4(g-1)..16+4g+3 (chunk 2+(g-1)/2).
    const u32x2 p0 = __builtin_bit_cast(u32x2, w0), p1 = __builtin_bit_cast(u32x2, w1);
    const auto x0 = __builtin_amdgcn_permlane16_swap(p0[0], p1[0], false, false);
    const auto x1 = __builtin_amdgcn_permlane16_swap(p0[1], p1[1], false, false);
    return shuffle(u32x4{x0[0], x1[0], x0[1], x1[1]}, osrc);
  };
  // One tile with clamped rows: first query row Rt, first key row
  // Yt = window_start(Rt).  The bias comes from the LDS table, the window
  // mask from the caps: the lanes' window starts are Yt or Yt + 1, so key
  // rows 1 .. k-1 are inside every lane's row window and only rows 0 and k
  // need a row test.
  auto edge_tile = [&](int Rt, int Yt, const vec &qv, float &lse_t) -> u32x4 {
    const int rq = min(Rt + qy, H - 1);
    const int rowrel = Yt - window_start(rq, H, KS);
    int bidx = G::MARGIN + (Yt - rq + KS - 1) * SIDE + (X0 + 4 * g - cq + KS - 1);
    asm volatile("" : "+v"(bidx));  // one base register; the reads use immediate offsets
    const float *bb = tab + bidx;
    f32x4 sc[NB];
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const bool rtest = a == 0 || a >= KS;
      float rcap = (unsigned)(rowrel + a) < (unsigned)KS ? INFINITY : -INFINITY;
      if (rtest) asm volatile("" : "+v"(rcap));
      f32x4 c;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c[i] = rtest ? fminf(fminf(bb[a * SIDE + i], ccap[i]), rcap)
                     : fminf(bb[a * SIDE + i], ccap[i]);
      sc[a] = Mma<T>::run(k_row(Yt + a), qv, c);
    }
    vec pbs[NB / 2];
    lse_t = weights(sc, pbs);
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, o2 = o0;
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) {
      vec va, vb;
      v_pair(Yt + 2 * j, va, vb);
      o0 = Mma<T>::run(va, pbs[j], o0);
      o1 = Mma<T>::run(vb, pbs[j], o1);
      o2 = Mma<T>::run(ones, pbs[j], o2);
    }
    return finish(o0, o1, o2);
  };

  // ring slots that no step writes (columns past the map, rows past a
  // plane) are read only under the -inf mask; zeros keep those reads finite
  // (the 0-weight products then add exactly 0)
  for (int e = tid * 16; e < G::TABOFF; e += G::THREADS * 16)
    *(u32x4 *)(lds + e) = u32x4{0u, 0u, 0u, 0u};

  int cur_h = -1, cur_strip = -1;
  for (int u = xcd_contiguous_id(blockIdx.x, gridDim.x); u < A.nunits; u += gridDim.x) {
    const Unit t = unit_at(u, A);
    const bool newstrip = t.strip != cur_strip;
    if (newstrip) {
      set_strip(t.strip);
      cur_strip = t.strip;
    }
    // the plane of q, k, v and of out as buffer resources (scalar
    // registers): loads take a 32-bit lane offset plus a scalar row offset;
    // stores of lanes without a query get an offset past the plane's end,
    // which the hardware drops
    const __amdgpu_buffer_rsrc_t ors =
        __builtin_amdgcn_make_buffer_rsrc((char *)out + t.pout, 0, outspan, kRsrcWord3);
    // lse from the class origin: class pixel (i, j) is map pixel
    // (d*i, d*j) from there
    __amdgpu_buffer_rsrc_t lrs;
    if constexpr (LSE)
      lrs = __builtin_amdgcn_make_buffer_rsrc(lse + t.lpix, 0, A.Hm * A.Wm * 4, kRsrcWord3);

    // Key/value rows of the unit: those of step 0, [lo0, hi0], as np0
    // groups of 4 from lo0, then one group of 4 per step.  Step s needs
    // rows [window_start(R), window_start(R + 3) + k - 1], R = q0 + 4s: all
    // in the groups up to s, and none that the group of step s + 1
    // overwrites (16 rows back).
    const int lo0 = window_start(t.q0, H, KS);
    const int hi0 = window_start(min(t.q0 + 3, t.q1 - 1), H, KS) + KS - 1;
    const int hiL = window_start(t.q1 - 1, H, KS) + KS - 1;  // the unit's last row
    const int np0 = (hi0 - lo0 + 4) >> 2;
    const int gbase = lo0 + 4 * np0 - 4;   // first row of the group of step s: gbase + 4s
    // a piece's row within a group of 4, in the unit's row order
    int prow[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) prow[j] = t.flip ? 3 - pc.row[j] : pc.row[j];
    // Rows y0 .. y0 + 3.  A group holding wanted rows (live: y0 <= hiL) is
    // clamped into the map (the last groups of a plane then repeat real
    // rows, which land in their own ring rows unchanged); any other group
    // reads through an empty buffer (zeros, no memory traffic) and lands in
    // ring rows no step reads unmasked before they are rewritten: the four
    // past the unit's last row for a group of a step, rows lo0 + 8 .. + 11
    // for the third group of step 0 (the group of step 1 rewrites them).
    auto issue = [&](Regs<NP> &rg, int y0, bool live) {
      const int yc = max(min(y0, H - 4), 0);
      const int ro = live ? (int)((uint32_t)(t.flip ? H - 4 - yc : yc) * A.si.y) : 0;
      const int span = live ? inspan : 0;
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc((char *)k + t.pin, 0, span, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc((char *)v + t.pin, 0, span, kRsrcWord3);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        rg.k[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, pc.goff[j], ro, 0);
        rg.v[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, pc.goff[j], ro, 0);
      }
    };
    auto commit = [&](const Regs<NP> &rg, int y0, bool live, int ydead) {
      const int yc = live ? max(min(y0, H - 4), 0) : ydead;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const uint32_t slot = (uint32_t)((yc + prow[j]) & (G::RING - 1));
        *(u32x4 *)(lds + pc.klds[j] + slot * G::KROW) = rg.k[j];
        *(u32x4 *)(lds + pc.vlds[j] + slot * G::VROW) = rg.v[j];
      }
    };
    // the query slices of step s, tile rows 0 and 1 (zeros, read through an
    // empty buffer, past the unit's last step)
    auto q_load = [&](int s, u32x4 &qa, u32x4 &qb) {
      const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
          (char *)q + t.pin, 0, s < t.nsteps ? inspan : 0, kRsrcWord3);
      const int R0 = t.q0 + 4 * min(s, t.nsteps - 1);
      int ra = min(R0 + lpy, t.q1 - 1), rb = min(R0 + 2 + lpy, t.q1 - 1);
      if (t.flip) {
        ra = H - 1 - ra;
        rb = H - 1 - rb;
      }
      qa = __builtin_amdgcn_raw_buffer_load_b128(qr, (uint32_t)ra * A.si.y + qcol, 0,
                                                 kQO);
      qb = __builtin_amdgcn_raw_buffer_load_b128(qr, (uint32_t)rb * A.si.y + qcol, 0,
                                                 kQO);
    };

    // ---- unit prologue.  The bias values, the rows of step 0 and its query
    // slices first; the group of step 1, the query slices of step 1 and the
    // group of step 2 only once the rows of step 0 are in, so that no unit's
    // first rows queue behind other units' later ones.
    __syncthreads();  // the previous unit is done with the ring and the table
    const int tabkey = 2 * t.h + (t.flip ? 1 : 0);
    const bool newtab = tabkey != cur_h;
    constexpr int NT1 = (G::NTAB + G::THREADS - 1) / G::THREADS;
    T tb1[NT1];
    if (newtab && has_rpb) {
      const T *rh = rpb + (int64_t)t.h * SIDE * SIDE;
#pragma unroll
      for (int it = 0; it < NT1; ++it) {
        const int bi = tid + it * G::THREADS - G::MARGIN;
        const int ri = bi / SIDE, ci = bi - ri * SIDE;
        tb1[it] = rh[(bi >= 0 && bi < SIDE * SIDE) ? (t.flip ? SIDE - 1 - ri : ri) * SIDE + ci
                                                    : 0];
      }
    }
    Regs<NP> p0, p1, p2, set0, set1;
    // the rows of step 0 (at most k + 3 <= 10 of them), then steps 1 and 2
    const bool live1 = lo0 + 4 <= hiL, live2 = np0 > 2;
    u32x4 qa0, qa1, qb0, qb1;  // query slices of the even / odd steps
    issue(p0, lo0, true);
    issue(p1, lo0 + 4, live1);
    issue(p2, lo0 + 8, live2);
    q_load(0, qa0, qa1);
    if (newtab) {
#pragma unroll
      for (int it = 0; it < NT1; ++it) {
        const int e = tid + it * G::THREADS, bi = e - G::MARGIN;
        if (e < G::NTAB)
          tab[e] = (has_rpb && bi >= 0 && bi < SIDE * SIDE) ? Elem<T>::to_f(tb1[it]) * kSqrtD
                                                             : 0.f;
      }
    }
    commit(p0, lo0, true, 0);
    commit(p1, lo0 + 4, live1, hiL + 1);
    commit(p2, lo0 + 8, live2, lo0 + 8);
    issue(set1, gbase + 4, gbase + 4 <= hiL);
    q_load(1, qb0, qb1);
    issue(set0, gbase + 8, gbase + 8 <= hiL);
    if (newtab) {
      __syncthreads();  // the table is complete
      cur_h = tabkey;
    }
    if (newtab || newstrip) build_cin();

    // One step: compute step s (query slices qs0, qs1, then reloaded with
    // those of step s + 2), then commit the group of step s + 1 from gc and
    // reload gc with the group of step s + 3.  The commit comes after the
    // compute so that a step waits only for its own query slices; waves
    // still computing step s read no slot it writes (it lands 16 rows past
    // the step's first key row minus 4 or more).
    auto step = [&](int s, Regs<NP> &gc, u32x4 &qs0, u32x4 &qs1) {
      __syncthreads();  // step s's rows visible
      const int R0 = t.q0 + 4 * s;                    // the step's first query row
      const int R = min(R0, t.q1 - 1);                // (a step past the unit computes a real one)
      const vec q0v = __builtin_bit_cast(vec, shuffle(qs0, qsrc));
      const vec q1v = __builtin_bit_cast(vec, shuffle(qs1, qsrc));
      u32x4 res0, res1;
      float lse0 = 0.f, lse1 = 0.f;
      if (R >= G::R && R + 3 + G::R <= H - 1) {
        // all four query rows unclamped: tile 1's key rows are tile 0's
        // shifted by 2; the accumulator inputs are the per-wave ones
        const int Y0 = R - G::R;
        // every LDS read of the step is issued before its first use: the
        // key rows, then the V^T operands (needed after the softmax)
        vec kr[NS];
#pragma unroll
        for (int a = 0; a < NS; ++a) kr[a] = k_row(Y0 + a);
        vec va[NS / 2], vb[NS / 2];
#pragma unroll
        for (int j = 0; j < NS / 2; ++j) v_pair(Y0 + 2 * j, va[j], vb[j]);
        f32x4 sc0[NB], sc1[NB];
#pragma unroll
        for (int a = 0; a < NB; ++a) sc0[a] = Mma<T>::run(kr[a], q0v, cin[a]);
#pragma unroll
        for (int a = 0; a < NB; ++a) sc1[a] = Mma<T>::run(kr[a + 2], q1v, cin[a]);
        vec pb0[NB / 2], pb1[NB / 2];
        lse0 = weights(sc0, pb0);
        f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, o2 = o0, u0 = o0, u1 = o0, u2 = o0;
#pragma unroll
        for (int j = 0; j < NB / 2; ++j) {
          o0 = Mma<T>::run(va[j], pb0[j], o0);
          o1 = Mma<T>::run(vb[j], pb0[j], o1);
          o2 = Mma<T>::run(ones, pb0[j], o2);
        }
        lse1 = weights(sc1, pb1);
#pragma unroll
        for (int j = 0; j < NB / 2; ++j) {
          u0 = Mma<T>::run(va[j + 1], pb1[j], u0);
          u1 = Mma<T>::run(vb[j + 1], pb1[j], u1);
          u2 = Mma<T>::run(ones, pb1[j], u2);
        }
        res0 = finish(o0, o1, o2);
        res1 = finish(u0, u1, u2);
      } else {
        // clamped rows (the first and last steps of a plane): the two tiles
        // each with its own key rows and accumulator inputs from the table
        // (unrolled, so that their independent products interleave)
        res0 = res1 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int Rt = min(R + 2 * tt, H - 1);
          vec qv;
#pragma unroll
          for (int i = 0; i < 8; ++i) qv[i] = tt ? q1v[i] : q0v[i];
          float lt;
          const u32x4 r = edge_tile(Rt, window_start(Rt, H, KS), qv, lt);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            res0[i] = tt ? res0[i] : r[i];
            res1[i] = tt ? r[i] : res1[i];
          }
          lse0 = tt ? lse0 : lt;
          lse1 = tt ? lt : lse1;
        }
      }
      // the query slices of step s + 2 into the registers just used
      q_load(s + 2, qs0, qs1);
      const bool ok0 = s < t.nsteps && lcol_ok && R0 + lpy < t.q1;
      const bool ok1 = s < t.nsteps && lcol_ok && R0 + 2 + lpy < t.q1;
      const int ya = t.flip ? H - 1 - (R0 + lpy) : R0 + lpy;
      const int yb = t.flip ? H - 3 - (R0 + lpy) : R0 + 2 + lpy;
      const uint32_t oo0 = ok0 ? (uint32_t)ya * A.so.y + ocol : 0x80000000u;
      const uint32_t oo1 = ok1 ? (uint32_t)yb * A.so.y + ocol : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b128(res0, ors, oo0, 0, kQO);
      __builtin_amdgcn_raw_buffer_store_b128(res1, ors, oo1, 0, kQO);
      if constexpr (LSE) {
        // lane (0, ql) writes query ql of each tile: row R0 + qy (+ 2),
        // column C + qx
        const bool col_ok = g == 0 && s < t.nsteps && tx < NTX && C + qx < W;
        const bool l0 = col_ok && R0 + qy < t.q1, l1 = col_ok && R0 + 2 + qy < t.q1;
        const int la = t.flip ? H - 1 - (R0 + qy) : R0 + qy;
        const int lb = t.flip ? H - 3 - (R0 + qy) : R0 + 2 + qy;
        const uint32_t lf0 = l0 ? (uint32_t)(la * A.Wm + C + qx) * (uint32_t)(4 * A.dil) : 0x80000000u;
        const uint32_t lf1 = l1 ? (uint32_t)(lb * A.Wm + C + qx) * (uint32_t)(4 * A.dil) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse0), lrs, lf0, 0, kQO);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse1), lrs, lf1, 0, kQO);
      }
      const int y1 = gbase + 4 * (s + 1), y3 = gbase + 4 * (s + 3);
      commit(gc, y1, y1 <= hiL, hiL + 1);
      issue(gc, y3, y3 <= hiL);
    };
    // Two steps per iteration so that register sets are fixed: the group of
    // step s + 1 sits in set (s + 1) % 2, the query slices of step s in
    // (qa, qb)[s % 2].  The first pair runs before the loop, so that the
    // loop is entered with the same operations in flight as on its back
    // edge.
    step(0, set1, qa0, qa1);
    if (t.nsteps > 1) {
      step(1, set0, qb0, qb1);
      int s = 2;
      for (; s + 1 < t.nsteps; s += 2) {
        step(s, set1, qa0, qa1);
        step(s + 1, set0, qb0, qb1);
      }
      if (s < t.nsteps) step(s, set1, qa0, qa1);
    }
  }
}

// m: the map's shape; c: the class map (m.H / d x m.W / d, dilation 1).
template <typename T, int KS, int NTX, bool STRIPS>
hipError_t launch_stream_t(const void *q, const void *k, const void *v, const void *rpb,
                           void *out, float *lse, const Shape &m, const Shape &c,
                           const ByteStrides &si, const ByteStrides &so, hipStream_t st) {
  using G = StreamGeo<KS, NTX, STRIPS>;
  StreamArgs a;
  a.s = c;
  a.si = ByteStrides{si.b, si.h, si.y * (uint32_t)m.dil, si.x * (uint32_t)m.dil};
  a.so = ByteStrides{so.b, so.h, so.y * (uint32_t)m.dil, so.x * (uint32_t)m.dil};
  a.dil = m.dil;
  a.Hm = m.H;
  a.Wm = m.W;
  a.oyi = (int)si.y;
  a.oxi = (int)si.x;
  a.oyo = (int)so.y;
  a.oxo = (int)so.x;
  a.nstrip = (c.W + G::CW - 1) / G::CW;
  const int64_t columns = (int64_t)m.B * m.heads * m.dil * m.dil * a.nstrip;
  // workgroups per compute unit: as many as its LDS holds, at most two
  // waves per SIMD (eight per compute unit)
  const int per_cu = std::max(1, std::min(160 * 1024 / G::LDS, 8 / G::WAVES));
  const int cus = device_compute_units() * per_cu;
  // rows per unit: a multiple of 4, split until there are about as many
  // units as workgroups that run at once
  int nseg = 1;
  while (columns * (nseg + 1) <= cus && (c.H + nseg) / (nseg + 1) >= 12) ++nseg;
  a.seg = (((c.H + nseg - 1) / nseg) + 3) & ~3;
  a.nseg = (c.H + a.seg - 1) / a.seg;
  const int64_t nunits = columns * a.nseg;
  if (nunits > INT_MAX) return hipErrorInvalidConfiguration;
  a.nunits = (int)nunits;
  a.fseg = make_fastdiv((uint32_t)a.nseg);
  a.fheads = make_fastdiv((uint32_t)m.heads);
  a.fdil = make_fastdiv((uint32_t)m.dil);
  a.fstrip = make_fastdiv((uint32_t)a.nstrip);
  const int grid = (int)(nunits < cus ? nunits : cus);
  auto kern = m.dil == 1 ? (lse ? stream_mfma_kernel<T, KS, NTX, true, true, STRIPS>
                                 : stream_mfma_kernel<T, KS, NTX, false, true, STRIPS>)
                         : (lse ? stream_mfma_kernel<T, KS, NTX, true, false, STRIPS>
                                : stream_mfma_kernel<T, KS, NTX, false, false, STRIPS>);
  kern<<<dim3((unsigned)grid), G::THREADS, 0, st>>>((const T *)q, (const T *)k, (const T *)v,
                                                    (const T *)rpb, (T *)out, lse, a);
  return hipGetLastError();
}

template <typename T, int KS>
hipError_t launch_stream_k(const void *q, const void *k, const void *v, const void *rpb,
                           void *out, float *lse, const Shape &m, const ByteStrides &si,
                           const ByteStrides &so, hipStream_t st) {
  Shape c = m;
  c.H = m.H / m.dil;
  c.W = m.W / m.dil;
  c.dil = 1;
  // one wave per 8-column tile column of the class map; wider maps in
  // strips of 56 columns
  if (c.W > 56) return launch_stream_t<T, KS, 7, true>(q, k, v, rpb, out, lse, m, c, si, so, st);
  switch ((c.W + 7) / 8) {
    case 1: return launch_stream_t<T, KS, 1, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
    case 2: return launch_stream_t<T, KS, 2, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
    case 3: return launch_stream_t<T, KS, 3, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
    case 4: return launch_stream_t<T, KS, 4, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
    case 5: return launch_stream_t<T, KS, 5, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
    case 6: return launch_stream_t<T, KS, 6, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
    default: return launch_stream_t<T, KS, 7, false>(q, k, v, rpb, out, lse, m, c, si, so, st);
  }
}

}  // namespace

// Maps (with dilation d: residue classes, all of one size when d divides H
// and W) on which the kernel beats the block-tiled one as measured: at k = 7
// those 33 columns wide or wider and at least 16 rows high (narrower or
// shorter classes spend a large share of their keys on clamped edge windows
// and too few rows to hide a unit's first window); at k = 3 and 5 any map at
// least one window and 4 rows high, several workgroups sharing a compute
// unit when the map is 32 columns wide or narrower.
bool stream_mfma_supported(const Shape &s, na2d_dtype_t dt) {
  if (dt != NA2D_DTYPE_BF16 && dt != NA2D_DTYPE_F16) return false;
  if (s.ks != 3 && s.ks != 5 && s.ks != 7) return false;
  if (s.H % s.dil != 0 || s.W % s.dil != 0) return false;
  const int hc = s.H / s.dil, wc = s.W / s.dil;
  if (s.ks == 7) return wc > 32 && hc >= 16;
  return wc >= s.ks && hc >= s.ks && hc >= 4;
}

hipError_t launch_stream_mfma(const void *q, const void *k, const void *v, const void *rpb,
                              void *out, float *lse, const Shape &s, const ByteStrides &si,
                              const ByteStrides &so, na2d_dtype_t dt, hipStream_t st) {
  if (dt == NA2D_DTYPE_BF16) {
    switch (s.ks) {
      case 3: return launch_stream_k<__bf16, 3>(q, k, v, rpb, out, lse, s, si, so, st);
      case 5: return launch_stream_k<__bf16, 5>(q, k, v, rpb, out, lse, s, si, so, st);
      default: return launch_stream_k<__bf16, 7>(q, k, v, rpb, out, lse, s, si, so, st);
    }
  }
  switch (s.ks) {
    case 3: return launch_stream_k<_Float16, 3>(q, k, v, rpb, out, lse, s, si, so, st);
    case 5: return launch_stream_k<_Float16, 5>(q, k, v, rpb, out, lse, s, si, so, st);
    default: return launch_stream_k<_Float16, 7>(q, k, v, rpb, out, lse, s, si, so, st);
  }
}

}  // namespace na2d
