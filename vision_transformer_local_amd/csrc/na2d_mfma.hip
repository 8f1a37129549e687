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
//   * A workgroup owns an RY x RX block of one class of one (batch, head)
//     plane.  It stages the block's key/value halo -- the union of its
//     queries' clamped windows, at most (RY+k-1) x (RX+k) sub-grid pixels --
//     in LDS once: K as [row][col] 64-byte pixels (16-byte chunks swizzled by
//     column against bank conflicts) and V transposed to [row][channel][col]
//     so the matrix cores can contract over pixels.  The LDS strides are
//     compile-time constants; rows past the staged halo are zero-filled, so
//     every LDS address in the tile loop is a per-lane base plus an immediate
//     offset and no index is clamped.
//   * A wave processes 16-query tiles (TY x TX sub-grid pixels).  The tile's
//     keys are NB = TY + k - 1 halo rows x 16 columns (the columns start at an
//     even LDS column so V reads are dword aligned).  Scores are produced
//     transposed, S^T = K . Q^T, one v_mfma_f32_16x16x32 per halo row, so
//     each lane ends up holding scores of ONE query: the softmax reductions
//     need two lane swaps, and the probabilities are already laid out as the
//     B operand of the second product out^T = V^T . P^T.
//   * The relative-position bias (pre-multiplied by sqrt(D)) and the window
//     mask (-inf outside the query's clamped window) enter as the accumulator
//     input of the score MFMA.  For tiles whose windows are all unclamped this
//     input is the same for every tile of the workgroup and is computed once.
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
  static constexpr int RY = KS <= 7 ? 28 : (KS <= 11 ? 8 : 16);  // block rows
  static constexpr int RX = KS <= 7 ? 8 : (KS <= 11 ? 8 : 4);    // block columns
  static constexpr int THREADS = KS <= 7 ? 512 : 256;            // workgroup size
  static constexpr int WAVES = THREADS / 64;
  static constexpr int NB = TY + KS - 1;          // key rows per tile (even)
  static constexpr int HRM = RY + KS - 1;         // halo rows (max)
  static constexpr int HCM = (RX + KS + 1) & ~1;  // halo columns (max, even)
  static constexpr int ROWS = HRM + TY;           // LDS rows incl. zero rows read by tiles
  static constexpr int COLS = HCM % 4 == 2 ? HCM : HCM + 2;  // odd dword count per V^T row
  static constexpr int SIDE = 2 * KS - 1;
  static constexpr int MARGIN = TY * SIDE + 32;  // keeps masked bias reads in bounds
  // Interior accumulator table: entry (u, w), u = key row - query row within
  // the tile's key block (-(TY-1)..NB-1), w = key column - query column
  // (-TX..15), holds bias * sqrt(D) inside the k x k window and -inf outside.
  static constexpr int IU = NB + TY - 1, IW = 16 + TX;
  static_assert(TX + KS <= 16, "key columns do not cover the tile");
  static_assert(NB % 2 == 0, "PV consumes key rows in pairs");
};

constexpr int kThreads = 256;  // whole-sub-grid kernel
constexpr int kWaves = kThreads / 64;
constexpr float kSqrtD = 5.656854249492380f;  // sqrt(32)

// Maximum over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename T, int KS>
__global__ __launch_bounds__(Geometry<KS>::THREADS) void fused_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, Shape s, FastDiv fdil, FastDiv fnbx,
    FastDiv fnby, FastDiv fheads, int total) {
  using G = Geometry<KS>;
  constexpr int kThreads = G::THREADS, kWaves = G::WAVES;
  using vec = typename Mma<T>::vec;
  constexpr int TY = G::TY, TX = G::TX, RY = G::RY, RX = G::RX, NB = G::NB;
  constexpr int SIDE = G::SIDE, MARGIN = G::MARGIN, ROWS = G::ROWS, COLS = G::COLS;
  constexpr int HCM = G::HCM;
  constexpr int D = kHeadDim;
  // V^T: [channel][row][column pair]; an odd channel stride (in dwords)
  // spreads the 16 channels one wave reads over distinct banks.
  constexpr int CROW = COLS / 2;                            // dwords per channel row
  constexpr int CSTRD = (ROWS * CROW) | 1;                  // dwords per channel
  constexpr int R = KS / 2;

  __shared__ u32x4 k_lds[ROWS * HCM * 4];            // [row][col][chunk ^ swz]
  __shared__ unsigned int vt_lds[D * CSTRD];         // [channel][row][col pair]
  __shared__ float b_lds[SIDE * SIDE + 2 * MARGIN];  // bias * sqrt(D), zero margins
  __shared__ float i_lds[G::IU * G::IW];             // interior accumulator table

  const int tid = threadIdx.x;
  const int dil = s.dil;
  uint32_t id = xcd_contiguous_id(blockIdx.x, total);
  uint32_t t = fast_div(id, fdil);
  const int rx = id - t * dil;
  id = t;
  t = fast_div(id, fnbx);
  const int bx = id - t * fnbx.div;
  id = t;
  t = fast_div(id, fnby);
  const int by = id - t * fnby.div;
  id = t;
  t = fast_div(id, fdil);
  const int ry = id - t * dil;
  const int64_t plane = t;
  const int h = (int)(t - fast_div(t, fheads) * fheads.div);

  const int Ly = class_len(s.H, ry, dil), Lx = class_len(s.W, rx, dil);
  const int rc0 = by * RY, cc0 = bx * RX;
  if (rc0 >= Ly || cc0 >= Lx) return;  // this class has fewer rows/columns
  const int rc1 = min(rc0 + RY, Ly), cc1 = min(cc0 + RX, Lx);
  // Halo = union of the block's windows (window starts are monotone).
  const int hy0 = window_start(rc0, Ly, KS), hy1 = window_start(rc1 - 1, Ly, KS) + KS;
  const int hx0 = window_start(cc0, Lx, KS);
  const int hx0e = hx0 & ~1;  // even LDS column origin
  const int HR = hy1 - hy0;

  const int64_t hw = (int64_t)s.H * s.W;
  const T *kp = k + plane * hw * D;
  const T *vp = v + plane * hw * D;

  // ---- stage bias, K and V^T -------------------------------------------
  // Each thread owns one (column, 16-byte chunk) slot of a halo row and walks
  // down the rows, so a load address is a uniform base plus a 32-bit offset
  // that grows by one uniform row stride per pass.  All global loads of the
  // workgroup are issued before any of them is consumed, so their latencies
  // overlap.  Rows past the halo (up to ROWS) are written as zeros.
  constexpr int KIPR = HCM * 4;             // K chunks per halo row
  constexpr int KRP = kThreads / KIPR;      // K rows per pass
  constexpr int KPASS = (ROWS + KRP - 1) / KRP;
  constexpr int VIPR = (COLS / 2) * 4;      // V (pixel pair, chunk) items per row
  constexpr int VRP = kThreads / VIPR;      // V rows per pass
  constexpr int VPASS = (ROWS + VRP - 1) / VRP;
  constexpr int NTY = (RY + TY - 1) / TY, NTX = (RX + TX - 1) / TX;  // tile grid of a block
  constexpr int NTILE = NTY * NTX;
  constexpr int QIT = (NTILE + kWaves - 1) / kWaves;  // Q tiles per wave
  static_assert(KRP >= 1 && VRP >= 1, "halo row wider than the workgroup");
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 15, g = lane >> 4;
  const int qy = ql / TX, qx = ql % TX;
  const int nty = (rc1 - rc0 + TY - 1) / TY, ntx = (cc1 - cc0 + TX - 1) / TX;

  // uniform: pixel of halo row 0, LDS column 0 (sub-grid (hy0, hx0e)), in bytes
  const int64_t org = (int64_t)(ry + hy0 * dil) * s.W + rx + hx0e * dil;
  const char *kb0 = (const char *)(kp + org * D);
  const char *vb0 = (const char *)(vp + org * D);
  const unsigned rowb = (unsigned)dil * (unsigned)s.W * (unsigned)(D * sizeof(T));
  const unsigned colb = (unsigned)dil * (unsigned)(D * sizeof(T));
  const int cmax = Lx - 1 - hx0e;  // last real column, relative to the LDS origin

  const int kr0 = min(tid / KIPR, KRP - 1), kcol = (tid % KIPR) >> 2, kch = tid & 3;
  const bool kact = tid < KRP * KIPR;
  const unsigned koff = (unsigned)min(kcol, cmax) * colb + kch * 16;
  // Loads are unconditional (rows clamped into the halo) so that they form
  // one straight-line batch; the LDS writes below decide data versus zero.
  u32x4 kreg[KPASS];
  {
    const unsigned first = koff + (unsigned)kr0 * rowb, last = koff + (unsigned)(HR - 1) * rowb;
#pragma unroll
    for (int it = 0; it < KPASS; ++it)
      kreg[it] = *(const u32x4 *)(kb0 + min(first + (unsigned)(it * KRP) * rowb, last));
  }
  const int vr0 = min(tid / VIPR, VRP - 1), vpair = (tid % VIPR) >> 2, vch = tid & 3;
  const bool vact = tid < VRP * VIPR;
  const unsigned voff0 = (unsigned)min(2 * vpair, cmax) * colb + vch * 16;
  const unsigned voff1 = (unsigned)min(2 * vpair + 1, cmax) * colb + vch * 16;
  u32x4 va[VPASS], vbr[VPASS];
  {
    const unsigned r0 = (unsigned)vr0 * rowb, rl = (unsigned)(HR - 1) * rowb;
#pragma unroll
    for (int it = 0; it < VPASS; ++it) {
      const unsigned ro = min(r0 + (unsigned)(it * VRP) * rowb, rl);
      va[it] = *(const u32x4 *)(vb0 + (voff0 + ro));
      vbr[it] = *(const u32x4 *)(vb0 + (voff1 + ro));
    }
  }
  // this wave's query rows, one 16-byte slice per lane and tile
  u32x4 qreg[QIT];
#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int tile = min(wave + it * kWaves, NTILE - 1);
    const int ty = tile / NTX, tx = tile % NTX;
    const int ci = min(rc0 + ty * TY + qy, rc1 - 1), cj = min(cc0 + tx * TX + qx, cc1 - 1);
    qreg[it] = *(const u32x4 *)(q + plane * hw * D +
                                ((int64_t)(ry + ci * dil) * s.W + rx + cj * dil) * D + g * 8);
  }

  for (int e = tid; e < SIDE * SIDE + 2 * MARGIN; e += kThreads) {
    const int t = e - MARGIN;
    float b = 0.f;
    if (rpb != nullptr && t >= 0 && t < SIDE * SIDE)
      b = Elem<T>::to_f(rpb[(int64_t)h * SIDE * SIDE + t]) * kSqrtD;
    b_lds[e] = b;
  }
  for (int e = tid; e < G::IU * G::IW; e += kThreads) {
    const int u = e / G::IW - (TY - 1), w = e % G::IW - TX;
    float b = -INFINITY;
    if ((unsigned)u < (unsigned)KS && (unsigned)w < (unsigned)KS)
      b = rpb != nullptr ? Elem<T>::to_f(rpb[((int64_t)h * SIDE + u + R) * SIDE + w + R]) * kSqrtD
                         : 0.f;
    i_lds[e] = b;
  }
  // Rows past the halo only need finite values (every key there is masked):
  // the clamped loads above hold real pixels, so all rows are written as is.
  {
    u32x4 *dst = k_lds + (kr0 * HCM + kcol) * 4 + (kch ^ ((kcol >> 1) & 3));
#pragma unroll
    for (int it = 0; it < KPASS; ++it) {
      const int row = kr0 + it * KRP;
      if (kact && row < ROWS) dst[it * KRP * HCM * 4] = kreg[it];
    }
  }
  {
    unsigned int *dst = vt_lds + (vch * 8) * CSTRD + vr0 * CROW + vpair;
#pragma unroll
    for (int it = 0; it < VPASS; ++it) {
      const int row = vr0 + it * VRP;
      if (vact && row < ROWS) {
        const u32x4 a = va[it], b = vbr[it];
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // dword w of a chunk = channels 2w, 2w+1
          dst[it * VRP * CROW + (2 * w) * CSTRD] = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);
          dst[it * VRP * CROW + (2 * w + 1) * CSTRD] =
              __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);
        }
      }
    }
  }
  __syncthreads();

  // ---- 16-query tiles ----------------------------------------------------
  const float c2 = kLog2e / kSqrtD;  // exp(S - Smax) = exp2((acc - accmax) * c2)
  const int chA = 8 * (ql >> 2) + (ql & 3);  // V^T channel of this lane (+4 for block 1)
  vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);

  // Accumulator input for tiles whose 16 windows are all unclamped: the mask
  // and bias then depend only on the lane, and on the (per-block constant)
  // parity shift dlt between the tile's first window column and its even
  // LDS column.
  const int dlt = ((cc0 - R) - hx0e) & 1;
  f32x4 cint[NB];
  {
    const float *tb = i_lds + (TY - 1 - qy) * G::IW + (TX + 4 * g - dlt - qx);
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) cint[a][i] = tb[a * G::IW + i];
  }

#pragma unroll
  for (int it = 0; it < QIT; ++it) {
    const int tile = wave + it * kWaves;
    if (tile >= NTILE) break;
    const int ty = tile / NTX, tx = tile % NTX;
    if (ty >= nty || tx >= ntx) continue;  // tile outside a ragged block
    const int tci0 = rc0 + ty * TY, tcj0 = cc0 + tx * TX;
    int ci = tci0 + qy, cj = tcj0 + qx;
    const bool valid = ci < rc1 && cj < cc1;
    ci = min(ci, rc1 - 1);  // ragged tile: recompute a real query, store nothing
    cj = min(cj, cc1 - 1);
    const int Y0 = window_start(tci0, Ly, KS), X0 = window_start(tcj0, Lx, KS);
    const int X0a = X0 - ((X0 - hx0e) & 1);  // even LDS column
    const int lrow0 = Y0 - hy0, lcol0 = X0a - hx0e;

    const int64_t qoff =
        plane * hw * D + ((int64_t)(ry + ci * dil) * s.W + rx + cj * dil) * D + g * 8;
    const vec qv = __builtin_bit_cast(vec, qreg[it]);

    // S^T rows: key (Y0 + a, X0a + 4g + i) against query ql, i = 0..3.
    const int kcol = lcol0 + ql;
    const u32x4 *kb = k_lds + (lrow0 * HCM + kcol) * 4 + (g ^ ((kcol >> 1) & 3));
    f32x4 sc[NB];
    const bool interior = tci0 - R >= 0 && tci0 + TY - 1 + R <= Ly - 1 && tcj0 - R >= 0 &&
                          tcj0 + TX - 1 + R <= Lx - 1;
    if (interior) {
#pragma unroll
      for (int a = 0; a < NB; ++a)
        sc[a] = Mma<T>::run(__builtin_bit_cast(vec, kb[a * HCM * 4]), qv, cint[a]);
    } else {
      const int sy = window_start(ci, Ly, KS), sx = window_start(cj, Lx, KS);
      const int rowrel = Y0 - sy, colrel = X0a + 4 * g - sx;
      const int bb = MARGIN + (Y0 - ci + KS - 1) * SIDE + (X0a + 4 * g - cj + KS - 1);
      float ccap[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ccap[i] = (unsigned)(colrel + i) < (unsigned)KS ? INFINITY : -INFINITY;
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const float rcap = (unsigned)(rowrel + a) < (unsigned)KS ? INFINITY : -INFINITY;
        f32x4 c;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = fminf(fminf(b_lds[bb + a * SIDE + i], rcap), ccap[i]);
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

    // out^T = V^T . P^T over pairs of key rows (32 keys per MFMA); a third
    // product against an all-ones matrix gives every lane its query's
    // denominator, summed over exactly the 16-bit weights used above.
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f}, o2 = {0.f, 0.f, 0.f, 0.f};
    const unsigned int *vb = vt_lds + chA * CSTRD + lrow0 * CROW + ((lcol0 + 4 * g) >> 1);
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) {
      vec pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<T>(sc[2 * j][i]);
        pb[4 + i] = static_cast<T>(sc[2 * j + 1][i]);
      }
      const unsigned int *r0 = vb + (2 * j) * CROW, *r1 = r0 + CROW;
      constexpr int C4 = 4 * CSTRD;  // channel + 4
      const u32x4 w0 = {r0[0], r0[1], r1[0], r1[1]};
      const u32x4 w1 = {r0[C4], r0[C4 + 1], r1[C4], r1[C4 + 1]};
      o0 = Mma<T>::run(__builtin_bit_cast(vec, w0), pb, o0);
      o1 = Mma<T>::run(__builtin_bit_cast(vec, w1), pb, o1);
      o2 = Mma<T>::run(ones, pb, o2);
    }
    const float l = o2[0];

    // lane holds channels 8g..8g+3 (o0) and 8g+4..8g+7 (o1) of query ql
    if (valid) {
      const float inv = __builtin_amdgcn_rcpf(l);
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

  const int lane = tid & 63, wave = tid >> 6;
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

template <typename T, int KS>
hipError_t launch_t(const void *q, const void *k, const void *v, const void *rpb, void *out,
                    const Shape &s, hipStream_t st) {
  using G = Geometry<KS>;
  const int Lymax = class_len(s.H, 0, s.dil), Lxmax = class_len(s.W, 0, s.dil);
  const int nby = (Lymax + G::RY - 1) / G::RY, nbx = (Lxmax + G::RX - 1) / G::RX;
  const int64_t total = (int64_t)s.B * s.heads * s.dil * s.dil * nby * nbx;
  if (total > INT_MAX) return hipErrorInvalidConfiguration;
  fused_mfma_kernel<T, KS><<<dim3((unsigned)total), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (T *)out, s,
      make_fastdiv((uint32_t)s.dil), make_fastdiv((uint32_t)nbx), make_fastdiv((uint32_t)nby),
      make_fastdiv((uint32_t)s.heads), (int)total);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, hipStream_t st, bool *supported) {
  const bool pow2_dil = (s.dil & (s.dil - 1)) == 0;
  if ((int64_t)s.ks * s.dil == s.H && (int64_t)s.ks * s.dil == s.W && pow2_dil) {
    switch (s.ks) {
      case 3: return launch_dense<T, 3>(q, k, v, rpb, out, s, st);
      case 5: return launch_dense<T, 5>(q, k, v, rpb, out, s, st);
      case 7: return launch_dense<T, 7>(q, k, v, rpb, out, s, st);
    }
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
  if (dt == NA2D_DTYPE_BF16) return launch_dtype<__bf16>(q, k, v, rpb, out, s, st, supported);
  if (dt == NA2D_DTYPE_F16) return launch_dtype<_Float16>(q, k, v, rpb, out, s, st, supported);
  *supported = false;
  return hipSuccess;
}

}  // namespace na2d
