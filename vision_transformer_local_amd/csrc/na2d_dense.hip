// na2d_dense.hip -- fused forward pass for maps whose residue classes are
// exactly k x k (H == W == k*d, d a power of two): every query attends to its
// whole class.  See the comment on dense_mfma_kernel.
#include "na2d_mfma_common.h"

#include <limits.h>

namespace na2d {
namespace {

using namespace mfma;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------------------
// Whole-class windows: H == k*d and W == k*d (d a power of two).
//
// Then every residue class is exactly k x k and every query's clamped window
// is its entire class, so the operator is dense attention with a bias inside
// each class (the NAT README's self-attention equivalence, applied per
// class).  A class is flattened: its N = k*k queries form NT tiles of 16 and
// its N keys NKB blocks of 16; key slots past N hold copies of the last key
// and get -inf, query slots past N recompute the last query and store
// nothing.  The MFMA accumulator input of a (tile, key block) pair -- bias *
// sqrt(D), -inf on padding -- is the same for every class of a head: it sits
// in an LDS table, one 16-byte entry per lane, rebuilt when the head changes.
//
// Work decomposition: classes are numbered head-major, (h, b, ry, rx) with
// rx fastest, and cut into blocks of SG classes that never straddle two
// heads.  Workgroups are persistent (one per compute unit), walk a contiguous
// run of blocks and keep two LDS buffers: while the 16 waves compute block i
// (TPW tiles each) from one buffer, the direct global->LDS path fills the
// other with block i+1.  K and V are staged as [class][key slot] 64-byte
// pixels, the 16-byte chunks XOR-swizzled by slot; the PV product reads V^T
// with ds_read_b64_tr_b16 as in the general kernel.
template <int KS> struct DenseGeometry {
  static constexpr int N = KS * KS;
  static constexpr int NT = (N + 15) / 16;              // query tiles per class
  static constexpr int NKB = ((N + 15) / 16 + 1) & ~1;  // key blocks (even: PV pairs)
  static constexpr int NK = NKB * 16;                   // key slots per class
  static constexpr int WAVES = 16, THREADS = WAVES * 64;
  static constexpr int TPW = 1;                         // tiles per wave
  static constexpr int SG = WAVES * TPW / NT;           // classes per block
  static constexpr int CB = NK * 64;                    // bytes per class and tensor
  static constexpr int DPT = SG * NK / 16;              // DMA instructions per tensor
  static constexpr int DPW = 2 * DPT / WAVES;           // ... per wave
  static constexpr int NCT = NT * NKB * 64 * 4;         // accumulator-table floats
  static constexpr int SIDE = 2 * KS - 1;
  static_assert(SG * NT == WAVES * TPW, "blocks hold whole classes");
  static_assert(DPW * WAVES == 2 * DPT, "DMA instructions spread evenly");
  static_assert(2 * 2 * SG * CB + 2 * NCT * 4 <= 160 * 1024, "LDS");
};

// Byte offset of pixel (0, 0) of class jh (numbered (b, ry, rx), rx fastest)
// of head h, for a view with byte strides st.
__device__ __forceinline__ int64_t class_base(int h, int jh, const Shape &s, int log2d,
                                              const ByteStrides &st) {
  const int d = s.dil;
  const int rx = jh & (d - 1), ry = (jh >> log2d) & (d - 1), b = jh >> (2 * log2d);
  return b * st.b + h * st.h + (int64_t)(ry * st.y + rx * st.x);
}

// Byte offset of the (batch, head) plane of class jh of head h.
__device__ __forceinline__ int64_t plane_base(int h, int jh, int log2d, const ByteStrides &st) {
  return (int64_t)(jh >> (2 * log2d)) * st.b + h * st.h;
}

// Key and value of padded pixels when the caller gives no pad vectors.
__device__ __attribute__((aligned(64))) const char kZeroPixel[64] = {};

// Block id -> (head, first class within the head, classes in the block).
// Blocks of one head are consecutive (f divides by the blocks per head),
// or, when the heads of a pixel share its lines (channels-last maps), the
// heads alternate (f divides by the head count), so that the heads' blocks
// of the same classes run back to back and share those lines in L2.
struct DenseBlock {
  int h, j0, n;
};

template <int KS>
__device__ __forceinline__ DenseBlock dense_block(int id, const FastDiv &f, int per_head,
                                                  bool hfast) {
  using G = DenseGeometry<KS>;
  DenseBlock b;
  const int t = (int)fast_div((uint32_t)id, f), r = id - t * (int)f.div;
  b.h = hfast ? r : t;
  b.j0 = (hfast ? t : r) * G::SG;
  b.n = min(G::SG, per_head - b.j0);
  return b;
}

// PAD: the map is padded to k*d x k*d (maybe_pad); pixels at row >= s.H or
// column >= s.W are staged from the head's pad vectors and their queries are
// neither read nor written.
template <typename T, int KS, bool PAD, bool LSE>
__global__ __launch_bounds__(DenseGeometry<KS>::THREADS) void dense_mfma_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ rpb, T *__restrict__ out, Shape s, ByteStrides si, ByteStrides so,
    FastDiv fblk, bool hfast, int per_head, int nblocks, int log2d,
    const T *__restrict__ pad_k, const T *__restrict__ pad_v, float *__restrict__ lse) {
  using G = DenseGeometry<KS>;
  using vec = typename Mma<T>::vec;
  constexpr int N = G::N, NT = G::NT, NKB = G::NKB, NK = G::NK, TPW = G::TPW, SG = G::SG;
  constexpr int CB = G::CB, DPT = G::DPT, DPW = G::DPW, SIDE = G::SIDE;
  constexpr int WAVES = G::WAVES, THREADS = G::THREADS;
  __shared__ __attribute__((aligned(16))) char kbuf0[SG * CB], vbuf0[SG * CB];
  __shared__ __attribute__((aligned(16))) char kbuf1[SG * CB], vbuf1[SG * CB];
  // two accumulator tables, [slot][tile][key block][lane][4]; head h uses slot
  // h & 1, so alternating heads (channels-last order) rebuild nothing
  __shared__ __attribute__((aligned(16))) float ctab[2 * G::NCT];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15, g = lane >> 4;
  const int wg = xcd_contiguous_id(blockIdx.x, gridDim.x);
  const int b0 = (int)((int64_t)nblocks * wg / gridDim.x);
  const int b1 = (int)((int64_t)nblocks * (wg + 1) / gridDim.x);
  if (b0 >= b1) return;
  const int d = s.dil;
  const unsigned rowb = (unsigned)d * si.y, colb = (unsigned)d * si.x;

  // ---- per-lane constants: DMA slots, query positions ----
  // DMA instruction i = wave + WAVES * m covers 16 key slots (4 lanes each)
  // of one class of one tensor; lane l lands at slot kg*16 + l/4, 16-byte
  // position l&3, which holds logical chunk (l&3) ^ swz(slot).
  unsigned doff[DPW];
  int drow[DPW], dcol[DPW], dlch[DPW];  // padded maps: the key's pixel offsets in its class
#pragma unroll
  for (int m = 0; m < DPW; ++m) {
    const int i = wave + WAVES * m, it = i % DPT;
    const int kg = it % (NK / 16);
    const int slot = kg * 16 + (lane >> 2), key = min(slot, N - 1);
    const int lch = (lane & 3) ^ ((slot >> 1) & 3);
    doff[m] = (unsigned)(key / KS) * rowb + (unsigned)(key % KS) * colb + lch * 16u;
    drow[m] = (key / KS) * d;
    dcol[m] = (key % KS) * d;
    dlch[m] = lch * 16;
  }
  // this wave's tiles: tile t = wave*TPW + u of the block is tile t % NT of
  // class t / NT; lane query slot tt*16 + ql (clamped to the last query)
  unsigned qoff[TPW], ooff[TPW];  // in q and in out
  int qrow[TPW], qcol[TPW];        // padded maps: the query's pixel offsets in its class
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tt = (wave * TPW + u) % NT;
    const int nq = min(tt * 16 + ql, N - 1);
    qoff[u] = (unsigned)(nq / KS) * rowb + (unsigned)(nq % KS) * colb;
    ooff[u] = (unsigned)(nq / KS) * ((unsigned)d * so.y) + (unsigned)(nq % KS) * ((unsigned)d * so.x);
    qrow[u] = (nq / KS) * d;
    qcol[u] = (nq % KS) * d;
  }
  // whether pixel (row, col) of class jh lies inside the unpadded map
  auto real = [&](int jh, int row, int col) -> bool {
    const int rx = jh & (d - 1), ry = (jh >> log2d) & (d - 1);
    return ry + row < s.H && rx + col < s.W;
  };

  // accumulator table for head h: entry (tt, kb, lane, i) = bias * sqrt(D)
  // of key slot kb*16 + 4g + i against query slot tt*16 + ql, -inf on
  // padding keys
  constexpr int CPT = (G::NCT + THREADS - 1) / THREADS;  // entries per thread
  auto ctab_src = [&](int e) -> int {  // rpb index of entry e, or -1 for -inf
    const int i = e & 3, l = (e >> 2) & 63, kb = (e >> 8) % NKB, tt = (e >> 8) / NKB;
    const int nk = kb * 16 + 4 * (l >> 4) + i;
    const int nq = min(tt * 16 + (l & 15), N - 1);
    if (nk >= N) return -1;
    return (nk / KS - nq / KS + KS - 1) * SIDE + (nk % KS - nq % KS + KS - 1);
  };
  T craw[CPT];
  auto load_ctab = [&](int h) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int e = min(tid + m * THREADS, G::NCT - 1);
      craw[m] = rpb != nullptr ? rpb[(int64_t)h * SIDE * SIDE + max(ctab_src(e), 0)]
                               : static_cast<T>(0.0f);
    }
  };
  auto store_ctab = [&](int slot) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int e = tid + m * THREADS;
      if (e < G::NCT)
        ctab[slot * G::NCT + e] = ctab_src(e) < 0 ? -INFINITY : Elem<T>::to_f(craw[m]) * kSqrtD;
    }
  };

  // ---- per-wave addresses of a block: the bases of the wave's copies and of
  // its tiles in q and out (uniform).  They are formed a round ahead, so
  // that the scalar arithmetic sits beside the previous block's compute and
  // the copies a barrier releases go out right after it.
  struct Addr {
    DenseBlock bk;
    const char *src[DPW];   // copy m: the class base in k or v (+ doff[m] per lane)
    int jh[DPW];            // copy m: its class (padded maps)
    int64_t qb[TPW], ob[TPW];  // tile u: its class base in q and in out
  };
  auto addr = [&](int id) -> Addr {
    Addr a;
    a.bk = dense_block<KS>(id, fblk, per_head, hfast);
#pragma unroll
    for (int m = 0; m < DPW; ++m) {
      const int i = wave + WAVES * m;
      const int c = (i % DPT) / (NK / 16);
      a.jh[m] = a.bk.j0 + min(c, a.bk.n - 1);
      a.src[m] = (const char *)(i >= DPT ? v : k) + class_base(a.bk.h, a.jh[m], s, log2d, si);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int jt = a.bk.j0 + min((wave * TPW + u) / NT, a.bk.n - 1);
      a.qb[u] = class_base(a.bk.h, jt, s, log2d, si);
      a.ob[u] = class_base(a.bk.h, jt, s, log2d, so);
    }
    return a;
  };
  // ---- staging of one block into a buffer ----
  auto stage = [&](const Addr &a, char *kb, char *vb) {
#pragma unroll
    for (int m = 0; m < DPW; ++m) {
      const int i = wave + WAVES * m;
      const bool isv = i >= DPT;
      const int it = i % DPT, c = it / (NK / 16), kg = it % (NK / 16);
      const char *src = a.src[m] + doff[m];
      if constexpr (PAD) {
        if (!real(a.jh[m], drow[m], dcol[m])) {
          const T *pv = isv ? pad_v : pad_k;
          src = (pv != nullptr ? (const char *)(pv + a.bk.h * kHeadDim) : kZeroPixel) + dlch[m];
        }
      }
      char *dst = (isv ? vb : kb) + c * CB + kg * 1024;
      __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)dst, 16, 0, 0);
    }
  };
  auto load_q = [&](const Addr &a, int u) -> u32x4 {
    if constexpr (PAD) {
      // a padded query is never stored: read pixel (0, 0) of its plane instead
      const int jh = a.bk.j0 + min((wave * TPW + u) / NT, a.bk.n - 1);
      if (!real(jh, qrow[u], qcol[u]))
        return *(const u32x4 *)((const char *)q + plane_base(a.bk.h, jh, log2d, si) + g * 16u);
    }
    return *(const u32x4 *)((const char *)q + a.qb[u] + qoff[u] + g * 16u);
  };

  const float c2 = kLog2e / kSqrtD;
  vec ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = static_cast<T>(1.0f);

  // LDS byte offsets are formed as one integer per lane and kept opaque, so
  // that every read is (array + offset) + constant: the compiler then still
  // knows which array it reads and does not wait for the DMA into the other
  // buffer before it.
  auto opaque = [](int x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  // one tile: returns the lane's 8 output channels, rounded, and (when lse
  // is given) the query's log-sum-exp in tlse
  auto tile = [&](const char *kb, const char *vb, int u, u32x4 qraw, int slot,
                  float &tlse) -> u32x4 {
    const int t = wave * TPW + u, c = t / NT, tt = t % NT;
    const vec qv = __builtin_bit_cast(vec, qraw);
    // key slot kbk*16 + ql, logical chunk g (the swizzle does not depend on kbk)
    const char *kp = kb + opaque(c * CB + ql * 64 + 16 * (g ^ ((ql >> 1) & 3)));
    const f32x4 *ct = (const f32x4 *)((const char *)ctab +
                                      opaque(slot * G::NCT * 4 + ((tt * NKB) * 64 + lane) * 16));
    f32x4 sc[NKB];
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) {
      const u32x4 kv = *(const u32x4 *)(kp + kbk * 1024);
      sc[kbk] = Mma<T>::run(__builtin_bit_cast(vec, kv), qv, ct[kbk * 64]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kbk][i]);
    mx = group_max(mx);
    const float mc = mx * c2;
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[kbk][i] = __builtin_amdgcn_exp2f(fmaf(sc[kbk][i], c2, -mc));
    if constexpr (LSE) {  // the fp32 weights' sum (not the 16-bit one the output is divided by)
      float l = 0.f;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int i = 0; i < 4; ++i) l += sc[kbk][i];
      tlse = window_lse(mc, group_sum(l));
    }
    // out^T = V^T . P^T, 32 keys per MFMA: P^T rows 8g'..8g'+7 are key slots
    // 32j + 4g' + 0..3 and 32j + 16 + 4g' + 0..3.  As a source of the
    // transposing read, lane (g, 4kk + qd) reads channels 4qd..4qd+3 (+16
    // for the second channel block) of slot 32j + 4g + kk (+16).
    // slot 32j + 4g + kk (+16 for the second half); its swizzle does not
    // depend on j
    const int qd = ql & 3, kk = ql >> 2, sl = 4 * g + kk, z = (sl >> 1) & 3;
    const int vrow = c * CB + sl * 64 + 8 * (qd & 1);
    const char *va = vb + opaque(vrow + 16 * ((qd >> 1) ^ z));
    const char *vc2 = vb + opaque(vrow + 16 * (((qd >> 1) | 2) ^ z));
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f}, o2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NKB / 2; ++j) {
      vec pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<T>(sc[2 * j][i]);
        pb[4 + i] = static_cast<T>(sc[2 * j + 1][i]);
      }
      const u32x2 a0 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(va + 2048 * j)));
      const u32x2 a1 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(va + 2048 * j + 1024)));
      const u32x2 c0 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vc2 + 2048 * j)));
      const u32x2 c1 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vc2 + 2048 * j + 1024)));
      o0 = Mma<T>::run(__builtin_bit_cast(vec, u32x4{a0[0], a0[1], a1[0], a1[1]}), pb, o0);
      o1 = Mma<T>::run(__builtin_bit_cast(vec, u32x4{c0[0], c0[1], c1[0], c1[1]}), pb, o1);
      o2 = Mma<T>::run(ones, pb, o2);
    }
    const float inv = __builtin_amdgcn_rcpf(o2[0]);
    typedef __attribute__((ext_vector_type(4))) T vec4;
    vec4 r0, r1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r0[i] = static_cast<T>(o0[i] * inv);
      r1[i] = static_cast<T>(o1[i] * inv);
    }
    const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
    return u32x4{w0[0], w0[1], w1[0], w1[1]};
  };
  // whether this lane's query of tile u exists in block bk
  auto tile_ok = [&](const DenseBlock &bk, int u) -> bool {
    const int t = wave * TPW + u, c = t / NT, tt = t % NT;
    bool ok = c < bk.n && tt * 16 + ql < N;
    if constexpr (PAD) ok = ok && real(bk.j0 + min(c, bk.n - 1), qrow[u], qcol[u]);
    return ok;
  };
  auto store = [&](const Addr &a, int u, u32x4 val, bool ok, float tlse) {
    if (ok) {
      char *o = (char *)out + a.ob[u] + ooff[u] + g * 8u;
      *(u32x2 *)o = u32x2{val[0], val[1]};
      *(u32x2 *)(o + 16 * sizeof(T)) = u32x2{val[2], val[3]};
      // with dense q, the query's index in [B, heads, H, W] order is its q
      // byte offset over the pixel's D channels
      if (LSE && g == 0)
        lse[(a.qb[u] + qoff[u]) / (kHeadDim * sizeof(T))] = tlse;
    }
  };

  // ---- prologue ----
  Addr acur = addr(b0);
  u32x4 qcur[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) qcur[u] = load_q(acur, u);
  load_ctab(acur.bk.h);
  stage(acur, kbuf0, vbuf0);
  store_ctab(acur.bk.h & 1);
  int slot_h[2] = {-1, -1};  // head whose table each slot holds
  slot_h[acur.bk.h & 1] = acur.bk.h;
  Addr anxt = addr(min(b0 + 1, b1 - 1));
  __syncthreads();

  u32x4 res[TPW];
  bool rok[TPW];
  float rlse[TPW];
  // One block from (kc, vc) while the next is staged into (kn, vn); called
  // with fixed arrays so that the compiler can tell the DMA target from the
  // buffer being read.
  auto step = [&](int bi, const char *kc, const char *vc, char *kn, char *vn) {
    const bool more = bi + 1 < b1;
    if (more) stage(anxt, kn, vn);
    u32x4 qnxt[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) qnxt[u] = load_q(anxt, u);
    const DenseBlock &cur = acur.bk, &nxt = anxt.bk;
    const int nslot = nxt.h & 1;
    const bool newtab = more && slot_h[nslot] != nxt.h;
    if (newtab) load_ctab(nxt.h);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      rok[u] = tile_ok(cur, u);
      rlse[u] = 0.f;
      res[u] = (wave * TPW + u) / NT < cur.n ? tile(kc, vc, u, qcur[u], cur.h & 1, rlse[u])
                                             : u32x4{0u, 0u, 0u, 0u};
    }
    if (!more) return;
    const Addr a2 = addr(min(bi + 2, b1 - 1));  // the round after next
    if (newtab) {
      // the slot the current block reads: wait until every wave is done with
      // it (the other slot was last read before the previous barrier)
      if (nslot == (cur.h & 1)) __syncthreads();
      store_ctab(nslot);
      slot_h[nslot] = nxt.h;
    }
    __syncthreads();  // also waits for the DMA (workgroup fence)
    // results leave after the barrier, whose wait then covers only the loads
#pragma unroll
    for (int u = 0; u < TPW; ++u) store(acur, u, res[u], rok[u], rlse[u]);
    acur = anxt;
    anxt = a2;
#pragma unroll
    for (int u = 0; u < TPW; ++u) qcur[u] = qnxt[u];
  };
  for (int bi = b0; bi < b1; bi += 2) {
    step(bi, kbuf0, vbuf0, kbuf1, vbuf1);
    if (bi + 1 >= b1) break;
    step(bi + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) store(acur, u, res[u], rok[u], rlse[u]);  // the last block
}

template <typename T, int KS>
hipError_t launch_dense(const void *q, const void *k, const void *v, const void *rpb, void *out,
                        const Shape &s, const ByteStrides &si, const ByteStrides &so,
                        const Pad &pad, hipStream_t st, float *lse) {
  using G = DenseGeometry<KS>;
  const int64_t per_head = (int64_t)s.B * s.dil * s.dil;  // classes of one head
  const int64_t bph = (per_head + G::SG - 1) / G::SG;      // blocks per head
  const int64_t nblocks = bph * s.heads;
  if (nblocks > INT_MAX || per_head > INT_MAX) return hipErrorInvalidConfiguration;
  int log2d = 0;
  while ((1 << log2d) < s.dil) ++log2d;
  const int64_t grid = nblocks < device_compute_units() ? nblocks : device_compute_units();
  // heads interleaved within pixels: alternate heads between blocks
  const bool hfast = s.heads > 1 && (uint64_t)si.h < si.x;
  const bool padded = pad.Hp > s.H || pad.Wp > s.W;
  // (padded maps come without lse: the caller checks)
  auto kernel = padded ? dense_mfma_kernel<T, KS, true, false>
                       : (lse ? dense_mfma_kernel<T, KS, false, true>
                              : dense_mfma_kernel<T, KS, false, false>);
  kernel<<<dim3((unsigned)grid), G::THREADS, 0, st>>>(
      (const T *)q, (const T *)k, (const T *)v, (const T *)rpb, (T *)out, s, si, so,
      make_fastdiv((uint32_t)(hfast ? s.heads : bph)), hfast, (int)per_head, (int)nblocks, log2d,
      (const T *)pad.k, (const T *)pad.v, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_mfma(const void *q, const void *k, const void *v, const void *rpb,
                             void *out, const Shape &s, const ByteStrides &si,
                             const ByteStrides &so, const Pad &pad, na2d_dtype_t dt,
                             hipStream_t st, bool *supported, float *lse) {
  *supported = true;
  const bool pow2_dil = (s.dil & (s.dil - 1)) == 0;
  // the (padded) map must be exactly k*d square: every class k x k
  if ((int64_t)s.ks * s.dil != pad.Hp || (int64_t)s.ks * s.dil != pad.Wp || !pow2_dil ||
      (s.ks != 3 && s.ks != 5 && s.ks != 7) || dt == NA2D_DTYPE_F32 ||
      (lse != nullptr && (pad.Hp > s.H || pad.Wp > s.W))) {
    *supported = false;
    return hipSuccess;
  }
  if (dt == NA2D_DTYPE_BF16) {
    switch (s.ks) {
      case 3: return launch_dense<__bf16, 3>(q, k, v, rpb, out, s, si, so, pad, st, lse);
      case 5: return launch_dense<__bf16, 5>(q, k, v, rpb, out, s, si, so, pad, st, lse);
      default: return launch_dense<__bf16, 7>(q, k, v, rpb, out, s, si, so, pad, st, lse);
    }
  }
  switch (s.ks) {
    case 3: return launch_dense<_Float16, 3>(q, k, v, rpb, out, s, si, so, pad, st, lse);
    case 5: return launch_dense<_Float16, 5>(q, k, v, rpb, out, s, si, so, pad, st, lse);
    default: return launch_dense<_Float16, 7>(q, k, v, rpb, out, s, si, so, pad, st, lse);
  }
}

}  // namespace na2d
