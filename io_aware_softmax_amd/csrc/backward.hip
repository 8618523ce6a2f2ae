// Attention backward (dQ, dK, dV) for fp16 / bf16 on gfx950 MFMA.
//
// The comfyai.app chapter "6.3 FlashAttention" notes (after "A simple
// implementation w/ C++", and in "Computation and GPU Memory") that for
// training the method keeps no score or weight matrix from the forward and
// recomputes them in the backward pass.  Here the weights are recomputed
// tile by tile from the per-row log-sum-exp the forward already writes:
// P_ij = exp(a_ij - lse_i), so no running maximum is needed.  With
// Dv_i = sum_d dO_id O_id (which equals sum_j P_ij dP_ij, since O = P V),
// the chain rule of O = softmax(a) V, a = scale Q K^T gives
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - Dv),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Nothing of size L x L reaches device memory.
//
// Three kernels on one stream:
//   * stats: per 64-query tile, lse in base-2 units and Dv (one pass over
//     O and dO); padded rows get lse = +inf and Dv = 0, so their weights
//     and score gradients are exactly zero downstream;
//   * dK/dV: one workgroup per 128 keys (4 waves x 32 keys held in VGPRs as
//     MFMA B operands), streaming 64-query tiles of Q, dO and the stats
//     through LDS by DMA, double buffered; dK and dV accumulate in registers;
//   * dQ: one workgroup per 128 queries (4 waves x 32 queries, Q and dO in
//     VGPRs), streaming 64-key tiles of K and V; dQ accumulates in
//     registers.  No atomics: every output element has one writer, and the
//     result does not depend on scheduling.
//
// Q, dO (dK/dV kernel) and K (dQ kernel) are read from LDS both along rows
// (A operand of a product over D) and across rows (B operand of a product
// over the tile's rows, ds_read_b64_tr_b16).  Tiles are stored unpadded with
// each 16-byte chunk c of row r at chunk c ^ swz(r): both read patterns are
// then free of bank conflicts (16 lanes reading one chunk of 16 rows hit 16
// different 4-bank groups; a half-wave's 4 rows x 64 B transposed read hits
// 64 different banks).
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "attn_internal.hpp"
#include "mask_dropout.hpp"
#include "mfma_tile.hpp"
#include "swz_tile.hpp"

namespace attn {
namespace {

using namespace mt;
using namespace st;

constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr int BW = 128;   // rows owned by a workgroup (4 waves x 32)
constexpr int kStatFloats = 2 * BQ;  // per stats tile: lse2[64], then -Dv[64]

// One stats tile (512 B) into LDS; lanes 32-63 fetch the same bytes again
// into the following 512 B (a whole instruction, never read).
__device__ __forceinline__ void dma_stats(const float* src, char* dst, int lane) {
  const unsigned off = 16u * (unsigned)(lane & 31);
  dma_run<1>(uniform_ptr(reinterpret_cast<const char*>(src)), &off, lds_addr(dst));
}

template <bool BF16>
__device__ __forceinline__ float load16(const unsigned short* p) {
  const unsigned short b = *p;
  if constexpr (BF16)
    return __builtin_bit_cast(float, (unsigned)b << 16);
  else
    return (float)__builtin_bit_cast(_Float16, b);
}


// ---------------------------------------------------------------------------
// stats: lse2 = lse * log2(e) and -Dv = -rowsum(dO o O), tile-blocked.  Dv
// is stored negated: the dP products of the kernels below start their
// accumulation from it (dP - Dv without a subtraction per element).
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(NT) void bwd_stats_kernel(BwdArgs a) {
  const int tile = blockIdx.x;  // bh * nqt + t
  const int nqt = (a.Lq + BQ - 1) / BQ;
  const int bh = tile / nqt, t = tile % nqt;
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int qi = t * BQ + r;
  float acc = 0.f;
  if (qi < a.Lq) {
    const size_t row = ((size_t)bh * a.Lq + qi) * D + part * (D / 4);
    if constexpr (DT == 0) {
      const float* o = static_cast<const float*>(a.o) + row;
      const float* g = static_cast<const float*>(a.dout) + row;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) acc = __builtin_fmaf(o[i], g[i], acc);
    } else {
      const unsigned short* o = static_cast<const unsigned short*>(a.o) + row;
      const unsigned short* g = static_cast<const unsigned short*>(a.dout) + row;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) acc = __builtin_fmaf(load16<DT == 2>(o + i), load16<DT == 2>(g + i), acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (part == 0) {
    float* st = a.stats + (size_t)tile * kStatFloats;
    st[r] = qi < a.Lq ? a.lse[(size_t)bh * a.Lq + qi] * kLog2e : INFINITY;
    st[BQ + r] = qi < a.Lq ? -acc : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys, loop over 64-query tiles.
// ---------------------------------------------------------------------------

// One whole, unmasked 64-query tile of a wave as a fixed sequence of MFMA
// slots (one wave per SIMD, so the overlap of matrix and vector work has to
// be in the instruction order):
//   slots [0, NS)          S_0 = Q_0 K^T and dP_0 = dO_0 V^T (block 0)
//   slots [NS, 2 NS)       S_1, dP_1, while the VALU turns S_0, dP_0 into
//                          P_0 and dS_0 (two row elements per slot)
//   slots [2 NS, 2NS + NG) dV += P_0^T dO_0, dK += dS_0^T Q_0, while the
//                          VALU turns block 1 into P_1, dS_1
//   slots [2NS + NG, N)    dV += P_1^T dO_1, dK += dS_1^T Q_1
// Each slot issues its MFMA, its VALU share, the LDS reads of the slot PF
// ahead and (through `hook`) now and then one DMA instruction of the next
// tile; a scheduling fence keeps the slots in this order.
template <int D>
struct BwdSlots {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int NS = 2 * KS;       // S and dP MFMAs of one block
  static constexpr int NG = 4 * DB;       // dV and dK MFMAs of one block
  static constexpr int N = 2 * NS + 2 * NG;
  static constexpr int PF = 4;            // read lookahead in slots
  // Elements go in pairs (one packed conversion each), pair k of block b at
  // slot E_b + k, one slot after the block's last S / dP product.
  static constexpr int E0 = NS + 1;
  static constexpr int E1 = 2 * NS + 1;
  static constexpr int PFS = 3;           // stats read lookahead in slots
  // Pairs 0-3 (elements 0-7) feed a block's first dV/dK k-step, pairs 4-7
  // the second; each must be ready before that k-step's first slot.
  static_assert(E0 + 3 < 2 * NS && E0 + 7 < 2 * NS + NG / 2, "block 0 elements late");
  static_assert(E1 + 3 < 2 * NS + NG && E1 + 7 < 2 * NS + NG + NG / 2, "block 1 elements late");
};


template <bool BF16, int D, class Hook>
__device__ __forceinline__ void dkdv_tile_fast(const char* Qs, const char* dOs, const float* st,
                                               const s16x8 (&kreg)[D / 16], const s16x8 (&vreg)[D / 16],
                                               f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                               const unsigned (&ra)[D / 16], const unsigned (&ta)[D / 32][2],
                                               int h, float c, Hook&& hook) {
  using T = SwzTile<D>;
  using S = BwdSlots<D>;
  s16x8 fr[S::N];
  f32x16 sc[2], dp[2];
  float2 l2[2][8];  // lse2 of element pair k, read PFS slots ahead
  // -Dv of the block's 16 queries in accumulator order: the dP products
  // start from it, so they end at dP - Dv.
  f32x16 nd[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float* src = st + BQ + 32 * b + 16 * half + 8 * h;
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      nd[b][8 * half + 0] = x0.x; nd[b][8 * half + 1] = x0.y; nd[b][8 * half + 2] = x0.z; nd[b][8 * half + 3] = x0.w;
      nd[b][8 * half + 4] = x1.x; nd[b][8 * half + 5] = x1.y; nd[b][8 * half + 6] = x1.z; nd[b][8 * half + 7] = x1.w;
    }
  s16x8 pa[2][2], sa[2][2];
  auto read = [&](int i) __attribute__((always_inline)) {
    if (i < 2 * S::NS) {
      const int b = i / S::NS, j = i % S::NS;
      fr[i] = *reinterpret_cast<const s16x8*>(((j & 1) ? dOs : Qs) + 32 * b * T::PITCH + ra[j >> 1]);
    } else {
      const int x = i - 2 * S::NS, b = x / S::NG, j = x % S::NG;
      const int s2 = j / (2 * S::DB), r = j % (2 * S::DB), db = r >> 1;
      const char* src = ((r & 1) ? Qs : dOs) + (32 * b + 16 * s2) * T::PITCH;
      const s16x4 lo = lds_read_tr(src + ta[db][0]);
      const s16x4 hi = lds_read_tr(src + ta[db][1]);
      fr[i] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // Elements 2k, 2k+1 of block b are queries 32 b + 16 (k / 4) + 8 h +
  // 2 (k % 4) + {0, 1} (consecutive: one 8-byte read each of lse2 and Dv).
  auto stats = [&](int b, int k) __attribute__((always_inline)) {
    const int q = 32 * b + 16 * (k >> 2) + 8 * h + 2 * (k & 3);
    l2[b][k] = *reinterpret_cast<const float2*>(st + q);
  };
  auto pair = [&](int b, int k) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 2 * k + u;
      const float lse2 = u ? l2[b][k].y : l2[b][k].x;
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][e], c, -lse2));
      pa[b][e >> 3][e & 7] = (short)round16<BF16>(p);
      sa[b][e >> 3][e & 7] = (short)round16<BF16>(p * dp[b][e]);  // dp holds dP - Dv
    }
  };
  static_for<S::PF>([&](auto I) __attribute__((always_inline)) { read(I); });
  __builtin_amdgcn_sched_barrier(0);
  static_for<S::N>([&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    if (i + S::PF < S::N) read(i + S::PF);
    if (i + S::PFS >= S::E0 && i + S::PFS < S::E0 + 8) stats(0, i + S::PFS - S::E0);
    if (i + S::PFS >= S::E1 && i + S::PFS < S::E1 + 8) stats(1, i + S::PFS - S::E1);
    if (i < 2 * S::NS) {
      const int b = i / S::NS, j = i % S::NS, t = j >> 1;
      if (j & 1)
        dp[b] = mfma32<BF16>(fr[i], vreg[t], t == 0 ? nd[b] : dp[b]);
      else
        sc[b] = mfma32<BF16>(fr[i], kreg[t], t == 0 ? f32x16{} : sc[b]);
    } else {
      const int x = i - 2 * S::NS, b = x / S::NG, j = x % S::NG;
      const int s2 = j / (2 * S::DB), r = j % (2 * S::DB), db = r >> 1;
      if (r & 1)
        dk[db] = mfma32<BF16>(sa[b][s2], fr[i], dk[db]);
      else
        dv[db] = mfma32<BF16>(pa[b][s2], fr[i], dv[db]);
    }
    if (i >= S::E0 && i < S::E0 + 8) pair(0, i - S::E0);
    if (i >= S::E1 && i < S::E1 + 8) pair(1, i - S::E1);
    hook(I);
    __builtin_amdgcn_sched_barrier(0);
  });
}
// KIND (mask kind: 0 none, 1 boolean, 2 additive) and DROP (dropout): with
// either, the slot-scheduled fast path is off and every tile goes block by
// block; each variant carries only its own per-element work.
template <bool BF16, int D, bool CAUSAL, int KIND, bool DROP>
__global__ __launch_bounds__(NT, 1) void bwd_dkdv_kernel(BwdArgs a, MaskDropout md) {
  constexpr bool EX = KIND != 0 || DROP;
  using T = SwzTile<D>;
  constexpr int KS = D / 16;  // k-steps of a product over D
  constexpr int DB = D / 32;  // 32-column blocks of D
  constexpr int STAGE = 2 * T::BYTES + 1024;  // Q tile, dO tile, stats
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int li = lane & 15, g = lane >> 4;
  const int Lq = a.Lq, Lk = a.Lk;
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int nkb = (Lk + BW - 1) / BW;
  const int nqt = (Lq + BQ - 1) / BQ;
  // Workgroups are dealt to the 8 XCDs round robin: consecutive key blocks
  // of one head (which stream the same Q / dO) share an XCD and its L2.
  // Causal: the first key blocks see the most queries and go first.
  // With a mask shared by the heads (mask_h == 1) and whole heads per XCD,
  // an XCD's workgroups take one key block of each of its heads in turn, so
  // that the heads running together read the same mask columns.
  const int total = a.BH * nkb;
  const int wg = blockIdx.x;
  int bh, kb;
  if (KIND != 0 && md.mask_h == 1 && a.BH % 8 == 0) {
    const int hx = a.BH / 8, r = wg / 8;
    bh = (wg % 8) * hx + r % hx;
    kb = r / hx;
  } else {
    const int logical = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
    bh = logical / nkb;
    kb = logical % nkb;
  }
  const int k0 = kb * BW, kw0 = k0 + 32 * w;
  const int t_begin = CAUSAL ? max(0, k0 - off) / BQ : 0;

  const unsigned short* Kg = static_cast<const unsigned short*>(a.k) + (size_t)bh * Lk * D;
  const unsigned short* Vg = static_cast<const unsigned short*>(a.v) + (size_t)bh * Lk * D;
  const char* Qb = static_cast<const char*>(a.q) + (size_t)bh * Lq * D * 2;
  const char* dOb = static_cast<const char*>(a.dout) + (size_t)bh * Lq * D * 2;
  const float* Sb = a.stats + (size_t)bh * nqt * kStatFloats;

  auto issue = [&](int t, char* stage) {
    const int q0 = t * BQ;
    const int rows_left = min(BQ, Lq - q0);
    dma_swz_tile<D>(Qb + (size_t)q0 * D * 2, stage, w, lane, rows_left);
    dma_swz_tile<D>(dOb + (size_t)q0 * D * 2, stage + T::BYTES, w, lane, rows_left);
    if (w == 0) dma_stats(Sb + (size_t)t * kStatFloats, stage + 2 * T::BYTES, lane);
  };
  issue(t_begin, smem);

  // K and V rows of this wave as B operands: lane (n, h) holds
  // X[kw0 + n][16 t + 8 h .. + 8].  Keys past Lk are zero (never stored).
  const int key = kw0 + n;
  s16x8 kreg[KS], vreg[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
    if (key < Lk) {
      xk = *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + 16 * t + 8 * h);
      xv = *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + 16 * t + 8 * h);
    }
    kreg[t] = __builtin_bit_cast(s16x8, xk);
    vreg[t] = __builtin_bit_cast(s16x8, xv);
  }
  // Wait for these loads here, before the tile loop: otherwise the compiler
  // (which does not count the DMA issued by inline assembly) puts a full
  // vmcnt(0) wait at their first use inside the loop, on every tile, and
  // that wait also drains the next tile's DMA just issued.
#pragma unroll
  for (int t = 0; t < KS; ++t) asm volatile("" ::"v"(kreg[t]), "v"(vreg[t]));

  // Per-lane LDS offsets.  Row reads (A operands over D): row perm_row(n),
  // chunk 2 t + h.  Transposed reads (B operands over queries): rows
  // 8 h + li / 4 (+ 4 for the upper half), bytes 64 db + 32 (g & 1) +
  // 8 (li & 3) of the unswizzled row.
  const int prow = perm_row(n);
  unsigned ra[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) ra[t] = prow * T::PITCH + 16 * ((2 * t + h) ^ T::swz(prow));
  unsigned ta[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 8 * h + (li >> 2) + 4 * hi;
      const int chunk = 4 * db + 2 * (g & 1) + ((li & 3) >> 1);
      ta[db][hi] = row * T::PITCH + 16 * (chunk ^ T::swz(row)) + 8 * (li & 1);
    }

  const size_t mslab = KIND != 0 ? mask_slab(md, bh, Lq, Lk) : 0;
  const size_t mask_lane_off = (size_t)(8 * h) * Lk + (unsigned)key;  // lane part of a mask element's index
  const PhiloxKey pk{md.k0, md.k1};

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float c = a.c;

  // Index of mask element r of the 32-query block starting at query qb:
  // query qb + c + 8 h (c = 16 (r / 8) + r % 8) of key `key`.  The row
  // starts at a wave-uniform address (row index clamped to Lq - 1, so in
  // bounds); the lane adds 8 h rows and its key, or nothing outside
  // [0, Lq) x [0, Lk).  Selects, no multiply under a lane condition (which
  // compiled to divergent branches).
  auto mask_idx = [&](int qb, int r) __attribute__((always_inline)) -> size_t {
    const int ru = qb + 16 * (r >> 3) + (r & 7);
    const bool in = ru + 8 * h < Lq && key < Lk;
    return mslab + (size_t)min(ru, Lq - 1) * Lk + (in ? mask_lane_off : 0);
  };
  // Boolean masks: the 32 bytes of a tile's two blocks are loaded one tile
  // ahead, before that tile's Q / dO DMA is issued.  The compiler does not
  // count the DMA (inline assembly), so waiting for mask loads issued after
  // it would also wait for the DMA; loaded before it and consumed after the
  // landing wait, they cost no wait inside the tile.
  constexpr bool PREF = KIND == 1;
  auto mask_prefetch = [&](int q0, unsigned char (&m)[2][16]) __attribute__((always_inline)) {
    const unsigned char* m8 = static_cast<const unsigned char*>(md.mask);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) m[b][r] = m8[mask_idx(q0 + 32 * b, r)];
  };
  auto mask_landed = [&](const unsigned char (&m)[2][16]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" ::"v"((unsigned)m[b][r]));
  };

  // One 32-query block b of the tile in `stage` (mraw: its prefetched
  // boolean mask bytes).
  auto block = [&](const char* stage, int q0, int b, const unsigned char (&mraw)[16]) __attribute__((always_inline)) {
    const int qb = q0 + 32 * b;
    if (qb >= Lq) return;
    if (CAUSAL && qb + 31 + off < kw0) return;  // no query of the block sees a key of the wave
    const char* Qs = stage;
    const char* dOs = stage + T::BYTES;
    const float* st = reinterpret_cast<const float*>(stage + 2 * T::BYTES);
    // Mask terms and dropout keep bits do not depend on the products: they
    // come first so that their loads and VALU work overlap the MFMAs.
    // Mask terms (base 2) of the 16 elements, from branch-free loads.
    float mt[16];
    if constexpr (EX) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mt[r] = 0.f;
    }
    if constexpr (KIND != 0) {
      // The term of an element outside [0, Lq) x [0, Lk) is whatever
      // in-bounds byte it read (mask_idx): a padded query row has
      // lse2 = +inf (weight 0 whatever the term), and a key past Lk only
      // feeds its own dK / dV row, which is never stored.  (A term that
      // depends on the range flag let the compiler sink a load into a branch
      // that waited for every load in flight.)
      if constexpr (KIND == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mt[r] = mraw[r] == 0 ? -INFINITY : 0.f;
      } else {
        const float* m32 = static_cast<const float*>(md.mask);
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = m32[mask_idx(qb, r)];
#pragma unroll
        for (int r = 0; r < 16; ++r) mt[r] = v[r] * kLog2e;
      }
    }
    // Dropout keep bits of the 16 elements (bit r).  Element r needs the
    // half (key mod 2) of word ((key mod 8) / 2) of the Philox block of
    // (key / 8, query of r).  The 8 lanes n = 8m .. 8m + 7 of a half-wave hold
    // the 8 keys of one block column and need the same 16 blocks.  Lane
    // u = n mod 8 computes the blocks of r = u and r = 8 + u: each gives the
    // keep bits of the 8 keys for one query, one byte (bit e: key 8m + e).
    // The 8 lanes then transpose their two 8 x 8 bit matrices at once in three
    // butterfly stages (k = 4, 2, 1): lanes u and u ^ k swap the k-bit
    // groups that sit on the wrong side, after which lane u holds bit r = the
    // keep bit of its own key for the query of r.  Lane exchanges are DPP
    // moves (xor 1 and 2: quad permutations; xor 4: the half-row mirror,
    // u -> 7 - u, then the quad permutation u -> u ^ 3); selections are bit
    // masks (a lane-dependent ternary chain here becomes divergent branches).
    unsigned kbits = 0xFFFFu;
    if constexpr (DROP) {
      const unsigned u = (unsigned)n & 7u;
      unsigned x = 0u;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int qi = qb + 16 * t + 8 * h + (int)u;  // query of r = 8 t + u
        const uint4 wd = philox4x32_10(make_uint4((unsigned)key >> 3, (unsigned)qi, (unsigned)bh, md.offset), pk);
        x |= keep_bits8(wd, md.thr) << (8 * t);
      }
      static_for<3>([&](auto S) __attribute__((always_inline)) {
        constexpr int k = 4 >> decltype(S)::value;
        constexpr unsigned lo = k == 4 ? 0x0F0Fu : (k == 2 ? 0x3333u : 0x5555u);
        unsigned y;
        if constexpr (k == 4) {
          y = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
          y = (unsigned)__builtin_amdgcn_mov_dpp((int)y, 0x1B, 0xF, 0xF, false);   // quad_perm [3,2,1,0]
        } else if constexpr (k == 2) {
          y = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
        } else {
          y = (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
        }
        const unsigned a = (x & lo) | ((y & lo) << k);     // lanes with bit k of u clear
        const unsigned b = (x & ~lo) | ((y >> k) & lo);    // lanes with bit k of u set
        const unsigned m = 0u - ((u / k) & 1u);
        x = (b & m) | (a & ~m);
      });
      kbits = x & 0xFFFFu;
    }
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      s = mfma32<BF16>(*reinterpret_cast<const s16x8*>(Qs + 32 * b * T::PITCH + ra[t]), kreg[t], s);
      dp = mfma32<BF16>(*reinterpret_cast<const s16x8*>(dOs + 32 * b * T::PITCH + ra[t]), vreg[t], dp);
    }
    if constexpr (DROP) {
      // Interleave the Philox rounds with the 16 products: after the first
      // operand reads, each MFMA is followed by one operand read and ~16
      // VALU instructions, which issue while the MFMA runs.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      static_for<2 * KS>([&](auto) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
      });
    }
    // Register r holds query qb + 16 (r / 8) + 8 h + r % 8 of key kw0 + n.
    float l2[16], dd[16];  // lse2 and -Dv of the block's queries
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int base = 32 * b + 16 * hh + 8 * h;
      *reinterpret_cast<float4*>(l2 + 8 * hh) = *reinterpret_cast<const float4*>(st + base);
      *reinterpret_cast<float4*>(l2 + 8 * hh + 4) = *reinterpret_cast<const float4*>(st + base + 4);
      *reinterpret_cast<float4*>(dd + 8 * hh) = *reinterpret_cast<const float4*>(st + BQ + base);
      *reinterpret_cast<float4*>(dd + 8 * hh + 4) = *reinterpret_cast<const float4*>(st + BQ + base + 4);
    }
    const bool masked = CAUSAL && qb + off < kw0 + 31;
    if constexpr (!EX) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mt[r] = 0.f;
    }
    s16x8 pa[2], sa[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = qb + 16 * (r >> 3) + 8 * h + (r & 7);
      // A masked-out element takes exponent -inf (weight 0) by a select
      // before the exponential: a row with every key masked has lse2 = -inf,
      // where mt - lse2 would be NaN.
      const float xe = __builtin_fmaf(s[r], c, mt[r] - l2[r]);
      float p = __builtin_amdgcn_exp2f(mt[r] == -INFINITY ? -INFINITY : xe);
      if (masked && key > qi + off) p = 0.f;
      // Dropout: the value product sees the kept weights scaled by 1/(1-p),
      // and dP reaches the softmax through the same factors.
      float pv = p, dpk = dp[r];
      if constexpr (DROP) {
        const float z = ((kbits >> r) & 1u) ? md.rp : 0.f;
        pv = p * z;
        dpk = dpk * z;
      }
      const float ds = p * (dpk + dd[r]);  // dd holds -Dv
      pa[r >> 3][r & 7] = (short)round16<BF16>(pv);
      sa[r >> 3][r & 7] = (short)round16<BF16>(ds);
    }
    // dV += P^T dO and dK += dS^T Q over the block's 32 queries (2 k-steps).
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int rowoff = (32 * b + 16 * s2) * T::PITCH;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 glo = lds_read_tr(dOs + rowoff + ta[db][0]);
        const s16x4 ghi = lds_read_tr(dOs + rowoff + ta[db][1]);
        const s16x4 qlo = lds_read_tr(Qs + rowoff + ta[db][0]);
        const s16x4 qhi = lds_read_tr(Qs + rowoff + ta[db][1]);
        const s16x8 gf = s16x8{glo[0], glo[1], glo[2], glo[3], ghi[0], ghi[1], ghi[2], ghi[3]};
        const s16x8 qf = s16x8{qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
        dv[db] = mfma32<BF16>(pa[s2], gf, dv[db]);
        dk[db] = mfma32<BF16>(sa[s2], qf, dk[db]);
      }
    }
  };

  // Per-lane source offsets of this wave's DMA instructions for a whole tile.
  unsigned doff[T::PER_WAVE];
#pragma unroll
  for (int i = 0; i < T::PER_WAVE; ++i) {
    const int slot = (w * T::PER_WAVE + i) * 64 + lane;
    const int row = slot / T::CPR;
    doff[i] = (unsigned)row * (D * 2) + 16u * (unsigned)((slot % T::CPR) ^ T::swz(row));
  }

  // A whole tile (64 queries before Lq) whose first query sees every key of
  // the wave takes the slot schedule, with the next tile's DMA spread over
  // its first slots (Q, then dO, then the stats); on the last tile the DMA
  // fetches the current tile again into the idle stage (never read).  Other
  // tiles (causal diagonal, Lq tail) issue the next tile's DMA first and go
  // block by block.
  // FAST: the caller knows the tile takes the slot schedule.
  auto tile = [&](char* stage, int q0, char* nstage, int tn, const unsigned char (&mcur)[2][16],
                  unsigned char (&mnext)[2][16], auto fast_tag) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const bool has_next = tn < nqt;
    if constexpr (FAST) {
      const int tf = has_next ? tn : tn - 1;
      const int rows_left = min(BQ, Lq - tf * BQ);
      unsigned cur[T::PER_WAVE];
      if (rows_left == BQ) {
#pragma unroll
        for (int i = 0; i < T::PER_WAVE; ++i) cur[i] = doff[i];
      } else {
#pragma unroll
        for (int i = 0; i < T::PER_WAVE; ++i) {
          const int slot = (w * T::PER_WAVE + i) * 64 + lane;
          const int row = slot / T::CPR;
          cur[i] = (unsigned)min(row, rows_left - 1) * (D * 2) + 16u * (unsigned)((slot % T::CPR) ^ T::swz(row));
        }
      }
      const char* qsrc = Qb + (size_t)tf * BQ * D * 2;
      const char* gsrc = dOb + (size_t)tf * BQ * D * 2;
      const float* ssrc = Sb + (size_t)tf * kStatFloats;
      auto hook = [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        constexpr int k = (i - 1) / 2;  // DMA instruction k at slot 2 k + 1
        if constexpr (i % 2 == 1 && k < T::PER_WAVE) {
          dma_run<1>(qsrc, &cur[k], lds_addr(nstage + (w * T::PER_WAVE + k) * 1024));
        } else if constexpr (i % 2 == 1 && k < 2 * T::PER_WAVE) {
          dma_run<1>(gsrc, &cur[k - T::PER_WAVE], lds_addr(nstage + T::BYTES + (w * T::PER_WAVE + k - T::PER_WAVE) * 1024));
        } else if constexpr (i % 2 == 1 && k == 2 * T::PER_WAVE) {
          if (w == 0) dma_stats(ssrc, nstage + 2 * T::BYTES, lane);
        }
      };
      dkdv_tile_fast<BF16, D>(stage, stage + T::BYTES, reinterpret_cast<const float*>(stage + 2 * T::BYTES), kreg,
                              vreg, dk, dv, ra, ta, h, c, hook);
    } else {
      if constexpr (PREF) {
        if (has_next) mask_prefetch(tn * BQ, mnext);
      }
      if (has_next) issue(tn, nstage);
      block(stage, q0, 0, mcur[0]);
      block(stage, q0, 1, mcur[1]);
    }
  };

  unsigned char mA[2][16] = {}, mB[2][16] = {};
  if constexpr (PREF) mask_prefetch(t_begin * BQ, mA);
  land_all();
  if constexpr (PREF) mask_landed(mA);
  __syncthreads();
  // Tiles alternate between the two stages (tile t in stage (t - t_begin)
  // mod 2); each loop body covers a pair so that every LDS address is a lane
  // offset plus an immediate.  The tiles that take the slot schedule (whole,
  // unmasked, at or past the wave's causal diagonal) form one contiguous
  // range [t_lo, t_hi); the loops run the generic tiles before it, the
  // range, and the generic tiles after it, so that each loop has one code
  // path and the compiler one register assignment per loop (a branch
  // between the two paths inside one loop made it shuffle the dK / dV
  // accumulators between registers on every tile).  The slot loop starts at
  // an even stage: a range starting at an odd one gives its first tile to
  // the generic loop, and an odd tail goes to the last loop.  Every wave
  // passes one barrier per tile whichever loop it is in.
  const std::integral_constant<bool, true> fast{};
  const std::integral_constant<bool, false> generic{};
  int t_lo = nqt, t_hi = nqt;
  if constexpr (!EX) {
    const int first = CAUSAL ? max(t_begin, (max(0, kw0 + 31 - off) + BQ - 1) / BQ) : t_begin;
    const int last = Lq / BQ;  // tiles before it are whole
    if (first < last) {
      t_lo = first + ((first - t_begin) & 1);
      t_hi = t_lo + 2 * (max(0, last - t_lo) / 2);
      if (t_lo >= t_hi) t_lo = t_hi = nqt;  // no pair left: every tile generic
    }
  }
  t_lo = __builtin_amdgcn_readfirstlane(t_lo);
  t_hi = __builtin_amdgcn_readfirstlane(t_hi);
  auto pair = [&](int t, auto tag) __attribute__((always_inline)) -> bool {  // false: no tile after t
    tile(smem, t * BQ, smem + STAGE, t + 1, mA, mB, tag);
    land_all();
    if constexpr (PREF) mask_landed(mB);
    __syncthreads();
    if (t + 1 >= nqt) return false;
    tile(smem + STAGE, (t + 1) * BQ, smem, t + 2, mB, mA, tag);
    land_all();
    if constexpr (PREF) mask_landed(mA);
    __syncthreads();
    return true;
  };
  int t = t_begin;
  for (; t < t_lo; t += 2)  // (t_lo - t_begin) is even or t_lo == nqt
    if (!pair(t, generic)) break;
  if (t_lo < t_hi) {
    for (t = t_lo; t < t_hi; t += 2) pair(t, fast);
    for (; t < nqt; t += 2)
      if (!pair(t, generic)) break;
  }

  // Register r of block db holds key kw0 + 8 (r / 4) + 4 h + r % 4,
  // column 32 db + n.
  unsigned short* dKg = static_cast<unsigned short*>(a.dk) + (size_t)bh * Lk * D;
  unsigned short* dVg = static_cast<unsigned short*>(a.dv) + (size_t)bh * Lk * D;
  const float scale = a.scale;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = kw0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (kr < Lk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dKg[(size_t)kr * D + 32 * db + n] = round16<BF16>(dk[db][r] * scale);
        dVg[(size_t)kr * D + 32 * db + n] = round16<BF16>(dv[db][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 128 queries, loop over 64-key tiles.
// ---------------------------------------------------------------------------
template <bool BF16, int D, bool CAUSAL, int KIND, bool DROP>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(BwdArgs a, MaskDropout md) {
  constexpr bool EX = KIND != 0 || DROP;
  using T = SwzTile<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int STAGE = 2 * T::BYTES;  // K tile, V tile
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h = lane >> 5;
  const int li = lane & 15, g = lane >> 4;
  const int Lq = a.Lq, Lk = a.Lk;
  const int off = Lk - Lq;
  const int nqb = (Lq + BW - 1) / BW;
  const int nqt = (Lq + BQ - 1) / BQ;
  // Consecutive query blocks of one head share an XCD (same K / V);
  // causal: the last query blocks (the most keys) go first.
  // A mask shared by the heads: query blocks of the XCD's heads in turn,
  // as in the dK/dV kernel.
  const int total = a.BH * nqb;
  const int wg = blockIdx.x;
  int bh, qpos;
  if (KIND != 0 && md.mask_h == 1 && a.BH % 8 == 0) {
    const int hx = a.BH / 8, r = wg / 8;
    bh = (wg % 8) * hx + r % hx;
    qpos = r / hx;
  } else {
    const int logical = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
    bh = logical / nqb;
    qpos = logical % nqb;
  }
  const int qblk = CAUSAL ? nqb - 1 - qpos : qpos;
  const int q0 = qblk * BW, wq0 = q0 + 32 * w;
  const int q_last = min(q0 + BW, Lq) - 1;
  const int kv_end = CAUSAL ? min(Lk, q_last + off + 1) : Lk;
  const int nkt = (kv_end + BQ - 1) / BQ;
  // Keys this wave needs: [0, w_key_end).
  const int w_key_end = wq0 >= Lq ? 0 : (CAUSAL ? min(Lk, min(wq0 + 31, Lq - 1) + off + 1) : Lk);

  const char* Kb = static_cast<const char*>(a.k) + (size_t)bh * Lk * D * 2;
  const char* Vb = static_cast<const char*>(a.v) + (size_t)bh * Lk * D * 2;
  auto issue = [&](int j, char* stage) {
    const int kv0 = j * BQ;
    const int rows_left = min(BQ, Lk - kv0);
    dma_swz_tile<D>(Kb + (size_t)kv0 * D * 2, stage, w, lane, rows_left);
    dma_swz_tile<D>(Vb + (size_t)kv0 * D * 2, stage + T::BYTES, w, lane, rows_left);
  };
  issue(0, smem);

  // Q and dO rows of this wave as B operands: lane (n, h) holds
  // X[wq0 + n][16 t + 8 h .. + 8]; the lane's lse2 and Dv.
  const int qi = wq0 + n;
  const unsigned short* Qg = static_cast<const unsigned short*>(a.q) + (size_t)bh * Lq * D;
  const unsigned short* dOg = static_cast<const unsigned short*>(a.dout) + (size_t)bh * Lq * D;
  s16x8 qreg[KS], oreg[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    u32x4 xq = {0u, 0u, 0u, 0u}, xo = {0u, 0u, 0u, 0u};
    if (qi < Lq) {
      xq = *reinterpret_cast<const u32x4*>(Qg + (size_t)qi * D + 16 * t + 8 * h);
      xo = *reinterpret_cast<const u32x4*>(dOg + (size_t)qi * D + 16 * t + 8 * h);
    }
    qreg[t] = __builtin_bit_cast(s16x8, xq);
    oreg[t] = __builtin_bit_cast(s16x8, xo);
  }
  float l2 = INFINITY, dd = 0.f;  // lse2 and -Dv of the lane's query
  if (qi < Lq) {
    const float* st = a.stats + ((size_t)bh * nqt + qi / BQ) * kStatFloats;
    l2 = st[qi % BQ];
    dd = st[BQ + qi % BQ];
  }
  // Wait for these loads here, before the tile loop: otherwise the compiler
  // (which does not count the DMA issued by inline assembly) puts a full
  // vmcnt(0) wait at their first use inside the loop, which drains the next
  // tile's DMA right after its issue, on every tile.
#pragma unroll
  for (int t = 0; t < KS; ++t) asm volatile("" ::"v"(qreg[t]), "v"(oreg[t]));
  asm volatile("" ::"v"(l2), "v"(dd));
  // Row of the lane's query in the mask (row 0 of the slab for padded
  // queries: in bounds, never stored).
  const size_t mrow = KIND != 0 ? mask_slab(md, bh, Lq, Lk) + (size_t)(qi < Lq ? qi : 0) * Lk : 0;
  const PhiloxKey pk{md.k0, md.k1};

  const int prow = perm_row(n);
  unsigned ra[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) ra[t] = prow * T::PITCH + 16 * ((2 * t + h) ^ T::swz(prow));
  unsigned ta[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 8 * h + (li >> 2) + 4 * hi;
      const int chunk = 4 * db + 2 * (g & 1) + ((li & 3) >> 1);
      ta[db][hi] = row * T::PITCH + 16 * (chunk ^ T::swz(row)) + 8 * (li & 1);
    }

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};
  const float c = a.c;

  // One 32-key block b of the tile in `stage`.  MASKED: the tile may hold
  // keys past Lk or (causal) past the diagonal of some query of the wave.
  auto block = [&](const char* stage, int kv0, int b, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int kb0 = kv0 + 32 * b;
    if (kb0 >= w_key_end) return;
    const char* Ks = stage;
    const char* Vs = stage + T::BYTES;
    // Mask terms and keep bits first: independent of the products, their
    // loads and VALU work overlap the MFMAs.
    float mt[16];
    unsigned keep[2] = {0xffu, 0xffu};
#pragma unroll
    for (int r = 0; r < 16; ++r) mt[r] = 0.f;
    if constexpr (EX) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key0 = kb0 + 16 * half + 8 * h;
        if constexpr (KIND != 0)
          mask_terms8_kind<KIND>(md, mrow + key0, key0, Lk, Lk % 8 == 0 && kb0 + 32 <= Lk,
                                 *reinterpret_cast<float(*)[8]>(mt + 8 * half));
        if constexpr (DROP) keep[half] = dropout_keep8(pk, key0, qi, bh, md.offset, md.thr);
      }
    }
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      s = mfma32<BF16>(*reinterpret_cast<const s16x8*>(Ks + 32 * b * T::PITCH + ra[t]), qreg[t], s);
      dp = mfma32<BF16>(*reinterpret_cast<const s16x8*>(Vs + 32 * b * T::PITCH + ra[t]), oreg[t], dp);
    }
    // Register r holds key kb0 + 16 (r / 8) + 8 h + r % 8 of query qi.
    const bool masked = MASKED && (kb0 + 32 > Lk || (CAUSAL && kb0 + 31 > wq0 + off));
    s16x8 sa[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float xe = __builtin_fmaf(s[r], c, mt[r] - l2);  // select before the exponential, as in dK/dV
      float p = __builtin_amdgcn_exp2f(mt[r] == -INFINITY ? -INFINITY : xe);
      if (masked) {
        const int kj = kb0 + 16 * (r >> 3) + 8 * h + (r & 7);
        if (kj >= Lk || (CAUSAL && kj > qi + off)) p = 0.f;
      }
      float dpk = dp[r];
      if constexpr (DROP) dpk = ((keep[r >> 3] >> (r & 7)) & 1u) ? dpk * md.rp : 0.f;
      sa[r >> 3][r & 7] = (short)round16<BF16>(p * (dpk + dd));  // dd holds -Dv
    }
    // dQ += dS K over the block's 32 keys (2 k-steps).
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int rowoff = (32 * b + 16 * s2) * T::PITCH;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 lo = lds_read_tr(Ks + rowoff + ta[db][0]);
        const s16x4 hi = lds_read_tr(Ks + rowoff + ta[db][1]);
        dq[db] = mfma32<BF16>(sa[s2], s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, dq[db]);
      }
    }
  };

  // -Dv of the lane's query in every register of an accumulator block: the
  // plain tiles' dP products start from it.
  f32x16 neg_dd;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_dd[r] = dd;  // dd holds -Dv
  // A whole tile without mask, dropout or masked keys (the plain
  // backward's common case), software-pipelined over its two blocks: the
  // S and dP products of block 1 are issued before the softmax work of
  // block 0, so that the wave's MFMAs and VALU overlap even when the other
  // wave of the SIMD is in the same phase.
  auto tile_plain = [&](const char* stage) __attribute__((always_inline)) {
    const char* Ks = stage;
    const char* Vs = stage + T::BYTES;
    f32x16 s[2], dp[2];
    // The S and dP products at raised priority: the SIMD's other wave
    // (another workgroup) issues its VALU work in their shadow instead of
    // contending for the matrix unit (+0.5% on the whole backward).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
      dp[b] = neg_dd;  // the products accumulate onto -Dv: dP - Dv in one go
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        s[b] = mfma32<BF16>(*reinterpret_cast<const s16x8*>(Ks + 32 * b * T::PITCH + ra[t]), qreg[t], s[b]);
        dp[b] = mfma32<BF16>(*reinterpret_cast<const s16x8*>(Vs + 32 * b * T::PITCH + ra[t]), oreg[t], dp[b]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s16x8 sa[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -l2));
        sa[r >> 3][r & 7] = (short)round16<BF16>(p * dp[b][r]);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int rowoff = (32 * b + 16 * s2) * T::PITCH;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const s16x4 lo = lds_read_tr(Ks + rowoff + ta[db][0]);
          const s16x4 hi = lds_read_tr(Ks + rowoff + ta[db][1]);
          dq[db] = mfma32<BF16>(sa[s2], s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, dq[db]);
        }
      }
    }
  };

  land_all();
  __syncthreads();
  // Tiles alternate between the two stages; each loop body covers a pair so
  // that every LDS address is a lane offset plus an immediate.  Tiles
  // [0, j_plain) hold no key past Lk or past the diagonal of any query of
  // the wave: they run without the masking code in a loop of their own (one
  // code path per loop), an even number of them so that the second loop
  // starts in the first stage.  Every wave passes one barrier per tile
  // whichever loop it is in.
  int j_plain = Lk / BQ;
  if (CAUSAL) j_plain = min(j_plain, max(0, wq0 + off + 1) / BQ);
  j_plain = __builtin_amdgcn_readfirstlane(min(j_plain, nkt) & ~1);
  auto run_tile = [&](const char* stage, int kv0, auto tag) __attribute__((always_inline)) {
    if constexpr (!EX && !decltype(tag)::value) {
      tile_plain(stage);
    } else {
      block(stage, kv0, 0, tag);
      block(stage, kv0, 1, tag);
    }
  };
  auto pair = [&](int j, auto tag) __attribute__((always_inline)) -> bool {  // false: no tile after j
    if (j + 1 < nkt) issue(j + 1, smem + STAGE);
    run_tile(smem, j * BQ, tag);
    land_all();
    __syncthreads();
    if (j + 1 >= nkt) return false;
    if (j + 2 < nkt) issue(j + 2, smem);
    run_tile(smem + STAGE, (j + 1) * BQ, tag);
    land_all();
    __syncthreads();
    return true;
  };
  int j = 0;
  for (; j < j_plain; j += 2) pair(j, std::integral_constant<bool, false>{});
  for (; j < nkt; j += 2)
    if (!pair(j, std::integral_constant<bool, true>{})) break;

  // Register r of block db holds query wq0 + 8 (r / 4) + 4 h + r % 4,
  // column 32 db + n.
  unsigned short* dQg = static_cast<unsigned short*>(a.dq) + (size_t)bh * Lq * D;
  const float scale = a.scale;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = wq0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (qr < Lq) {
#pragma unroll
      for (int db = 0; db < DB; ++db) dQg[(size_t)qr * D + 32 * db + n] = round16<BF16>(dq[db][r] * scale);
    }
  }
}

template <int DT, int D, bool CAUSAL, int KIND, bool DROP>
hipError_t launch_typed(const BwdArgs& a, const MaskDropout& md, hipStream_t s) {
  const int nqt = (a.Lq + BQ - 1) / BQ;
  bwd_stats_kernel<DT, D><<<dim3(a.BH * nqt), dim3(NT), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.Lk + BW - 1) / BW;
  const int nqb = (a.Lq + BW - 1) / BW;
  bwd_dkdv_kernel<DT == 2, D, CAUSAL, KIND, DROP><<<dim3(a.BH * nkb), dim3(NT), 0, s>>>(a, md);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dq_kernel<DT == 2, D, CAUSAL, KIND, DROP><<<dim3(a.BH * nqb), dim3(NT), 0, s>>>(a, md);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int BH, int Lq) {
  return (size_t)BH * ((Lq + BQ - 1) / BQ) * kStatFloats * sizeof(float);
}

template <int DT, int KIND, bool DROP>
hipError_t launch_kd(int D, bool causal, const BwdArgs& a, const MaskDropout& md, hipStream_t s) {
  if (D == 128)
    return causal ? launch_typed<DT, 128, true, KIND, DROP>(a, md, s)
                  : launch_typed<DT, 128, false, KIND, DROP>(a, md, s);
  return causal ? launch_typed<DT, 64, true, KIND, DROP>(a, md, s) : launch_typed<DT, 64, false, KIND, DROP>(a, md, s);
}

template <int DT>
hipError_t launch_dt(int D, bool causal, const BwdArgs& a, const MaskDropout* md, hipStream_t s) {
  if (md == nullptr || (md->kind == 0 && !md->dropout)) return launch_kd<DT, 0, false>(D, causal, a, MaskDropout{}, s);
  if (md->kind == 1)
    return md->dropout ? launch_kd<DT, 1, true>(D, causal, a, *md, s) : launch_kd<DT, 1, false>(D, causal, a, *md, s);
  if (md->kind == 2)
    return md->dropout ? launch_kd<DT, 2, true>(D, causal, a, *md, s) : launch_kd<DT, 2, false>(D, causal, a, *md, s);
  return launch_kd<DT, 0, true>(D, causal, a, *md, s);
}

hipError_t launch_bwd(int dtype, int D, bool causal, const BwdArgs& a, hipStream_t s, const MaskDropout* md) {
  return dtype == 2 ? launch_dt<2>(D, causal, a, md, s) : launch_dt<1>(D, causal, a, md, s);
}

}  // namespace attn
