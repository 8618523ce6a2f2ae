// Attention forward with a general mask and dropout fused into the tile, for
// fp16 / bf16 on gfx950 MFMA.
//
// The comfyai.app chapter "6.3 FlashAttention" (section 6.3.3, "Kernel
// Fusion") lists the steps of one tile as scores, scale, mask, softmax,
// dropout and the value product, all on chip.  Here a key of a row is
// excluded when a boolean mask is zero, an additive mask is -inf, it lies
// past Lk, or (causal) past the bottom-right diagonal; an additive mask is
// added to the scaled scores.  The softmax statistics are the online ones of
// the quidproquo.cc guide ("Mechanism: run with the wrong answer, then
// correct it": reference d, denominator s, output corrected by
// exp(d_old - d_new)) over the un-dropped weights, so LSE does not depend on
// dropout; the weights that enter the value product are the kept ones, and
// O is scaled by 1 / (1 - p) at the end.  As in the plain prefill, d is a
// lazy bound: it moves (above the tile maximum, by a headroom) only when a
// weight sum of the wave passes 2^8, so the common tile computes no maximum
// and folds -d into the mask term, one fma per score before the exp.  A row
// with no key left gets O = 0 and LSE = -inf.
//
// Work decomposition: one workgroup = 4 waves x 32 queries; lane (n, h) of a
// wave owns query n.  64-key tiles of K and V go HBM -> LDS by DMA (double
// buffered, XOR-swizzled rows).  S^T = K Q^T puts 16 keys of the lane's
// query in its registers, which are then directly the B operand (P^T) of
// O^T += V^T P^T, V^T being read from LDS with ds_read_b64_tr_b16.  The mask
// rows are read from device memory 8 keys at a time; the keep bits of 8 keys
// come from one Philox4x32-10 block (a 16-bit half of a word per key).
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "attn_internal.hpp"
#include "mask_dropout.hpp"
#include "mfma_tile.hpp"
#include "swz_tile.hpp"

namespace attn {
namespace {

using namespace mt;
using namespace st;

constexpr int NT = 256;
constexpr int BW = 128;  // queries per workgroup

// KIND: mask kind (0 none, 1 boolean, 2 additive); DROP: dropout on.  Each
// variant carries only its own per-element work.
template <bool BF16, int D, bool CAUSAL, int KIND, bool DROP>
__global__ __launch_bounds__(NT, 2) void prefill_ex_kernel(PrefillArgs a, MaskDropout md, float c) {
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
  // Workgroups are dealt to the 8 XCDs round robin.  Each XCD takes the
  // query blocks of a contiguous range of heads (same K / V in its L2);
  // causal: the last query blocks (the most keys) go first.  Within the
  // range, consecutive workgroups take consecutive query blocks of one head,
  // except for a mask shared by the heads (mask_h == 1) with whole heads per
  // XCD: then they take one query block of each head of the range in turn,
  // so that the heads that run together read the same mask rows (one L2
  // fill of those rows serves them all).
  const int total = a.BH * nqb;
  const int wg = blockIdx.x;
  int bh, qpos;
  if (KIND != 0 && md.mask_h == 1 && a.BH % 8 == 0) {
    const int hx = a.BH / 8, r = wg / 8;  // heads per XCD, position in the XCD's range
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

  // Q of the lane's query as the B operand: Q[qi][16 t + 8 h .. + 8].
  const int qi = wq0 + n;
  const unsigned short* Qg = static_cast<const unsigned short*>(a.q) + (size_t)bh * Lq * D;
  s16x8 qreg[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < Lq) x = *reinterpret_cast<const u32x4*>(Qg + (size_t)qi * D + 16 * t + 8 * h);
    qreg[t] = __builtin_bit_cast(s16x8, x);
  }
  // Wait for the Q loads here, before the tile loop: otherwise the compiler
  // (which does not count the DMA issued by inline assembly) puts a full
  // vmcnt(0) wait at their first use inside the loop, draining the next
  // tile's DMA just issued.
#pragma unroll
  for (int t = 0; t < KS; ++t) asm volatile("" ::"v"(qreg[t]));
  const size_t mrow = KIND != 0 && qi < Lq ? mask_slab(md, bh, Lq, Lk) + (size_t)qi * Lk : 0;
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

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  // Reference d of the row (base-2 units of the scaled, masked scores; the
  // same in both halves) and this half's share of the denominator s,
  // relative to d.  The reference moves only when a weight sum of the
  // wave passes 2^8 (or a row has none yet), as in the plain kernel.
  float m_ref = -INFINITY;
  float l_run = 0.f;
  // bf16: sum of the rounding errors w - bf16(w) of each lane's largest kept
  // weight per tile.  The value product takes the rounded weights and s the
  // unrounded ones; with the reference above the maximum the largest weight
  // is no longer exactly 1, so its rounding would reach O unmatched.
  float e_run = 0.f;

  // Boolean masks: the raw bytes of a whole, aligned tile are loaded one
  // tile ahead, before that tile's K/V DMA is issued.  The compiler does not
  // count the DMA (inline assembly), so waiting for mask loads issued after
  // it would also wait for the DMA; loaded before it and consumed after the
  // landing wait, they cost no wait inside the tile.
  constexpr bool PREF = KIND == 1 && !DROP;  // with dropout: no registers to spare
  auto raw_load = [&](int kv0, uint2 (&raw)[4]) __attribute__((always_inline)) {
    if (Lk % 8 == 0 && kv0 + BQ <= Lk) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        raw[grp] = *reinterpret_cast<const uint2*>(static_cast<const unsigned char*>(md.mask) + mrow + kv0 +
                                                   32 * (grp >> 1) + 16 * (grp & 1) + 8 * h);
    }
  };
  auto raw_landed = [&](const uint2 (&raw)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) asm volatile("" ::"v"(raw[grp].x), "v"(raw[grp].y));
  };

  // Masks not loaded a tile ahead (additive: 128 bytes per lane and tile;
  // boolean with dropout: no registers to spare): the tile loads its own
  // terms and the next tile's K/V DMA is issued only after those terms have
  // been added to the scores.  Any wait for the mask loads is a full vmcnt
  // wait (the compiler does not count the DMA, which is inline assembly), so
  // with the DMA issued first it would also wait for the DMA.
  constexpr bool LATE_DMA = KIND != 0 && !PREF;

  // Additive masks without dropout: the 128 bytes of a lane's terms for the
  // next tile are loaded once this tile's weights are done (its own terms
  // are dead by then), after the next tile's K/V DMA.  The landing wait at
  // the end of the tile then waits for the DMA but leaves those 8 loads in
  // flight (vmcnt(8)); they are consumed after the next tile's score
  // products, so their latency spans the value products, the barrier and
  // the score products.
  constexpr bool PREF_ADD = KIND == 2 && !DROP;
  constexpr int kAmLoads = 8;  // global_load_dwordx4 per lane and tile
  float4 am[kAmLoads];
  const float* m32 = static_cast<const float*>(md.mask);
  // Whole tiles of aligned rows take the loads (the in-tile path reads the rest).
  auto am_vec = [&](int kv0) __attribute__((always_inline)) { return Lk % 8 == 0 && kv0 + BQ <= Lk; };
  auto am_load = [&](int kv0) __attribute__((always_inline)) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const size_t i0 = mrow + kv0 + 32 * (grp >> 1) + 16 * (grp & 1) + 8 * h;
      am[2 * grp] = *reinterpret_cast<const float4*>(m32 + i0);
      am[2 * grp + 1] = *reinterpret_cast<const float4*>(m32 + i0 + 4);
    }
  };
  // End-of-tile landing: every DMA issued so far has landed; with `keep`,
  // the last kAmLoads vector loads (issued after it) may still be in flight.
  auto land = [&](bool keep) __attribute__((always_inline)) {
    if (keep)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAmLoads) : "memory");
    else
      land_all();
  };

  // Returns whether the next tile's mask terms were loaded (PREF_ADD).
  auto tile = [&](const char* stage, int kv0, const uint2 (&raw)[4], auto&& issue_next)
                  __attribute__((always_inline)) -> bool {
    if (kv0 >= w_key_end) {
      if constexpr (LATE_DMA) issue_next();
      return false;
    }
    const char* Ks = stage;
    const char* Vs = stage + T::BYTES;
    // Mask terms of the tile's 32 keys, loaded before the score products so
    // that the loads overlap them.
    const bool whole = kv0 + BQ <= Lk;        // no key of the tile at or past Lk
    const bool vec = Lk % 8 == 0 && whole;     // whole, aligned mask rows for the tile
    // Every term carries -d, so one fma per score gives exp2's argument
    // (no reference yet: 0, and the weights are recomputed below).
    const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
    float t8[4][8];
    if constexpr (KIND != 0) {
      if (PREF_ADD && vec) {
        // Terms loaded a tile ahead: read after the score products below.
      } else if (PREF && vec) {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            t8[grp][e] = (((e < 4 ? raw[grp].x : raw[grp].y) >> (8 * (e & 3))) & 0xffu) ? nm : -INFINITY;
      } else {
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int key0 = kv0 + 32 * (grp >> 1) + 16 * (grp & 1) + 8 * h;
          mask_terms8_kind<KIND>(md, mrow + key0, key0, Lk, vec, t8[grp], nm);
        }
      }
    }
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x16{};
#pragma unroll
      for (int t = 0; t < KS; ++t)
        s[b] = mfma32<BF16>(*reinterpret_cast<const s16x8*>(Ks + 32 * b * T::PITCH + ra[t]), qreg[t], s[b]);
    }
    if constexpr (PREF_ADD) {
      if (vec) {
        // After the score products (fence), so that the wait for these loads
        // comes as late as possible.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float4 x = am[2 * grp + (e >> 2)];
            const float m = (e & 3) == 0 ? x.x : (e & 3) == 1 ? x.y : (e & 3) == 2 ? x.z : x.w;
            t8[grp][e] = __builtin_fmaf(m, kLog2e, nm);
          }
      }
    }
    // Register r of block b holds key kv0 + 32 b + 16 (r / 8) + 8 h + r % 8.
    unsigned keep[4] = {0xffu, 0xffu, 0xffu, 0xffu};
    if constexpr (DROP) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        keep[grp] = dropout_keep8(pk, kv0 + 32 * (grp >> 1) + 16 * (grp & 1) + 8 * h, qi, bh, md.offset, md.thr);
    }
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int b = grp >> 1, r = 8 * (grp & 1) + e;
        if constexpr (KIND != 0)
          s[b][r] = __builtin_fmaf(s[b][r], c, t8[grp][e]);
        else
          s[b][r] = __builtin_fmaf(s[b][r], c, nm);
      }
    if constexpr (LATE_DMA) issue_next();
    // Keys past Lk (without a mask: only in the last tile) and, in tiles
    // that cross the wave's first diagonal, keys past the query's diagonal.
    if (KIND == 0 && !whole) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kv0 + 32 * (grp >> 1) + 16 * (grp & 1) + 8 * h + e >= Lk) s[grp >> 1][8 * (grp & 1) + e] = -INFINITY;
    }
    if (CAUSAL && kv0 + BQ - 1 > wq0 + off) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kv0 + 32 * (grp >> 1) + 16 * (grp & 1) + 8 * h + e > qi + off) s[grp >> 1][8 * (grp & 1) + e] = -INFINITY;
    }
    // Weights exp2(a - d) of the un-dropped scores (their sum is s), the
    // kept ones rounded to the MFMA type for the value product, and (bf16)
    // the rounding error of the lane's largest kept weight.
    float psum = 0.f, e_t = 0.f;
    s16x8 pb[4];
    auto weights = [&]() __attribute__((always_inline)) {
      psum = 0.f;
      float wmax = 0.f;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int b = grp >> 1, half = grp & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[b][8 * half + e]);
          psum = grp || e ? psum + p : p;  // the first weight starts the sum
          const float w = !DROP || ((keep[grp] >> e) & 1u) ? p : 0.f;
          if constexpr (BF16) wmax = fmaxf(wmax, w);
          pb[grp][e] = (short)round16<BF16>(w);
        }
      }
      if constexpr (BF16) e_t = wmax - __builtin_bit_cast(float, (unsigned)round16<true>(wmax) << 16);
    };
    weights();
    bool loaded = false;
    if constexpr (PREF_ADD) {
      if (kv0 + BQ < w_key_end && am_vec(kv0 + BQ)) {
        am_load(kv0 + BQ);
        loaded = true;
      }
    }
    // Every weight of a lane is at most its sum: with no sum above 2^8 (and
    // every row with a reference) the weights are bounded and d stays.
    // Otherwise the guide's running maximum d_k = max(d_{k-1}, tile max),
    // with headroom: a row whose tile maximum passed d moves d kHeadroom
    // above it, O~ and s take the correction exp(d_old - d_new), and the
    // weights are redone from the scores (still in s, shifted by -d).
    if (__builtin_expect(__any(!(psum <= 256.f) || m_ref == -INFINITY), 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
      mx = halves_max(mx == -INFINITY ? -INFINITY : mx - nm);
      const bool grow = mx > m_ref;
      const float m_new = grow ? mx + (BF16 ? 24.f : 0.f) : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      m_ref = m_new;
      l_run *= alpha;
      if constexpr (BF16) e_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      // Shift the scores from -d_old to -d_new (a row without a reference
      // yet keeps 0); rows that did not move add exactly 0.
      const float delta = (m_ref == -INFINITY ? 0.f : -m_ref) - nm;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] += delta;
      weights();
    }
    l_run += psum;
    if constexpr (BF16) e_run += e_t;
    // O^T += V^T P^T over the tile's four 16-key k-steps.
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* src = Vs + 16 * stp * T::PITCH;
        const s16x4 lo = lds_read_tr(src + ta[db][0]);
        const s16x4 hi = lds_read_tr(src + ta[db][1]);
        oacc[db] = mfma32<BF16>(s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, pb[stp], oacc[db]);
      }
    }
    return loaded;
  };

  uint2 rawA[4] = {}, rawB[4] = {};
  if constexpr (PREF) raw_load(0, rawA);
  if constexpr (PREF_ADD) {
    if (0 < w_key_end && am_vec(0)) am_load(0);
  }
  land_all();
  if constexpr (PREF) raw_landed(rawA);
  __syncthreads();
  for (int j = 0; j < nkt; j += 2) {
    if constexpr (PREF) {
      if (j + 1 < nkt) raw_load((j + 1) * BQ, rawB);
    }
    auto next_a = [&]() __attribute__((always_inline)) {
      if (j + 1 < nkt) issue(j + 1, smem + STAGE);
    };
    if constexpr (!LATE_DMA) next_a();
    land(tile(smem, j * BQ, rawA, next_a));
    if constexpr (PREF) raw_landed(rawB);
    __syncthreads();
    if (j + 1 >= nkt) break;
    if constexpr (PREF) {
      if (j + 2 < nkt) raw_load((j + 2) * BQ, rawA);
    }
    auto next_b = [&]() __attribute__((always_inline)) {
      if (j + 2 < nkt) issue(j + 2, smem);
    };
    if constexpr (!LATE_DMA) next_b();
    land(tile(smem + STAGE, (j + 1) * BQ, rawB, next_b));
    if constexpr (PREF) raw_landed(rawA);
    __syncthreads();
  }

  // Register r of block db holds column 32 db + 8 (r / 4) + 4 h + r % 4 of
  // the lane's query.
  // O divides by s less the rounding errors of the largest weights (bf16);
  // LSE takes s itself.
  const float l_tot = halves_sum(l_run);
  const float l_o = BF16 ? l_tot - halves_sum(e_run) : l_tot;
  const float inv = l_tot > 0.f ? (DROP ? md.rp : 1.f) / l_o : 0.f;
  if (qi < Lq) {
    unsigned short* Og = static_cast<unsigned short*>(a.o) + ((size_t)bh * Lq + qi) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const unsigned lo = (unsigned)round16<BF16>(oacc[db][4 * jj] * inv) |
                            ((unsigned)round16<BF16>(oacc[db][4 * jj + 1] * inv) << 16);
        const unsigned hi = (unsigned)round16<BF16>(oacc[db][4 * jj + 2] * inv) |
                            ((unsigned)round16<BF16>(oacc[db][4 * jj + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(Og + 32 * db + 8 * jj + 4 * h) = make_uint2(lo, hi);
      }
    if (h == 0) a.lse[(size_t)bh * Lq + qi] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <bool BF16, int D, bool CAUSAL, int KIND, bool DROP>
hipError_t launch_kd(const PrefillArgs& a, const MaskDropout& md, hipStream_t s) {
  const int nqb = (a.Lq + BW - 1) / BW;
  const float c = a.neg ? -a.c : a.c;
  prefill_ex_kernel<BF16, D, CAUSAL, KIND, DROP><<<dim3(a.BH * nqb), dim3(NT), 0, s>>>(a, md, c);
  return hipGetLastError();
}

// Neither mask nor dropout takes the dropout variant with p = 0 (threshold
// 0 keeps every weight, 1 / (1 - p) = 1): correct, only slower; the entry
// point sends that case to the plain kernel.
template <bool BF16, int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, const MaskDropout& md, hipStream_t s) {
  if (md.kind == 1)
    return md.dropout ? launch_kd<BF16, D, CAUSAL, 1, true>(a, md, s) : launch_kd<BF16, D, CAUSAL, 1, false>(a, md, s);
  if (md.kind == 2)
    return md.dropout ? launch_kd<BF16, D, CAUSAL, 2, true>(a, md, s) : launch_kd<BF16, D, CAUSAL, 2, false>(a, md, s);
  return launch_kd<BF16, D, CAUSAL, 0, true>(a, md, s);
}

template <bool BF16>
hipError_t dispatch_d(int D, bool causal, const PrefillArgs& a, const MaskDropout& md, hipStream_t s) {
  if (D == 64) return causal ? launch<BF16, 64, true>(a, md, s) : launch<BF16, 64, false>(a, md, s);
  return causal ? launch<BF16, 128, true>(a, md, s) : launch<BF16, 128, false>(a, md, s);
}

}  // namespace

hipError_t launch_prefill_ex(int dtype, int D, bool causal, const PrefillArgs& a, const MaskDropout& md,
                             hipStream_t s) {
  return dtype == 2 ? dispatch_d<true>(D, causal, a, md, s) : dispatch_d<false>(D, causal, a, md, s);
}

}  // namespace attn
