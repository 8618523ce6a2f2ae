// Tiled one-pass attention forward (prefill) for fp16 / bf16 on gfx950 MFMA.
//
// Method: the online softmax of the quidproquo.cc guide "Faster Generation,
// Part 1: Flash Attention" (section "Mechanism: run with the wrong answer,
// then correct it", both "Expand" boxes): for each key tile the running row
// maximum d, running denominator s and output accumulator are corrected by
// exp(d_old - d_new) before the tile's contribution is added.  The output is
// kept un-normalised (O~ = s * O) and divided by s once at the end, which is
// the same quantity as the guide's per-chunk normalised O_k.  The tile fusion
// (scores, scale, mask, softmax and the value product inside one kernel, no
// score matrix in device memory) is the comfyai.app chapter "6.3
// FlashAttention", section 6.3.3 ("Kernel Fusion", "Full Forward Process").
// The loop order is query-tile outer, key-tile inner, so d, s and O stay in
// registers for the whole pass (the guide's single-query walk), instead of
// the chapter's key-outer order that writes O, l, m back after every tile.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows):
//   * each wave owns 32 query rows; Q is loaded once into VGPRs as the B
//     operand of v_mfma_f32_32x32x16_{bf16,f16};
//   * key/value tiles of 64 rows are staged HBM -> VGPR -> LDS with 16-byte
//     coalesced loads, double buffered (the next tile's global loads are in
//     flight while the current tile is computed);
//   * S^T = K_j Q^T is computed so that each lane holds 32 scores of ONE
//     query: row statistics need no cross-lane reduction except one
//     permlane32 swap per tile;
//   * K rows are read in a bit-permuted order (bits 2 and 3 of the row index
//     swapped) so that the score registers of a lane are already the B
//     operand (P^T, 8 consecutive keys) of the P V product;
//   * V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16
//     to form the A operand (V^T) of O^T += V^T P^T.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "attn_internal.hpp"

namespace attn {
namespace {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;  // query rows per workgroup
constexpr int BN = 64;   // key rows per tile
constexpr int NT = 256;  // threads per workgroup

template <int D>
struct Tile {
  // LDS row pitches.  K: +16 B so that 16 lanes reading 16 B each from 16
  // consecutive rows hit 16 disjoint 4-bank groups.  V: +64 B so that the
  // four rows of one transposed read land in four disjoint 16-bank groups.
  static constexpr int KPITCH = D * 2 + 16;
  static constexpr int VPITCH = D * 2 + 64;
  static constexpr int KBYTES = BN * KPITCH;
  static constexpr int STAGE = KBYTES + BN * VPITCH;
  static constexpr int CHUNKS = BN * D / 8 / NT;  // 16-byte chunks per thread per tensor
  static constexpr int KSTEPS = D / 16;           // MFMA k-steps of Q K^T
  static constexpr int DBLK = D / 32;             // 32-wide blocks of the output
};

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round to the 16-bit MFMA type, nearest even.
template <bool BF16>
__device__ __forceinline__ unsigned short round16(float x) {
  if constexpr (BF16)
    return __builtin_bit_cast(unsigned short, (__bf16)x);
  else
    return __builtin_bit_cast(unsigned short, (_Float16)x);
}

// Max and sum of a value held by lanes l and l^32 (the two halves of a wave
// that share one query row).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void prefill_mfma_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ O, float* __restrict__ LSE,
    int BH, int Lq, int Lk, int nqt, float c, unsigned qsign) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;  // query column of the S^T / O^T tiles owned by this lane
  const int h = lane >> 5;  // which 8-wide k slice this lane feeds to the MFMA

  // Workgroup -> (batch*head, query tile).  Workgroups are dealt to the 8
  // XCDs round robin; remap so that consecutive logical tiles (the query
  // tiles of one head, which stream the same K/V) share an XCD and its L2.
  // Causal: heavier (later) query tiles of a head are dispatched first.
  const int total = BH * nqt;
  const int wg = blockIdx.x;
  const int logical = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
  const int bh = logical / nqt;
  const int qt = CAUSAL ? nqt - 1 - logical % nqt : logical % nqt;
  const int q0 = qt * BM;
  const int off = Lk - Lq;  // bottom-right causal alignment

  const unsigned short* Qh = Q + (size_t)bh * Lq * D;
  const unsigned short* Kh = K + (size_t)bh * Lk * D;
  const unsigned short* Vh = V + (size_t)bh * Lk * D;

  const int q_last = min(q0 + BM, Lq) - 1;
  const int kv_end = CAUSAL ? min(Lk, q_last + off + 1) : Lk;
  const int nkv = (kv_end + BN - 1) / BN;
  const int wq0 = q0 + 32 * w;  // first query of this wave
  const bool wave_live = wq0 < Lq;
  const int w_key_end = CAUSAL ? min(Lk, min(wq0 + 31, Lq - 1) + off + 1) : Lk;

  // Q^T fragment (B operand): lane (n, h) holds Q[qi][16t + 8h .. +8].
  const int qi = wq0 + n;
  s16x8 qreg[T::KSTEPS];
#pragma unroll
  for (int t = 0; t < T::KSTEPS; ++t) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < Lq) x = *reinterpret_cast<const u32x4*>(Qh + (size_t)qi * D + 16 * t + 8 * h);
    x ^= qsign;
    qreg[t] = __builtin_bit_cast(s16x8, x);
  }

  // Staging registers for the next K/V tile.
  u32x4 kst[T::CHUNKS], vst[T::CHUNKS];
  auto gload = [&](int kv0) {
#pragma unroll
    for (int u = 0; u < T::CHUNKS; ++u) {
      const int ci = tid + NT * u;
      const int row = ci / (D / 8), col = ci % (D / 8);
      const int key = kv0 + row;
      u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (key < Lk) {
        kx = *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + col * 8);
        vx = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + col * 8);
      }
      kst[u] = kx;
      vst[u] = vx;
    }
  };
  auto sstore = [&](int stage) {
    char* base = smem + stage * T::STAGE;
#pragma unroll
    for (int u = 0; u < T::CHUNKS; ++u) {
      const int ci = tid + NT * u;
      const int row = ci / (D / 8), col = ci % (D / 8);
      *reinterpret_cast<u32x4*>(base + row * T::KPITCH + col * 16) = kst[u];
      *reinterpret_cast<u32x4*>(base + T::KBYTES + row * T::VPITCH + col * 16) = vst[u];
    }
  };

  f32x16 oacc[T::DBLK];
#pragma unroll
  for (int i = 0; i < T::DBLK; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max, base-2 scaled-score units
  float l_run = 0.f;        // this lane's part of the running denominator

  // Tile row read by this lane for S^T: bits 2 and 3 of n swapped, so the
  // accumulator register r of block blk holds key 32 blk + 16 (r/8) + 8 h + r%8.
  const int prow = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int g = lane >> 4, li = lane & 15;

  if (nkv > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const int kv0 = j * BN;
    if (j + 1 < nkv) gload(kv0 + BN);

    if (wave_live && kv0 < w_key_end) {
      const char* Ks = smem + (j & 1) * T::STAGE;
      const char* Vs = Ks + T::KBYTES;

      // ---- scores S^T = K_j Q^T (two 32-key blocks) ----
      f32x16 sacc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        sacc[blk] = f32x16{};
        const char* kp = Ks + (32 * blk + prow) * T::KPITCH + 16 * h;
#pragma unroll
        for (int t = 0; t < T::KSTEPS; ++t)
          sacc[blk] = mfma32<BF16>(*reinterpret_cast<const s16x8*>(kp + 32 * t), qreg[t], sacc[blk]);
      }

      // ---- mask: keys past Lk, and keys after the diagonal (causal) ----
      const bool need_mask = (kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
      unsigned live = 0xffffffffu;
      if (need_mask) {
        live = 0u;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * blk + 16 * (r >> 3) + 8 * h + (r & 7);
            const bool ok = key < Lk && (!CAUSAL || key <= qi + off);
            live |= (ok ? 1u : 0u) << (16 * blk + r);
            if (!ok) sacc[blk][r] = -INFINITY;
          }
      }

      // ---- running max (guide: d_k = max(d_{k-1}, max of chunk k)) ----
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
      mx = halves_max(mx);
      const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
      const float m_new = fmaxf(m_run, m_tile);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      // Correction of the old state: exp(d_{k-1} - d_k) (0 on the first tile).
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      // ---- P = exp(a - d_k): fp32 into the denominator, rounded for the MFMA ----
      s16x8 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int blk = s >> 1, r = 8 * (s & 1) + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][r], c, -m_use));
          if (need_mask && !((live >> (16 * blk + r)) & 1u)) p = 0.f;
          pb[s][e] = (short)round16<BF16>(p);
          psum += p;  // the denominator keeps fp32 weights (exact LSE)
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < T::DBLK; ++i) oacc[i] *= alpha;

      // ---- O^T += V_j^T P^T ----
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int db = 0; db < T::DBLK; ++db) {
          const char* vp = Vs + (16 * s + 8 * h + (li >> 2)) * T::VPITCH +
                           (32 * db + 16 * (g & 1) + 4 * (li & 3)) * 2;
          const s16x4 lo = lds_read_tr(vp);
          const s16x4 hi = lds_read_tr(vp + 4 * T::VPITCH);
          const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = mfma32<BF16>(a, pb[s], oacc[db]);
        }
      }
    }

    if (j + 1 < nkv) sstore((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O~ / s, lse = ln 2 (d + log2 s) ----
  const float l_tot = halves_sum(l_run);
  if (wave_live && qi < Lq) {
    const float inv = 1.f / l_tot;
    unsigned short* Oq = O + (size_t)bh * Lq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * db + 8 * jj + 4 * h;
        const unsigned lo = (unsigned)round16<BF16>(oacc[db][4 * jj + 0] * inv) |
                            ((unsigned)round16<BF16>(oacc[db][4 * jj + 1] * inv) << 16);
        const unsigned hi = (unsigned)round16<BF16>(oacc[db][4 * jj + 2] * inv) |
                            ((unsigned)round16<BF16>(oacc[db][4 * jj + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(Oq + d) = make_uint2(lo, hi);
      }
    if (h == 0) LSE[(size_t)bh * Lq + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  const int nqt = (a.Lq + BM - 1) / BM;
  const unsigned qsign = a.neg ? 0x80008000u : 0u;
  hipLaunchKernelGGL((prefill_mfma_kernel<BF16, D, CAUSAL>), dim3(a.BH * nqt), dim3(NT), 0, s,
                     static_cast<const unsigned short*>(a.q), static_cast<const unsigned short*>(a.k),
                     static_cast<const unsigned short*>(a.v), static_cast<unsigned short*>(a.o), a.lse,
                     a.BH, a.Lq, a.Lk, nqt, a.c, qsign);
  return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch_d(int D, bool causal, const PrefillArgs& a, hipStream_t s) {
  if (D == 64) return causal ? launch<BF16, 64, true>(a, s) : launch<BF16, 64, false>(a, s);
  return causal ? launch<BF16, 128, true>(a, s) : launch<BF16, 128, false>(a, s);
}

}  // namespace

hipError_t launch_prefill_mfma(int dtype, int D, bool causal, const PrefillArgs& a, hipStream_t s) {
  return dtype == 2 ? dispatch_d<true>(D, causal, a, s) : dispatch_d<false>(D, causal, a, s);
}

}  // namespace attn
