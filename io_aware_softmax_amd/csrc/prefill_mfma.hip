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
#include <type_traits>

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
// Largest lag (base 2) of the reference maximum behind the true running
// maximum: weights exp(a - d) stay below 2^8.
constexpr float kTau = 8.f;

template <int D>
struct Tile {
  // K and V tiles are stored row-major without padding; the 16-byte chunk c
  // of row r sits at chunk position c ^ swz(r).  The swizzle makes both LDS
  // read patterns conflict-free: 16 lanes reading the same chunk of 16
  // consecutive rows (K, ds_read_b128), and the 4 rows x 4 chunks of one
  // half-wave transposed read (V, ds_read_b64_tr_b16).
  static constexpr int ROWB = D * 2;              // bytes per row
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int TBYTES = BN * ROWB;        // one tensor tile
  static constexpr int STAGE = 2 * TBYTES;        // K tile then V tile
  static constexpr int CHUNKS = TBYTES / 16 / NT; // 16-byte chunks per thread per tensor
  static constexpr int KSTEPS = D / 16;           // MFMA k-steps of Q K^T
  static constexpr int DBLK = D / 32;             // 32-wide blocks of the output
  __device__ static constexpr int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // Byte offset of element column `col` (a multiple of 4) of row r.
  __device__ static constexpr int off(int r, int col) {
    return r * ROWB + ((((col >> 3) ^ swz(r))) << 4) + ((col & 7) << 1);
  }
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
  // Two pipeline stages in separate arrays so that the compiler can tell the
  // stage being filled by DMA from the stage being read.
  __shared__ __attribute__((aligned(16))) char stage0[T::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[T::STAGE];

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

  // K/V tiles go HBM -> LDS by DMA (global_load_lds_dwordx4): one
  // instruction moves 64 lanes x 16 B into 1 KB of consecutive LDS; lane l
  // fetches the global chunk that the swizzle places in slot l.  Rows past
  // Lk read row Lk-1 (in bounds) and their V slots are zeroed afterwards.
  // Per-lane source offsets (bytes within a tile) are computed once.
  unsigned src_off[T::CHUNKS];
  int src_row[T::CHUNKS];
#pragma unroll
  for (int u = 0; u < T::CHUNKS; ++u) {
    const int slot = (u * (NT / 64) + w) * 64 + lane;
    src_row[u] = slot / T::CPR;
    src_off[u] = src_row[u] * T::ROWB + (((slot % T::CPR) ^ T::swz(src_row[u])) << 4);
  }
  const char* Kb = reinterpret_cast<const char*>(Kh);
  const char* Vb = reinterpret_cast<const char*>(Vh);
  auto dma = [&](char* stage, int kv0) {
    const bool full = kv0 + BN <= Lk;
    const unsigned tile_off = (unsigned)kv0 * T::ROWB;
#pragma unroll
    for (int u = 0; u < T::CHUNKS; ++u) {
      unsigned o = tile_off + src_off[u];
      if (!full && kv0 + src_row[u] >= Lk)  // clamp to row Lk-1, same chunk
        o = (unsigned)(Lk - 1) * T::ROWB + (src_off[u] % T::ROWB);
      char* dst = stage + (u * (NT / 64) + w) * 1024;
      __builtin_amdgcn_global_load_lds(Kb + o, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Vb + o, (__attribute__((address_space(3))) void*)(dst + T::TBYTES),
                                       16, 0, 0);
    }
  };
  // Wait for this thread's DMA, then zero the V slots of rows past Lk.
  auto land = [&](char* stage, int kv0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kv0 + BN > Lk) {
#pragma unroll
      for (int u = 0; u < T::CHUNKS; ++u) {
        if (kv0 + src_row[u] >= Lk)
          *reinterpret_cast<u32x4*>(stage + T::TBYTES + ((u * (NT / 64) + w) * 64 + lane) * 16) =
              u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x16 oacc[T::DBLK];
#pragma unroll
  for (int i = 0; i < T::DBLK; ++i) oacc[i] = f32x16{};
  // Reference maximum d of the row (base-2 scaled-score units) and this
  // lane's part of the denominator s, both relative to that reference.
  float m_ref = -INFINITY;
  float l_run = 0.f;

  // Tile row read by this lane for S^T: bits 2 and 3 of n swapped, so the
  // accumulator register r of block blk holds key 32 blk + 16 (r/8) + 8 h + r%8.
  const int prow = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int g = lane >> 4, li = lane & 15;

  // One key tile.  MASK selects the variant for tiles that hold masked keys
  // (the causal diagonal band and the Lk tail); all other tiles run without
  // any per-score masking work.
  auto tile = [&](const char* Ks, const char* Vs, int kv0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;

    // ---- scores S^T = K_j Q^T (two 32-key blocks); fragments read ahead ----
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int krow = 32 * blk + prow;
      s16x8 kf[T::KSTEPS];
#pragma unroll
      for (int t = 0; t < T::KSTEPS; ++t)
        kf[t] = *reinterpret_cast<const s16x8*>(Ks + T::off(krow, 16 * t + 8 * h));
      sacc[blk] = f32x16{};
#pragma unroll
      for (int t = 0; t < T::KSTEPS; ++t) sacc[blk] = mfma32<BF16>(kf[t], qreg[t], sacc[blk]);
    }

    // ---- mask: keys past Lk, and keys after the diagonal (causal) ----
    unsigned live = 0xffffffffu;
    if constexpr (MASK) {
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

    // ---- running maximum (guide: d_k = max(d_{k-1}, max of chunk k)) ----
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
    mx = halves_max(mx);
    const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
    // The reference d moves to the new maximum only when the tile's maximum
    // exceeds it by more than kTau (base 2); then O~ and s are corrected by
    // exp(d_old - d_new) as in the guide.  Otherwise d stays, the weights
    // exp(a - d) are at most 2^kTau, and O~ / s is unchanged in real
    // arithmetic (the correction holds for any reference).  The check is per
    // row; the branch is taken by the whole wave if any row needs it.
    const bool grow = m_tile > m_ref + kTau;
    if (__any(grow)) {
      const float m_new = grow ? m_tile : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < T::DBLK; ++i) oacc[i] *= alpha;
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;

    // ---- P = exp(a - d): fp32 into the denominator, rounded for the MFMA ----
    s16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int blk = st >> 1, r = 8 * (st & 1) + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][r], c, -m_use));
        if constexpr (MASK) p = ((live >> (16 * blk + r)) & 1u) ? p : 0.f;
        pb[st][e] = (short)round16<BF16>(p);
        psum += p;  // the denominator keeps fp32 weights (exact LSE)
      }
    }
    l_run += psum;

    // ---- O^T += V_j^T P^T; V^T fragments via transposed LDS reads ----
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      s16x8 vf[T::DBLK];
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db) {
        const int vrow = 16 * st + 8 * h + (li >> 2);
        const int vcol = 32 * db + 16 * (g & 1) + 4 * (li & 3);
        const s16x4 lo = lds_read_tr(Vs + T::off(vrow, vcol));
        const s16x4 hi = lds_read_tr(Vs + T::off(vrow + 4, vcol));
        vf[db] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db) oacc[db] = mfma32<BF16>(vf[db], pb[st], oacc[db]);
    }
  };

  // One pipeline step: start the DMA of tile j+1 into `nxt`, compute tile j
  // from `cur`, wait for the DMA, then one barrier for the workgroup.
  auto step = [&](int j, char* cur, char* nxt) {
    const int kv0 = j * BN;
    const bool more = j + 1 < nkv;
    if (more) dma(nxt, kv0 + BN);
    if (wave_live && kv0 < w_key_end) {
      const bool need_mask = (kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
      if (need_mask)
        tile(cur, cur + T::TBYTES, kv0, std::integral_constant<bool, true>{});
      else
        tile(cur, cur + T::TBYTES, kv0, std::integral_constant<bool, false>{});
    }
    if (more) land(nxt, kv0 + BN);
    __syncthreads();
  };

  dma(stage0, 0);
  land(stage0, 0);
  __syncthreads();
  for (int j = 0; j < nkv; j += 2) {
    step(j, stage0, stage1);
    if (j + 1 < nkv) step(j + 1, stage1, stage0);
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
    if (h == 0) LSE[(size_t)bh * Lq + qi] = (m_ref + log2f(l_tot)) * kLn2;
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
