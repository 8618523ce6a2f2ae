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
constexpr int NW = NT / 64;  // waves per workgroup
// Largest lag (base 2) of the reference maximum behind the true running
// maximum: weights exp(a - d) stay below 2^8.
constexpr float kTau = 8.f;

template <int D>
struct Tile {
  // LDS rows are padded so that every read address is a lane base plus an
  // immediate offset, and both read patterns are bank-conflict-free:
  //  K: pitch = D*2 + 16 B (an odd number of 16-byte slots): 16 lanes
  //     reading one 16-byte chunk of 16 consecutive rows hit 16 different
  //     4-bank groups (ds_read_b128).
  //  V: pitch = D*2 + 64 B (4 mod 16 slots): the 4 rows x 64 B of one
  //     half-wave transposed read (ds_read_b64_tr_b16) hit disjoint banks.
  static constexpr int CPR = D / 8;                 // 16-byte data chunks per row
  static constexpr int KSPR = CPR + 1;              // K slots per row (1 pad slot)
  static constexpr int VSPR = CPR + 4;              // V slots per row (4 pad slots)
  static constexpr int KPITCH = KSPR * 16;
  static constexpr int VPITCH = VSPR * 16;
  static constexpr int KBYTES = BN * KPITCH;
  static constexpr int STAGE = KBYTES + BN * VPITCH;
  static constexpr int KINST = BN * KSPR / 64;      // 64-lane DMA instructions per K tile
  static constexpr int VINST = BN * VSPR / 64;      // ... per V tile
  static constexpr int KSTEPS = D / 16;             // MFMA k-steps of Q K^T
  static constexpr int DBLK = D / 32;               // 32-wide blocks of the output
  static constexpr int KI = (KINST + NW - 1) / NW;  // K DMA instructions per wave
  static constexpr int VI = (VINST + NW - 1) / NW;  // V DMA instructions per wave
  static_assert(BN * KSPR % 64 == 0 && BN * VSPR % 64 == 0, "whole DMA instructions");
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

__device__ __forceinline__ __attribute__((address_space(3))) void* to_lds(char* p) {
  return (__attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}


// K/V tiles go HBM -> LDS by DMA (global_load_lds_dwordx4): one instruction
// moves 64 lanes x 16 B into 1 KB of consecutive LDS, here a run of 16-byte
// slots of the padded tile.  Lane l of DMA instruction i fills slot 64 i + l
// (row = slot / slots-per-row, chunk = the rest); pad slots fetch chunk 0 of
// their row again (in bounds, never read).  Wave w issues instructions w,
// w + 4, ...
//
// Byte offset, within one tile of the source tensor, of the chunk that lane
// `lane` fetches for DMA instruction `inst` of a tile with `spr` slots per
// row.
template <int D>
__device__ __forceinline__ unsigned dma_src_offset(int inst, int lane, int spr) {
  const int slot = inst * 64 + lane;
  const int row = slot / spr;
  const int chunk = slot - row * spr;
  return (unsigned)row * (D * 2) + (unsigned)(chunk < D / 8 ? chunk : 0) * 16;
}

// Rows at or past `rows_left` (keys past Lk) are redirected to row
// rows_left - 1 of the tile, which is in bounds.
template <int D>
__device__ __forceinline__ unsigned dma_clamp(unsigned off, int rows_left) {
  const int row = (int)(off / (D * 2));
  return row < rows_left ? off : (unsigned)(rows_left - 1) * (D * 2) + off % (D * 2);
}

// Issue this wave's DMA instructions for one tile of one tensor.
template <int D, int INST, int PER_WAVE>
__device__ __forceinline__ void dma_tile(const char* src_tile, char* dst_tile, const unsigned* src_off,
                                         int w, bool full, int rows_left) {
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int inst = i * NW + w;
    if (inst < INST) {
      const unsigned o = full ? src_off[i] : dma_clamp<D>(src_off[i], rows_left);
      __builtin_amdgcn_global_load_lds(src_tile + o, to_lds(dst_tile + inst * 1024), 16, 0, 0);
    }
  }
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
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

  // K/V tiles go HBM -> LDS by DMA (see dma_tile).  Rows past Lk read row
  // Lk-1 (in bounds) and their V slots are zeroed once the DMA has landed.
  const char* Kb = reinterpret_cast<const char*>(Kh);
  const char* Vb = reinterpret_cast<const char*>(Vh);
  unsigned k_src[T::KI];
  unsigned v_src[T::VI];
#pragma unroll
  for (int i = 0; i < T::KI; ++i) k_src[i] = dma_src_offset<D>(i * NW + w, lane, T::KSPR);
#pragma unroll
  for (int i = 0; i < T::VI; ++i) v_src[i] = dma_src_offset<D>(i * NW + w, lane, T::VSPR);
  auto dma = [&](char* stage, int kv0) {
    const bool full = kv0 + BN <= Lk;
    const size_t base = (size_t)kv0 * (D * 2);  // uniform tile offset
    dma_tile<D, T::KINST, T::KI>(Kb + base, stage, k_src, w, full, Lk - kv0);
    dma_tile<D, T::VINST, T::VI>(Vb + base, stage + T::KBYTES, v_src, w, full, Lk - kv0);
  };
  // Wait for this thread's DMA, then zero the V slots of rows past Lk.
  auto land = [&](char* stage, int kv0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kv0 + BN > Lk) {
#pragma unroll
      for (int i = 0; i < T::VI; ++i) {
        const int inst = i * NW + w;
        const int slot = inst * 64 + lane;
        if (inst < T::VINST && kv0 + slot / T::VSPR >= Lk)
          *reinterpret_cast<u32x4*>(stage + T::KBYTES + slot * 16) = u32x4{0u, 0u, 0u, 0u};
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

    // ---- scores S^T = K_j Q^T (two 32-key blocks) ----
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const char* kp = Ks + (32 * blk + prow) * T::KPITCH + 16 * h;
      sacc[blk] = f32x16{};
#pragma unroll
      for (int t = 0; t < T::KSTEPS; ++t)
        sacc[blk] = mfma32<BF16>(*reinterpret_cast<const s16x8*>(kp + 32 * t), qreg[t], sacc[blk]);
    }

    // Phase fences: keep the scheduler from stretching live ranges across
    // the score, softmax and value phases (the register file is full).
    __builtin_amdgcn_sched_barrier(0);

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
    __builtin_amdgcn_sched_barrier(0);

    // ---- O^T += V_j^T P^T; V^T fragments via transposed LDS reads ----
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st) __builtin_amdgcn_sched_barrier(0);
      s16x8 vf[T::DBLK];
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db) {
        const char* vp = Vs + (16 * st + 8 * h + (li >> 2)) * T::VPITCH +
                         (32 * db + 16 * (g & 1) + 4 * (li & 3)) * 2;
        const s16x4 lo = lds_read_tr(vp);
        const s16x4 hi = lds_read_tr(vp + 4 * T::VPITCH);
        vf[db] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int db = 0; db < T::DBLK; ++db) oacc[db] = mfma32<BF16>(vf[db], pb[st], oacc[db]);
    }
  };

  // Tiles [0, j_mask) of this wave hold no masked key; tiles from j_mask on
  // (the causal diagonal band of the wave's rows, the Lk tail) do.  Two
  // loops instead of a per-tile choice keep the accumulators in one set of
  // registers.  Every wave runs nkv steps, so barriers stay matched.
  int j_mask = nkv;
  if (CAUSAL) {
    // first tile whose last key lies past the diagonal of the wave's first row
    const int first_bad = wq0 + off - BN + 2;
    j_mask = first_bad <= 0 ? 0 : (first_bad + BN - 1) / BN;
  }
  if (Lk % BN) j_mask = min(j_mask, Lk / BN);
  j_mask = __builtin_amdgcn_readfirstlane(min(j_mask, nkv));

  dma(stage0, 0);
  land(stage0, 0);
  __syncthreads();
  // One pipeline step per tile j: start the DMA of tile j+1 into the other
  // stage, compute tile j, wait for the DMA, then one workgroup barrier.
  int j = 0;
  for (; j < j_mask; ++j) {
    char* cur = (j & 1) ? stage1 : stage0;
    char* nxt = (j & 1) ? stage0 : stage1;
    const int kv0 = j * BN;
    if (j + 1 < nkv) dma(nxt, kv0 + BN);
    if (wave_live) tile(cur, cur + T::KBYTES, kv0, std::integral_constant<bool, false>{});
    if (j + 1 < nkv) land(nxt, kv0 + BN);
    __syncthreads();
  }
  for (; j < nkv; ++j) {
    char* cur = (j & 1) ? stage1 : stage0;
    char* nxt = (j & 1) ? stage0 : stage1;
    const int kv0 = j * BN;
    if (j + 1 < nkv) dma(nxt, kv0 + BN);
    if (wave_live && kv0 < w_key_end) tile(cur, cur + T::KBYTES, kv0, std::integral_constant<bool, true>{});
    if (j + 1 < nkv) land(nxt, kv0 + BN);
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
