// Tiled one-pass attention forward (prefill) for fp16 / bf16 at D = 128 on
// gfx950: two wave groups in opposite phases ("ping-pong").
//
// Method: the online softmax of the quidproquo.cc guide "Faster Generation,
// Part 1: Flash Attention" (section "Mechanism: run with the wrong answer,
// then correct it", both "Expand" boxes): for each key tile the running row
// maximum d, running denominator s and output accumulator are corrected by
// exp(d_old - d_new) before the tile's contribution is added.  The output is
// kept un-normalised (O~ = s * O) and divided by s once at the end.  Scores,
// scale, mask, softmax and the value product are fused per tile with no
// score matrix in device memory (comfyai.app chapter "6.3 FlashAttention",
// section 6.3.3, "Kernel Fusion" and "Full Forward Process").
//
// Work decomposition.  A workgroup of 8 waves owns 256 query rows (32 per
// wave) of one (batch, head) and streams the key/value tiles of 64 rows once
// for all of them.  Waves w and w + 4 share a SIMD.  Waves 0-3 (group 0) and
// 4-7 (group 1) run the same per-tile work half a step apart:
//   matrix phase   S_{j+1} = K_{j+1} Q^T and O~ += V_j^T P_j^T (32 MFMAs at
//                  D = 128, operands read from LDS a few MFMAs ahead);
//   softmax phase  P_{j+1} = exp(a - d) against the row's reference d,
//                  rounded to the MFMA type, s += sum; the reference moves
//                  (and O~, s are corrected) only when a weight sum says so.
// While one wave of a SIMD is in its matrix phase the other is in its
// softmax phase, so the MFMA pipe runs one wave's products while the vector
// ALU runs the other wave's exponentials.  A workgroup barrier separates the
// half steps; the matrix-phase wave runs at the higher issue priority and
// leaves its last two value products for after the barrier, where they
// cover the other wave's wait for its first LDS operands.
// Group 0 issues the K/V tile DMA (HBM -> LDS, no VGPR round trip) for the
// next step during its matrix phase and waits for it at the end of its
// softmax phase, so each DMA has most of a step to land.  K/V tiles are
// double buffered: step j reads K_{j+1} and V_j while K_{j+2} and V_{j+1}
// land.  A persistent workgroup starts its next item inside the current
// item's last step (which needs neither scores nor Q): the next Q, K_0,
// K_1 and V_0 load while the last value products run.
//
// Register layout (per wave, as in the single-group kernel): Q^T is the B
// operand of v_mfma_f32_32x32x16; K rows are read with bits 2 and 3 of the
// row index swapped so that each lane's score registers are already the B
// operand (P^T, 8 consecutive keys) of the value product; V is read
// transposed from row-major LDS with ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_internal.hpp"
#include "mfma_tile.hpp"

namespace attn {
namespace {

using namespace mt;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup
constexpr int kRun = 2;             // DMA instructions per M0 run
constexpr int kDmaWaves = 4;        // the 4 waves of group 0 issue the DMA
// Largest weight exp(a - d) of the common path: 2^8 (the reference maximum
// may lag the true running maximum by up to 8, base 2).
constexpr float kTauWeight = 256.f;
// Headroom (base 2) of a new reference above the tile maximum that set it.
// bf16 weights keep the fp32 exponent range, so a reference 24 above the
// maximum (weights down to 2^-24 at first) costs no precision and makes
// later maxima rarely pass it; fp16 weights would leave the fp16 range, so
// there the reference is the maximum itself.
template <bool BF16>
constexpr float kHeadroom = BF16 ? 24.f : 0.f;

// V tile in LDS.  D = 128: unpadded rows of 256 B whose four 64-byte
// granules are XOR-swizzled by the row's low two bits (granule g of row r at
// g ^ (r mod 4)); the four rows x 64 B of one half-wave transposed read then
// fall in four different granules, i.e. disjoint banks, and the tile is 16
// whole DMA instructions.  D = 64 keeps the padded rows of Tile.
template <int D>
struct VTile {
  static constexpr bool SWZ = D == 128;
  static constexpr int SPR = SWZ ? D / 8 : Tile<D>::VSPR;  // 16-byte slots per row
  static constexpr int PITCH = SPR * 16;
  static constexpr int BYTES = BN * PITCH;
  static constexpr int INST = BN * SPR / 64;
  // Source offset, within the tile in device memory, of the 16 bytes that
  // lane `lane` of DMA instruction `inst` writes to LDS slot 64 inst + lane.
  __device__ static unsigned src_offset(int inst, int lane) {
    if constexpr (SWZ) {
      const int row = 4 * inst + (lane >> 4);  // 4 rows per instruction
      const int pchunk = lane & 15;            // physical 16-byte chunk in the row
      const int lchunk = 4 * ((pchunk >> 2) ^ (row & 3)) + (pchunk & 3);
      return (unsigned)row * (D * 2) + (unsigned)lchunk * 16;
    } else {
      return dma_src_offset<D>(inst, lane, SPR);
    }
  }
  // LDS byte offset (within a V tile) of this lane's transposed read of
  // 32-column block db for key row `row` (row mod 4 = the lane's rows').
  __device__ static int read_offset(int row, int db, int colbyte) {
    if constexpr (SWZ)
      return row * PITCH + ((db ^ (row & 3)) * 64) + colbyte;
    else
      return row * PITCH + 64 * db + colbyte;
  }
};

template <int D>
struct Layout {
  using T = Tile<D>;
  using VT = VTile<D>;
  static constexpr int K0 = 0;
  static constexpr int K1 = T::KBYTES;
  static constexpr int V0 = 2 * T::KBYTES;
  static constexpr int V1 = 2 * T::KBYTES + VT::BYTES;
  static constexpr int KV = 2 * (T::KBYTES + VT::BYTES);
  static constexpr int OPITCH = D * 2 + 16;  // staging pitch of O rows
  static constexpr int OST = KV;             // O staging, apart from the tiles so that the
                                             // next item's tiles can land meanwhile
  static constexpr int TOTAL = KV + kWaves * 32 * OPITCH;
  static_assert(TOTAL <= 160 * 1024, "one workgroup per CU");
};

// Workgroup barrier that does not wait for outstanding vector-memory loads
// (the DMA in flight), only for this wave's LDS and scalar traffic.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

#ifndef PP_DEFER
#define PP_DEFER 2
#endif
// Value products a matrix phase leaves for after the barrier that ends it.
// Their operands are already in registers, so they keep the MFMA pipe busy
// while the other wave of the SIMD, now in its matrix phase, waits for its
// first LDS operands.
constexpr int kDefer = PP_DEFER;

// Matrix phase of one wave: S = K_{j+1} Q^T (DO_S) and O~ += V_j^T P_j^T
// (DO_PV), one MFMA per slot, each operand read PF slots ahead.  hook(i)
// runs at the start of slot i (the DMA issue of the next tiles rides here:
// the wave waits for the MFMA pipe anyway, so a stalled DMA issue costs
// little).  With DO_PV, mid() (the barrier that ends the phase) runs before
// the last kDefer products.
template <bool BF16, int D, bool DO_S, bool DO_PV, class Hook, class Mid>
__device__ __forceinline__ void matrix_phase(const char* kbase, const char* vbase, const int (&vl)[D / 32],
                                             const s16x8 (&qreg)[D / 16],
                                             f32x16 (&s)[2], const s16x8 (&pb)[4], f32x16 (&oacc)[D / 32],
                                             Hook&& hook, Mid&& mid) {
  using T = Tile<D>;
  constexpr int NS = DO_S ? 2 * T::KSTEPS : 0;
  constexpr int NP = DO_PV ? 4 * T::DBLK : 0;
  constexpr int N = NS + NP;
  static_assert(!DO_PV || kDefer < NP, "deferred products are value products");
  constexpr int PF = 6;
  s16x8 fr[N];
  auto read = [&](int r) __attribute__((always_inline)) {
    if (r < NS) {
      fr[r] = *reinterpret_cast<const s16x8*>(kbase + 32 * (r & 1) * T::KPITCH + 32 * (r >> 1));
    } else {
      const int x = r - NS, st = x / T::DBLK, db = x % T::DBLK;
      const char* p = vbase + vl[db] + 16 * st * VTile<D>::PITCH;
      const s16x4 lo = lds_read_tr(p);
      const s16x4 hi = lds_read_tr(p + 4 * VTile<D>::PITCH);
      fr[r] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
#pragma unroll
  for (int r = 0; r < (PF < N ? PF : N); ++r) read(r);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (DO_PV && i == N - kDefer) {
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
    hook(i);
    if (i + PF < N) read(i + PF);
    if (i < NS) {
      s[i & 1] = mfma32<BF16>(fr[i], qreg[i >> 1], i < 2 ? f32x16{} : s[i & 1]);
    } else {
      const int x = i - NS;
      oacc[x % T::DBLK] = mfma32<BF16>(fr[i], pb[x / T::DBLK], oacc[x % T::DBLK]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// SPLIT: the keys of every (batch*head, query tile) are cut into the
// contiguous ranges `plan` lists, each an item of its own; an item writes its
// rows' normalised partial output and log-sum-exp (part_o, part_l) instead of
// O and LSE, and prefill_split_combine merges them.  The unsplit kernel never
// reads the last three arguments.
template <bool BF16, int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void prefill_pp_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ O, float* __restrict__ LSE, int BH,
    int Lq, int Lk, int nqt, float c, unsigned qsign, int slots_per_xcd, int items_per_xcd,
    float* __restrict__ part_o, float* __restrict__ part_l, const PrefillSplitPlan plan) {
  using T = Tile<D>;
  using LY = Layout<D>;
  using KP = DmaPlan<T::KINST, kRun, kDmaWaves>;
  using VP = DmaPlan<LY::VT::INST, kRun, kDmaWaves>;
  __shared__ __attribute__((aligned(16))) char smem[LY::TOTAL];
  auto kb = [&](int i) __attribute__((always_inline)) -> char* { return smem + ((i & 1) ? LY::K1 : LY::K0); };
  auto vb = [&](int i) __attribute__((always_inline)) -> char* { return smem + ((i & 1) ? LY::V1 : LY::V0); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave 0..7, in an SGPR
  const int grp = w >> 2;                                   // 0 leads, 1 lags and issues the DMA
  const int wd = w & 3;                                     // DMA slot of a group-1 wave
  const int n = lane & 31;  // query column of the S^T / O^T tiles owned by this lane
  const int h = lane >> 5;  // which 8-wide k slice this lane feeds to the MFMA

  // Workgroup -> work items (batch*head, query tile of 256 rows).
  // Workgroups are dealt to the 8 XCDs round robin.  The items are split
  // into 8 contiguous ranges (the query tiles of a few heads, which stream
  // the same K/V) and XCD x works on range x, so those tiles share its L2.
  // Within a range the order is head-major, causal tiles of a head
  // heaviest first.  slots_per_xcd == 0: one item per workgroup, item =
  // workgroup index.  Otherwise the S = slots_per_xcd workgroups of an XCD
  // walk its range in rounds of S items in snake order (slot s takes
  // position s of even rounds and S-1-s of odd ones, pairing heavy causal
  // tiles with light ones); a workgroup with several items runs them one
  // after the other and loads the next item's first tiles and Q while it
  // writes the current output.
  const int total = BH * (SPLIT ? plan.items : nqt);
  const int wg = blockIdx.x;
  const int xcd = wg % 8, slot = wg / 8;
  const int range_lo = xcd * items_per_xcd;
  const int range_n = max(0, min(items_per_xcd, total - range_lo));
  auto item_at = [&](int round) __attribute__((always_inline)) -> int {  // -1: none
    if (slots_per_xcd == 0) return round == 0 ? wg : -1;
    const int pos = round * slots_per_xcd + ((round & 1) ? slots_per_xcd - 1 - slot : slot);
    return pos < range_n ? range_lo + pos : -1;
  };
  const int off = Lk - Lq;  // bottom-right causal alignment

  // Per-item values (wave-uniform ones in SGPRs).
  int bh = 0, nkv = 0, wq0 = 0, w_nkv = 0, j_mask = 0, qi = 0;
  int jl_s = 0, sp_s = 0;  // SPLIT: first key tile of the item's range, range index
  const char* Kb = nullptr;
  const char* Vb = nullptr;
  s16x8 qreg[T::KSTEPS];
  auto setup = [&](int logical) __attribute__((always_inline)) {
    int qt, n_ranges = 1;
    if constexpr (SPLIT) {
      bh = logical / plan.items;
      const unsigned e = plan.item[logical % plan.items];
      qt = (int)(e >> 5);
      sp_s = (int)(e & 31u);
      n_ranges = plan.ranges[qt];
    } else {
      bh = logical / nqt;
      qt = CAUSAL ? nqt - 1 - logical % nqt : logical % nqt;
    }
    const int q0 = qt * kRows;
    Kb = reinterpret_cast<const char*>(K + (size_t)bh * Lk * D);
    Vb = reinterpret_cast<const char*>(V + (size_t)bh * Lk * D);
    const int q_last = min(q0 + kRows, Lq) - 1;
    const int kv_end = CAUSAL ? min(Lk, q_last + off + 1) : Lk;
    nkv = __builtin_amdgcn_readfirstlane((kv_end + BN - 1) / BN);  // tiles the workgroup streams
    wq0 = q0 + 32 * w;                                             // first query of this wave
    const int w_key_end = CAUSAL ? min(Lk, min(wq0 + 31, Lq - 1) + off + 1) : Lk;
    // Tiles [0, w_nkv) are computed by this wave; tiles [0, j_mask) hold no
    // masked key for it (the causal diagonal band and the Lk tail do).
    w_nkv = __builtin_amdgcn_readfirstlane(wq0 < Lq ? (w_key_end + BN - 1) / BN : 0);
    int jm = w_nkv;
    if (CAUSAL) {
      const int first_bad = wq0 + off - BN + 2;  // first kv0 whose last key passes the diagonal
      jm = min(jm, first_bad <= 0 ? 0 : (first_bad + BN - 1) / BN);
    }
    if (Lk % BN) jm = min(jm, Lk / BN);
    j_mask = __builtin_amdgcn_readfirstlane(jm);
    if constexpr (SPLIT) {
      // Key tiles [jl, jh) of the query tile's [0, nkv), balanced so that no
      // range is empty (the plan keeps a tile's range count <= its nkv); the
      // counts below become local to that range.
      const int jl = sp_s * nkv / n_ranges;
      const int jh = (sp_s + 1) * nkv / n_ranges;
      jl_s = __builtin_amdgcn_readfirstlane(jl);
      nkv = __builtin_amdgcn_readfirstlane(jh - jl);
      w_nkv = __builtin_amdgcn_readfirstlane(max(0, min(w_nkv - jl, nkv)));
      j_mask = __builtin_amdgcn_readfirstlane(max(0, min(j_mask - jl, nkv)));
    }
    qi = wq0 + n;
  };
  // Q^T fragment (B operand): lane (n, h) holds Q[qi][16t + 8h .. +8].  The
  // loads are left in flight: nothing reads qreg before the item's first
  // barrier (sign_q below, or the first product).  A row past Lq loads row
  // Lq - 1 instead (finite scores; such rows are never stored).
  auto load_q = [&]() __attribute__((always_inline)) {
    const unsigned short* Qr = Q + ((size_t)bh * Lq + min(qi, Lq - 1)) * D + 8 * h;
#pragma unroll
    for (int t = 0; t < T::KSTEPS; ++t)
      qreg[t] = __builtin_bit_cast(s16x8, *reinterpret_cast<const u32x4*>(Qr + 16 * t));
  };
  // A negative scale runs as scale |c| on -Q (flipped sign bits), so that
  // masked scores (-inf) keep weight 0.
  auto sign_q = [&]() __attribute__((always_inline)) {
    if (qsign != 0u) {
#pragma unroll
      for (int t = 0; t < T::KSTEPS; ++t)
        qreg[t] = __builtin_bit_cast(s16x8, __builtin_bit_cast(u32x4, qreg[t]) ^ qsign);
    }
  };

  // DMA of one K or V tile by group 0 (DmaPlan over its 4 waves); rows past
  // Lk read row Lk-1 and the V slots of those rows are zeroed once landed.
  unsigned k_src[KP::N];
  unsigned v_src[VP::N];
#pragma unroll
  for (int i = 0; i < KP::N; ++i)
    k_src[i] = dma_src_offset<D>(KP::inst(i, wd), lane, T::KSPR) + kDmaBias - KP::pos_in_run(i) * 1024u;
#pragma unroll
  for (int i = 0; i < VP::N; ++i)
    v_src[i] = LY::VT::src_offset(VP::inst(i, wd), lane) + kDmaBias - VP::pos_in_run(i) * 1024u;
  auto biased = [](const char* p) __attribute__((always_inline)) {
    return reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(p) - kDmaBias);
  };
  // kv0 arguments are local to the item's key range (SPLIT adds its start).
  auto dma_k = [&](char* buf, int kv0) __attribute__((always_inline)) {
    if constexpr (SPLIT) kv0 += jl_s * BN;
    const char* g = biased(Kb + (size_t)kv0 * (D * 2));
    if (kv0 + BN <= Lk)
      dma_tile_whole<KP>(g, buf, k_src, wd);
    else
      dma_tile_ragged<D, KP>(g, buf, k_src, wd, Lk - kv0);
  };
  auto dma_v = [&](char* buf, int kv0) __attribute__((always_inline)) {
    if constexpr (SPLIT) kv0 += jl_s * BN;
    const char* g = biased(Vb + (size_t)kv0 * (D * 2));
    if (kv0 + BN <= Lk)
      dma_tile_whole<VP>(g, buf, v_src, wd);
    else
      dma_tile_ragged<D, VP>(g, buf, v_src, wd, Lk - kv0);
  };
  // Wait for this wave's DMA; zero the V slots of rows past Lk it filled.
  auto land = [&](char* vbuf, int kv0) __attribute__((always_inline)) {
    if constexpr (SPLIT) kv0 += jl_s * BN;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (vbuf != nullptr && kv0 + BN > Lk) {
#pragma unroll
      for (int i = 0; i < VP::N; ++i) {
        if (i < VP::U || wd < VP::X) {
          const int slot = VP::inst(i, wd) * 64 + lane;
          if (kv0 + slot / LY::VT::SPR >= Lk) *reinterpret_cast<u32x4*>(vbuf + slot * 16) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  f32x16 oacc[T::DBLK];
  // Reference maximum d of the row (base-2 scaled-score units) and this
  // lane's part of the denominator s, both relative to that reference.
  float m_ref = -INFINITY;
  float l_run = 0.f;
  // bf16: sum over tiles of the rounding error (fp32 weight minus its bf16
  // value) of this lane's largest weight of the tile.  The value product
  // takes the rounded weights, so O is divided by l_run - e_run: the row's
  // dominant weight then enters numerator and denominator with the same
  // rounding and O stays a convex combination of the value rows (with the
  // unrounded sum alone, a dominant weight off by up to 2^-8 relative moves
  // O by that much of |v|).  LSE keeps the unrounded sum.
  float e_run = 0.f;
  f32x16 sc[2];  // scores of the tile between the matrix and softmax phases
  s16x8 pb[4];   // weights of the tile between the softmax and matrix phases
#pragma unroll
  for (int i = 0; i < 2; ++i) sc[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = s16x8{};

  // Tile row read by this lane for S^T: bits 2 and 3 of n swapped, so the
  // accumulator register r of block blk holds key 32 blk + 16 (r/8) + 8 h + r%8.
  const int prow = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int g = lane >> 4, li = lane & 15;
  const int k_lane = prow * T::KPITCH + 16 * h;
  // Transposed V reads: lane rows 8h + li/4 (+ 16 per k-step, + 4 for the
  // upper half), bytes 32 (g & 1) + 8 (li & 3) of each 64-byte column block.
  int v_lane[T::DBLK];
#pragma unroll
  for (int db = 0; db < T::DBLK; ++db)
    v_lane[db] = LY::VT::read_offset(8 * h + (li >> 2), db, (16 * (g & 1) + 4 * (li & 3)) * 2);

  // DMA of K_{j+2} and V_{j+1} by a group-0 wave, spread over the slots
  // of its matrix phase (runs of kRun instructions; the extra instruction
  // of an uneven split goes first).  Only for whole tiles; the other cases
  // are issued in one go before the phase.
  constexpr int NR = KP::RUNS + VP::RUNS;  // DMA runs per step (K first)
  constexpr int NSLOT = 2 * T::KSTEPS + 4 * T::DBLK;  // MFMA slots of a matrix phase
  static_assert(NR <= NSLOT - 4, "every DMA run needs a slot of its own");
  auto dma_hook = [&](const char* kg, char* kdst, const char* vg, char* vdst) __attribute__((always_inline)) {
    return [=, &k_src, &v_src](int i) __attribute__((always_inline)) {
      if (i == 0) {
        if constexpr (KP::X != 0) {
          if (wd < KP::X) dma_run<1>(kg, k_src + KP::U, lds_addr(kdst + KP::inst(KP::U, wd) * 1024));
        }
        if constexpr (VP::X != 0) {
          if (wd < VP::X) dma_run<1>(vg, v_src + VP::U, lds_addr(vdst + VP::inst(VP::U, wd) * 1024));
        }
      }
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        if (i == 2 + q * (NSLOT - 4) / NR) {
          if (q < KP::RUNS) {
            const int i0 = KP::run_first(q);
            dma_run_n(KP::run_len(q), kg, k_src + i0, lds_addr(kdst + KP::inst(i0, wd) * 1024));
          } else {
            const int i0 = VP::run_first(q - KP::RUNS);
            dma_run_n(VP::run_len(q - KP::RUNS), vg, v_src + i0, lds_addr(vdst + VP::inst(i0, wd) * 1024));
          }
        }
      }
    };
  };
  auto no_hook = [](int) __attribute__((always_inline)) {};
  auto no_mid = []() __attribute__((always_inline)) {};
  // The barrier that ends a matrix phase; the deferred products after it
  // run at the softmax phase's issue priority.
  auto end_phase = [&]() __attribute__((always_inline)) {
    barrier_lds();
    __builtin_amdgcn_s_setprio(0);
  };

  // Matrix phase of step j: S_{j+1} and O~ += V_j P_j.  Every wave runs
  // both products on every step so that the loop has one code path: a wave
  // past its last tile computes scores it never uses (K buffers always hold
  // finite key rows) and multiplies V_j (loaded, finite) by zero weights.
  // Group 0 (issue = true) also issues the DMA of the tiles of step j+1.
  // issue_tag: 0 none (group 1), 1 spread over the slots (K_{j+2} and
  // V_{j+1} whole), 2 in one go before the phase (ragged or absent tiles).
  // mid: the barrier that ends the phase (run before its last kDefer
  // products; the caller runs none after the call).
  auto matrix = [&](int j, auto issue_tag) __attribute__((always_inline)) {
    constexpr int ISSUE = decltype(issue_tag)::value;
    if constexpr (ISSUE == 1) {
      const int jg = SPLIT ? j + jl_s : j;  // tile index in the head
      matrix_phase<BF16, D, true, true>(kb(j + 1) + k_lane, vb(j), v_lane, qreg, sc, pb, oacc,
                                        dma_hook(biased(Kb + (size_t)(jg + 2) * BN * (D * 2)), kb(j + 2),
                                                 biased(Vb + (size_t)(jg + 1) * BN * (D * 2)), vb(j + 1)),
                                        end_phase);
    } else {
      if constexpr (ISSUE == 2) {
        if (j + 2 < nkv) dma_k(kb(j + 2), (j + 2) * BN);
        if (j + 1 < nkv) dma_v(vb(j + 1), (j + 1) * BN);
      }
      matrix_phase<BF16, D, true, true>(kb(j + 1) + k_lane, vb(j), v_lane, qreg, sc, pb, oacc, no_hook,
                                        end_phase);
    }
  };
  // The last steps of an item (DMA issued in one go): a wave past its last
  // tile (causal: the early rows of an item end a few tiles before its last)
  // runs no products.
  auto matrix_tail = [&](int j, auto issue_tag) __attribute__((always_inline)) {
    if constexpr (decltype(issue_tag)::value == 2) {
      if (j + 2 < nkv) dma_k(kb(j + 2), (j + 2) * BN);
      if (j + 1 < nkv) dma_v(vb(j + 1), (j + 1) * BN);
    }
    if (j < w_nkv)
      matrix_phase<BF16, D, true, true>(kb(j + 1) + k_lane, vb(j), v_lane, qreg, sc, pb, oacc, no_hook,
                                        end_phase);
    else
      end_phase();
  };
  // The item's last step (j = nkv - 1) needs no scores: value products only
  // (none for a wave past its last tile); mid as for matrix_phase.
  auto matrix_last = [&](int j, auto&& mid) __attribute__((always_inline)) {
    if (j < w_nkv)
      matrix_phase<BF16, D, false, true>(kb(j + 1) + k_lane, vb(j), v_lane, qreg, sc, pb, oacc, no_hook, mid);
    else
      mid();
  };
  auto prio_low = []() __attribute__((always_inline)) { __builtin_amdgcn_s_setprio(0); };
  auto matrix_first = [&]() __attribute__((always_inline)) {  // step -1: S_0 only
    matrix_phase<BF16, D, true, false>(kb(0) + k_lane, vb(0), v_lane, qreg, sc, pb, oacc, no_hook, no_mid);
  };
  using NoIssue = std::integral_constant<int, 0>;
  using IssueSpread = std::integral_constant<int, 1>;
  using IssueUpfront = std::integral_constant<int, 2>;

  // P = exp(a - d) for the 32 scores of this lane against the reference
  // -neg_m, rounded to the MFMA type for the value product; returns the sum
  // of the fp32 weights (the denominator sums those: exact LSE) and, for
  // bf16, the lane's largest weight in wmax.
  auto weights = [&](float neg_m, float& wmax) __attribute__((always_inline)) -> float {
    float psum = 0.f, mx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int st = e >> 3, blk = st >> 1, r = 8 * (st & 1) + (e & 7);
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][r], c, neg_m));
      pb[st][e & 7] = (short)round16<BF16>(p);
      psum = e ? psum + p : p;  // the first weight starts the sum (no add of 0)
      if constexpr (BF16) mx = fmaxf(mx, p);
    }
    wmax = mx;
    return psum;
  };

  // Softmax phase of tile t (scores in sc).  Keys past Lk and (causal) past
  // the diagonal get score -inf and so weight exp2(-inf) = 0 (the scale is
  // positive here).  The weights are first taken against the current
  // reference d.  Every weight of a lane is at most that lane's sum, so when
  // no sum exceeds 2^8 (and every row has a reference) the weights stay
  // within 2^8 and the reference may stay.  Otherwise (a maximum jumped,
  // or an exponential overflowed to inf) the tile maximum is taken, the
  // reference advanced and the weights recomputed; the scores are still in
  // sc.  A tile this wave does not compute gets zero weights.
  auto softmax_tile = [&](int t) __attribute__((always_inline)) {
    // The common path falls through: the branches below are rarely taken
    // (a taken branch stalls this wave's vector issue while the other
    // wave's products run).
    if (__builtin_expect(t >= w_nkv, 0)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = s16x8{};
      return;
    }
    if (__builtin_expect(t >= j_mask, 0)) {
      // Score r of block blk is key kv0 + 8h + (32 blk + 16 (r/8) + r%8);
      // the lane's last allowed key (Lk - 1, or its query's diagonal) as an
      // offset `lim` on that constant: one compare per score.
      const int kv0 = (SPLIT ? t + jl_s : t) * BN;
      int lim = (CAUSAL ? min(Lk - 1, qi + off) : Lk - 1) - kv0 - 8 * h;
      asm volatile("" : "+v"(lim));  // per tile: keeps the compares in the loop
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * blk + 16 * (r >> 3) + (r & 7) > lim) sc[blk][r] = -INFINITY;
    }
    // This lane's largest score of the tile (keys excluded above are -inf).
    auto lane_max = [&]() __attribute__((always_inline)) -> float {
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          mx = fmaxf(mx, sc[blk][r]);
          mx = fmaxf(mx, sc[blk][r + 1]);
        }
      return mx;
    };
    // bf16: rounding error of the lane's largest weight (the weights are
    // monotone in the scores, so this is the weight of its largest score).
    auto round_error = [&](float wmax) __attribute__((always_inline)) -> float {
      return wmax - __builtin_bit_cast(float, (unsigned)round16<true>(wmax) << 16);
    };
    // Common path: against the current reference.  A row without one
    // (m_ref = -inf) gets weights +inf or NaN here, so its sum fails the
    // check below and the weights are recomputed there.
    float wmax;
    float psum = weights(-m_ref, wmax);
    float e_t = BF16 ? round_error(wmax) : 0.f;
    // The packed weights are complete before the check below, so the check
    // is the last thing of the phase on the common path.
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pb[i]));
    if (__builtin_expect(__any(!(psum <= kTauWeight)), 0)) {
      const float mx = halves_max(lane_max());
      // The guide's running maximum d_k = max(d_{k-1}, max of chunk k)
      // with headroom: a row whose tile maximum passed its reference moves
      // the reference kHeadroom above that maximum and corrects O~ and s by
      // exp(d_old - d_new); exact for any reference, and later tiles may
      // rise kHeadroom + 8 before they come back here.
      const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
      const bool grow = m_tile > m_ref;
      const float m_new = grow ? m_tile + kHeadroom<BF16> : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      m_ref = m_new;
      l_run *= alpha;
      if constexpr (BF16) e_run *= alpha;
#pragma unroll
      for (int i = 0; i < T::DBLK; ++i) oacc[i] *= alpha;
      // A row still without a reference (every key so far masked, split
      // key ranges only) keeps weight 0 for its masked scores.
      const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
      psum = weights(neg_m, wmax);
      if constexpr (BF16) e_t = round_error(wmax);
    }
    l_run += psum;
    if constexpr (BF16) e_run += e_t;
  };

  // First tiles of an item (K_0, V_0, K_1), by group 0.
  auto first_tiles = [&]() __attribute__((always_inline)) {
    dma_k(kb(0), 0);
    dma_v(vb(0), 0);
    if (1 < nkv) dma_k(kb(1), BN);
  };

  // ---- next item started during the current item's last step (unsplit
  //      kernel): that step reads no K tile and no Q, so the next item's
  //      Q, K_0, K_1 (and V_0 when the last V tile sits in the other
  //      buffer) load while the last value products run, instead of all
  //      waves sending their epilogue traffic through the memory pipe at
  //      once.  The current item's output rows are saved first. ----
  unsigned short* o_rows = nullptr;  // O row wq0 of the finishing item
  float* l_rows = nullptr;           // its LSE row wq0
  int rows_cur = 0;                  // its rows from wq0 on
  bool v0_issued = false;            // V_0 of the next item already issued
  int round = 0;
  int logical = item_at(0);
  auto begin_next = [&](bool issue_dma) __attribute__((always_inline)) {
    o_rows = O + ((size_t)bh * Lq + wq0) * D;
    l_rows = LSE + (size_t)bh * Lq + wq0;
    rows_cur = Lq - wq0;
    const int nkv_cur = nkv;
    logical = item_at(++round);
    if (logical >= 0) {
      setup(logical);
      if (issue_dma) {
        dma_k(kb(0), 0);
        if (1 < nkv) dma_k(kb(1), BN);
        v0_issued = (nkv_cur & 1) == 0;  // the last V tile is in buffer 1
        if (v0_issued) dma_v(vb(0), 0);
      }
      load_q();
    }
  };
  // O = O~ / s and lse = ln 2 (d + log2 s) of the finishing item.  Each wave
  // stages its 32 rows of O in LDS so that the global stores are whole
  // 16-byte chunks of consecutive rows.
  auto store_rows = [&]() __attribute__((always_inline)) {
    char* ob = smem + LY::OST + w * 32 * LY::OPITCH;
    const float l_tot = halves_sum(l_run);
    const float inv = 1.f / (BF16 ? halves_sum(l_run - e_run) : l_tot);
#pragma unroll
    for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * db + 8 * jj + 4 * h;
        const unsigned lo = (unsigned)round16<BF16>(oacc[db][4 * jj + 0] * inv) |
                            ((unsigned)round16<BF16>(oacc[db][4 * jj + 1] * inv) << 16);
        const unsigned hi = (unsigned)round16<BF16>(oacc[db][4 * jj + 2] * inv) |
                            ((unsigned)round16<BF16>(oacc[db][4 * jj + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(ob + n * LY::OPITCH + d * 2) = make_uint2(lo, hi);
      }
    if (h == 0 && n < rows_cur) l_rows[n] = (m_ref + log2f(l_tot)) * kLn2;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staged rows
    constexpr int ROWS = 64 / T::CPR;  // rows per 64-lane store
    u32x4 orow[32 / ROWS];
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
      const int row = ROWS * i + lane / T::CPR, chunk = lane % T::CPR;
      orow[i] = *reinterpret_cast<const u32x4*>(ob + row * LY::OPITCH + chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < 32 / ROWS; ++i) {
      const int row = ROWS * i + lane / T::CPR, chunk = lane % T::CPR;
      if (row < rows_cur) *reinterpret_cast<u32x4*>(o_rows + (size_t)row * D + chunk * 8) = orow[i];
    }
  };
  if (logical < 0) return;  // the whole workgroup: no barrier pending
  setup(logical);
  if (grp == 0) first_tiles();
  load_q();
  if (grp == 0) land(vb(0), 0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < T::DBLK; ++i) oacc[i] = f32x16{};
    m_ref = -INFINITY;
    l_run = 0.f;
    e_run = 0.f;
    barrier_lds();  // the item's first tiles have landed
    sign_q();

    // ---- the two groups' schedules, as separate loops (each wave executes
    //      the same sequence of barriers) ----
    // Step j: group 0 runs matrix(j) then softmax(j+1); group 1 runs
    // softmax(j) then matrix(j), half a step later.  Group 0 issues the DMA
    // of K_{j+2} and V_{j+1} during its matrix phase and waits for it at
    // the end of its softmax phase.  Step -1 computes S_0 only.
    if (grp == 0) {
      __builtin_amdgcn_s_setprio(1);
      matrix_first();
      barrier_lds();
      __builtin_amdgcn_s_setprio(0);
      softmax_tile(0);
      barrier_lds();
      // Steps whose next tiles K_{j+2} and V_{j+1} are whole, then the rest.
      // Steps past the wave's last tile (j >= w_nkv, causal) run in the
      // second loop, which leaves out their products.
      const int j_spread = max(0, min(min(nkv - 2, w_nkv), Lk / BN - 2 - (SPLIT ? jl_s : 0)));
      int j = 0;
      auto spread_step = [&](int jj) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        matrix(jj, IssueSpread{});
        softmax_tile(jj + 1);
        land(vb(jj + 1), (jj + 1) * BN);
        barrier_lds();
      };
      // Two steps per iteration: the buffer parity of each is then known at
      // compile time and the tile offsets fold into the LDS read offsets.
      for (; j + 1 < j_spread; j += 2) {
        spread_step(j);
        spread_step(j + 1);
      }
      if (j < j_spread) spread_step(j++);
      for (; j < (SPLIT ? nkv : nkv - 1); ++j) {
        __builtin_amdgcn_s_setprio(1);
        matrix_tail(j, IssueUpfront{});
        softmax_tile(j + 1);
        if (j + 1 < nkv) land(vb(j + 1), (j + 1) * BN);
        barrier_lds();
      }
      if constexpr (!SPLIT) {
        // Last step: value products, then the next item's loads and this
        // item's rows while group 1 finishes its value products.
        __builtin_amdgcn_s_setprio(1);
        matrix_last(j, end_phase);
        begin_next(true);
        store_rows();
        barrier_lds();
        if (logical >= 0 && !v0_issued) dma_v(vb(0), 0);  // buffer 0 read until now
      }
    } else {
      barrier_lds();
      __builtin_amdgcn_s_setprio(1);
      matrix_first();
      barrier_lds();
      auto step = [&](int jj) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(0);
        softmax_tile(jj);
        barrier_lds();
        __builtin_amdgcn_s_setprio(1);
        matrix(jj, NoIssue{});
      };
      // Full steps j < nkv - 1, two per iteration as for group 0, up to the
      // wave's last tile; steps past it without products; then the last
      // step, which needs no scores.
      int j = 0;
      const int j_full = min(nkv - 1, w_nkv);
      for (; j + 1 < j_full; j += 2) {
        step(j);
        step(j + 1);
      }
      if (j < j_full) step(j++);
      for (; j + 1 < nkv; ++j) {
        __builtin_amdgcn_s_setprio(0);
        softmax_tile(j);
        barrier_lds();
        __builtin_amdgcn_s_setprio(1);
        matrix_tail(j, NoIssue{});
      }
      if (j < nkv) {
        __builtin_amdgcn_s_setprio(0);
        softmax_tile(j);
        barrier_lds();
        __builtin_amdgcn_s_setprio(1);
        if constexpr (SPLIT) {
          matrix_tail(j, NoIssue{});
        } else {
          matrix_last(j, prio_low);
          begin_next(false);
          store_rows();
          barrier_lds();
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);

    if constexpr (SPLIT) {
      // ---- epilogue of a key range: normalised partial O and its
      //      log-sum-exp (-inf, with O = 0, for a row with no key in it) ----
      const float l_tot = halves_sum(l_run);
      const float l_o = BF16 ? halves_sum(l_run - e_run) : l_tot;
      const float inv = l_tot > 0.f ? 1.f / l_o : 0.f;
      if (qi < Lq) {
        const size_t prow_ix = ((size_t)sp_s * BH + bh) * Lq + qi;
        float* po = part_o + prow_ix * D;
#pragma unroll
        for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<float4*>(po + 32 * db + 8 * jj + 4 * h) =
                make_float4(oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv, oacc[db][4 * jj + 2] * inv,
                            oacc[db][4 * jj + 3] * inv);
        if (h == 0) part_l[prow_ix] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      }
      logical = item_at(++round);
      if (logical < 0) break;
      setup(logical);
      if (grp == 0) first_tiles();
      load_q();
      if (grp == 0) land(vb(0), 0);
      continue;
    }
    // ---- unsplit: the rows were stored and the next item's loads issued
    //      in the last step ----
    if (logical < 0) break;
    if (grp == 0) land(vb(0), 0);
  }
}

template <bool BF16, int D, bool CAUSAL, bool SPLIT>
hipError_t launch(const PrefillArgs& a, hipStream_t s, const PrefillSplitPlan& plan, float* part_o, float* part_l) {
  const int nqt = (a.Lq + kRows - 1) / kRows;
  const unsigned qsign = a.neg ? 0x80008000u : 0u;
  const int total = a.BH * (SPLIT ? plan.items : nqt);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int resident = 0;
  e = resident_workgroups(dev, reinterpret_cast<const void*>(&prefill_pp_kernel<BF16, D, CAUSAL, SPLIT>),
                          kThreads, &resident);
  if (e != hipSuccess) return e;
  const int cap = resident / 8 * 8;
  int grid, slots, per;
  if (cap >= 8 && total > cap) {  // persistent: one resident wave of workgroups
    grid = cap;
    slots = cap / 8;
    per = (total + 7) / 8;
  } else if (total % 8 == 0) {  // one item each, contiguous ranges per XCD
    grid = total;
    slots = total / 8;
    per = total / 8;
  } else {
    grid = total;
    slots = 0;
    per = 0;
  }
  hipLaunchKernelGGL((prefill_pp_kernel<BF16, D, CAUSAL, SPLIT>), dim3(grid), dim3(kThreads), 0, s,
                     static_cast<const unsigned short*>(a.q), static_cast<const unsigned short*>(a.k),
                     static_cast<const unsigned short*>(a.v), static_cast<unsigned short*>(a.o), a.lse, a.BH, a.Lq,
                     a.Lk, nqt, a.c, qsign, slots, per, part_o, part_l, plan);
  return hipGetLastError();
}

// Merge of the key ranges of a split prefill, one row of D = 128 per 128
// threads; the row's query tile has plan.ranges[qt] ranges.  With lse_p the
// ranges' log-sum-exps and m = max_p lse_p,
// O = sum_p exp(lse_p - m) O_p / sum_p exp(lse_p - m) and
// LSE = m + ln sum_p exp(lse_p - m) -- the guide's output correction with a
// key range as the chunk (ranges without a key, lse_p = -inf, drop out).
template <bool BF16>
__global__ __launch_bounds__(256) void prefill_split_combine(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_l,
                                                             unsigned short* __restrict__ O, float* __restrict__ LSE,
                                                             int rows, int Lq, const PrefillSplitPlan plan) {
  const int row = blockIdx.x * 2 + (threadIdx.x >> 7);  // (b h) * Lq + q
  const int d = threadIdx.x & 127;
  if (row >= rows) return;
  const int n_split = plan.ranges[(row % Lq) / kRows];
  float m = -INFINITY;
  for (int p = 0; p < n_split; ++p) m = fmaxf(m, part_l[(size_t)p * rows + row]);
  float acc = 0.f, wsum = 0.f;
  if (m != -INFINITY) {
    for (int p = 0; p < n_split; ++p) {
      const float lp = part_l[(size_t)p * rows + row];
      const float wp = lp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((lp - m) * kLog2e);
      wsum += wp;
      acc = __builtin_fmaf(wp, part_o[((size_t)p * rows + row) * 128 + d], acc);
    }
  }
  O[(size_t)row * 128 + d] = round16<BF16>(wsum > 0.f ? acc / wsum : 0.f);
  if (d == 0) LSE[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

}  // namespace

template <int D>
hipError_t launch_unsplit(int dtype, bool causal, const PrefillArgs& a, hipStream_t s) {
  static const PrefillSplitPlan none{};  // not read by the unsplit kernel
  if (dtype == 2)
    return causal ? launch<true, D, true, false>(a, s, none, nullptr, nullptr)
                  : launch<true, D, false, false>(a, s, none, nullptr, nullptr);
  return causal ? launch<false, D, true, false>(a, s, none, nullptr, nullptr)
                : launch<false, D, false, false>(a, s, none, nullptr, nullptr);
}

hipError_t launch_prefill_pp(int dtype, int D, bool causal, const PrefillArgs& a, hipStream_t s) {
  return D == 64 ? launch_unsplit<64>(dtype, causal, a, s) : launch_unsplit<128>(dtype, causal, a, s);
}

hipError_t launch_prefill_pp_split(int dtype, bool causal, const PrefillArgs& a, const PrefillSplitPlan& plan,
                                   float* part_o, float* part_l, hipStream_t s) {
  hipError_t e;
  if (dtype == 2)
    e = causal ? launch<true, 128, true, true>(a, s, plan, part_o, part_l)
               : launch<true, 128, false, true>(a, s, plan, part_o, part_l);
  else
    e = causal ? launch<false, 128, true, true>(a, s, plan, part_o, part_l)
               : launch<false, 128, false, true>(a, s, plan, part_o, part_l);
  if (e != hipSuccess) return e;
  const int rows = a.BH * a.Lq;
  if (dtype == 2)
    prefill_split_combine<true><<<dim3((rows + 1) / 2), dim3(256), 0, s>>>(
        part_o, part_l, static_cast<unsigned short*>(a.o), a.lse, rows, a.Lq, plan);
  else
    prefill_split_combine<false><<<dim3((rows + 1) / 2), dim3(256), 0, s>>>(
        part_o, part_l, static_cast<unsigned short*>(a.o), a.lse, rows, a.Lq, plan);
  return hipGetLastError();
}

bool prefill_pp_plan_splits(int BH, int Lq, int Lk, bool causal, int cus, int forced, PrefillSplitPlan* plan) {
  const int nqt = (Lq + kRows - 1) / kRows;
  if (nqt < 1 || nqt > kSplitMaxTiles) return false;
  const int off = Lk - Lq;
  int nkv[kSplitMaxTiles];
  long long kv_sum = 0;
  int min_nkv = 1 << 30;
  for (int qt = 0; qt < nqt; ++qt) {
    const int q_last = min((qt + 1) * kRows, Lq) - 1;
    nkv[qt] = causal ? (min(Lk, q_last + off + 1) + BN - 1) / BN : (Lk + BN - 1) / BN;
    kv_sum += nkv[qt];
    min_nkv = min(min_nkv, nkv[qt]);
  }
  if (min_nkv < 1) return false;  // a tile without keys: the unsplit kernel handles it
  int count[kSplitMaxTiles];
  if (forced > 0) {
    const int sp = min(forced, min(min_nkv, 16));
    if (sp < 2 || (long long)nqt * sp > kSplitMaxItems) return false;
    for (int qt = 0; qt < nqt; ++qt) count[qt] = sp;
  } else {
    if ((long long)BH * nqt * 2 > cus) return false;
    // Range size R (key tiles): from an even share of the whole job per
    // compute unit, grown until one range per workgroup covers the shape.
    long long R = max(8LL, ((long long)BH * kv_sum + cus - 1) / cus);
    for (;; ++R) {
      long long items = 0;
      for (int qt = 0; qt < nqt; ++qt) {
        count[qt] = (int)min((long long)kSplitMaxRanges, (nkv[qt] + R - 1) / R);
        items += count[qt];
      }
      if (items <= kSplitMaxItems && BH * items <= cus) break;
    }
    bool any = false;
    for (int qt = 0; qt < nqt; ++qt) any = any || count[qt] > 1;
    if (!any) return false;
  }
  int t = 0, mx = 1;
  for (int i = 0; i < nqt; ++i) {
    const int qt = causal ? nqt - 1 - i : i;  // heaviest tiles first
    plan->ranges[qt] = (unsigned char)count[qt];
    mx = max(mx, count[qt]);
    for (int sp = 0; sp < count[qt]; ++sp) plan->item[t++] = (unsigned short)((qt << 5) | sp);
  }
  plan->items = t;
  plan->max_ranges = mx;
  return true;
}

}  // namespace attn
