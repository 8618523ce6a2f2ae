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
//   * key/value tiles of 64 rows go HBM -> LDS by DMA (no VGPR round trip),
//     double buffered one tile out of phase (the next tiles land while the
//     current ones are computed);
//   * S^T = K_j Q^T is computed so that each lane holds 32 scores of ONE
//     query: row statistics need no cross-lane reduction except one
//     permlane32 swap per tile;
//   * K rows are read in a bit-permuted order (bits 2 and 3 of the row index
//     swapped) so that the score registers of a lane are already the B
//     operand (P^T, 8 consecutive keys) of the P V product;
//   * V stays row-major in LDS and is read transposed with ds_read_b64_tr_b16
//     to form the A operand (V^T) of O^T += V^T P^T.
//
// Reference maximum: the guide's correction exp(d_old - d_new) gives the same
// O and LSE for any reference d, so d moves only when needed.  fp16 computes
// the weights against the current d and checks that no lane's weight sum
// passes 2^8 (then no weight does, and the fp16 weights cannot overflow);
// otherwise the tile's row maximum becomes d, O~ and s are corrected and the
// weights recomputed (rare).  bf16 keeps a look-ahead: the row maximum of the
// next tile is reduced while the current one's value product runs, d moves
// before that tile's weights when it passes d + 8, and the same maximum
// gives the rounding term of the largest weight (below).
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_internal.hpp"
#include "mfma_tile.hpp"

namespace attn {
namespace {

using namespace mt;

constexpr int BM = 128;  // query rows per workgroup
constexpr int NT = 256;  // threads per workgroup
constexpr int NW = NT / 64;  // waves per workgroup
// Largest lag (base 2) of the reference maximum behind the true running
// maximum: weights exp(a - d) stay below 2^8.
constexpr float kTau = 8.f;

// ---- steady-state step as a fixed sequence of MFMA slots ----
// One step of a wave computes S_{j+1} = K_{j+1} Q^T (NS MFMAs), the weights
// P_j of the scores it already holds (VALU), O~ += V_j^T P_j (NP MFMAs) and
// the row maximum of S_{j+1} (VALU).  The order is fixed in source: slot i
// issues one MFMA, a share of the softmax elements, a share of the max
// reduction and now and then one DMA run for the next tiles; every even slot
// issues the LDS reads of the operand pair PF slots ahead (K fragments, then
// V fragments, so V reads overlap the end of the S products), the later
// operand first, so that a single wait covers both MFMAs of the pair.  A
// scheduling fence keeps the slots apart.  A few softmax elements run before
// slot 0 so that the first K reads are in flight while the VALU works.
constexpr int kDmaRun = 2;  // DMA instructions per M0 run

template <int D, bool LOOKAHEAD>
struct Slots {
  using T = Tile<D>;
  using KP = DmaPlan<T::KINST, kDmaRun, NW>;
  using VP = DmaPlan<T::VINST, kDmaRun, NW>;
  static constexpr int NS = 2 * T::KSTEPS;   // S MFMAs
  static constexpr int NP = 4 * T::DBLK;     // P V MFMAs
  static constexpr int N = NS + NP;
  static constexpr int PF = 4;               // read lookahead, in slots (even)
  static constexpr int F = 6;                // softmax elements before slot 0
  // Slots the other elements spread over: with the look-ahead maximum the
  // weights may run into the first value products of their k-step; with the
  // weight-sum check every weight is done before the first value product.
  static constexpr int NV = LOOKAHEAD ? NS + 2 * T::DBLK : NS;
  static constexpr int NR = KP::RUNS + VP::RUNS;  // DMA runs per step (K first)
  // Slot of softmax element e >= F, of max step m (values 2m, 2m+1), of DMA run q.
  static constexpr int elem_slot(int e) { return (e - F) * NV / (32 - F); }
  static constexpr int max_slot(int m) { return NS + 2 + m * (NP - 2) / 16; }
  static constexpr int dma_slot(int q) { return 1 + q * (N - 2) / NR; }
  static constexpr bool deadlines_met() {
    // P_j rows of k-step st feed PV slot NS + st * DBLK.
    for (int st = 0; st < 4; ++st)
      if (8 * st + 7 >= F && elem_slot(8 * st + 7) >= NS + st * T::DBLK) return false;
    return true;
  }
  static_assert(deadlines_met(), "softmax element scheduled after its value product");
  static_assert(LOOKAHEAD || elem_slot(31) < NS, "weights must be done before the check");
  static_assert(PF % 2 == 0 && NS % 2 == 0 && NP % 2 == 0, "operand pairs");
  static_assert(max_slot(15) < N && dma_slot(NR - 1) < N, "slot overflow");
};

// The weight-sum check failed for some row of the wave (fp16): the tile's
// row maximum (base-2 scaled units) becomes the reference where it is above
// the old one, O~ and the lane's sum s take the guide's correction
// exp(d_old - d_new), and the weights of the tile are recomputed (now all at
// most 1).  `live` gives the unmasked keys when MASK.
template <bool BF16, int D, bool MASK>
__device__ __forceinline__ void move_reference(const f32x16 (&s)[2], s16x8 (&pb)[4], f32x16 (&oacc)[D / 32],
                                                         float c, unsigned live, float& m_ref, float& l_run,
                                                         float& psum) {
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
  mx = halves_max(mx);
  const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
  const bool grow = m_tile > m_ref;
  const float m_new = grow ? m_tile : m_ref;
  const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
  m_ref = m_new;
  l_run *= alpha;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
  const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
  psum = 0.f;
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int blk = st >> 1, r = 8 * (st & 1) + e;
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][r], c, -m_use));
      if constexpr (MASK) p = ((live >> (16 * blk + r)) & 1u) ? p : 0.f;
      pb[st][e] = (short)round16<BF16>(p);
      psum = st || e ? psum + p : p;  // the first weight starts the sum
    }
}

// Weight-sum check: false when every weight of every row of the wave is at
// most 2^kTau and every row has a reference (a NaN sum fails too).
__device__ __forceinline__ bool weights_bounded(float psum, float m_ref) {
  constexpr float kSumMax = 256.f;  // 2^kTau
  return !__builtin_expect(__any(!(psum <= kSumMax) || m_ref == -INFINITY), 0);
}

template <bool BF16, int D>
__device__ __forceinline__ void fast_step(const char* kp, const char* vp, const s16x8 (&qreg)[D / 16],
                                          const f32x16 (&sc)[2], f32x16 (&sn)[2], f32x16 (&oacc)[D / 32],
                                          float c, float& m_ref, float& l_run, float& mx_out,
                                          const char* kgbase, char* kdst, const unsigned* k_off,
                                          const char* vgbase, char* vdst, const unsigned* v_off, int w) {
  constexpr bool LOOKAHEAD = BF16;
  using T = Tile<D>;
  using S = Slots<D, LOOKAHEAD>;
  using KP = typename S::KP;
  using VP = typename S::VP;
  if constexpr (VP::X != 0) {
    if (w < VP::X) dma_run<1>(vgbase, v_off + VP::U, lds_addr(vdst + VP::inst(VP::U, w) * 1024));
  }
  if constexpr (KP::X != 0) {
    if (w < KP::X) dma_run<1>(kgbase, k_off + KP::U, lds_addr(kdst + KP::inst(KP::U, w) * 1024));
  }
  s16x8 fr[S::N];
  s16x8 pb[4];
  float psum = 0.f;
  float mx = -INFINITY;
  const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
  auto read = [&](int r) {
    if (r < S::NS) {
      fr[r] = *reinterpret_cast<const s16x8*>(kp + 32 * (r & 1) * T::KPITCH + 32 * (r >> 1));
    } else {
      const int x = r - S::NS, st = x / T::DBLK, db = x % T::DBLK;
      const char* p = vp + 16 * st * T::VPITCH + 64 * db;
      const s16x4 lo = lds_read_tr(p);
      const s16x4 hi = lds_read_tr(p + 4 * T::VPITCH);
      fr[r] = s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto read_pair = [&](int r) {  // operands r and r + 1, the later one first
    read(r + 1);
    read(r);
  };
  auto elem = [&](int e) {
    const int blk = e >> 4, r = e & 15;
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[blk][r], c, neg_m));
    pb[e >> 3][e & 7] = (short)round16<BF16>(p);
    psum = e ? psum + p : p;  // the first weight starts the sum
  };
  auto dma = [&](int q) {
    if (q < KP::RUNS) {
      const int i0 = KP::run_first(q);
      dma_run_n(KP::run_len(q), kgbase, k_off + i0, lds_addr(kdst + KP::inst(i0, w) * 1024));
    } else {
      const int qv = q - KP::RUNS;
      const int i0 = VP::run_first(qv);
      dma_run_n(VP::run_len(qv), vgbase, v_off + i0, lds_addr(vdst + VP::inst(i0, w) * 1024));
    }
  };
#pragma unroll
  for (int r = 0; r < S::PF; r += 2) read_pair(r);
#pragma unroll
  for (int e = 0; e < S::F; ++e) elem(e);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < S::N; ++i) {
    if (i % 2 == 0 && i + S::PF < S::N) read_pair(i + S::PF);
#pragma unroll
    for (int q = 0; q < S::NR; ++q)
      if (S::dma_slot(q) == i) dma(q);
    if (i < S::NS) {
      const int blk = i & 1;
      sn[blk] = mfma32<BF16>(fr[i], qreg[i >> 1], i < 2 ? f32x16{} : sn[blk]);
    } else {
      const int x = i - S::NS;
      oacc[x % T::DBLK] = mfma32<BF16>(fr[i], pb[x / T::DBLK], oacc[x % T::DBLK]);
    }
#pragma unroll
    for (int e = S::F; e < 32; ++e)
      if (S::elem_slot(e) == i) elem(e);
    if constexpr (LOOKAHEAD) {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        if (S::max_slot(m) == i) {
          mx = fmaxf(mx, sn[m >> 3][2 * (m & 7)]);
          mx = fmaxf(mx, sn[m >> 3][2 * (m & 7) + 1]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!LOOKAHEAD) {
      // Every weight of the tile is done: check them before the first value
      // product uses them.
      if (i == S::NS - 1) {
        if (!weights_bounded(psum, m_ref)) move_reference<BF16, D, false>(sc, pb, oacc, c, 0u, m_ref, l_run, psum);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  l_run += psum;
  mx_out = mx;
}

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void prefill_mfma_kernel(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K,
    const unsigned short* __restrict__ V, unsigned short* __restrict__ O, float* __restrict__ LSE,
    int BH, int Lq, int Lk, int nqt, float c, unsigned qsign) {
  using T = Tile<D>;
  // K tiles and V tiles are double buffered in their own arrays, one tile out
  // of phase: step j reads K_{j+1} and V_j while K_{j+2} and V_{j+1} land.
  __shared__ __attribute__((aligned(16))) char kb0[T::KBYTES];
  __shared__ __attribute__((aligned(16))) char kb1[T::KBYTES];
  __shared__ __attribute__((aligned(16))) char vb0[T::VBYTES];
  __shared__ __attribute__((aligned(16))) char vb1[T::VBYTES];

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
  const char* Kb = reinterpret_cast<const char*>(K + (size_t)bh * Lk * D);
  const char* Vb = reinterpret_cast<const char*>(V + (size_t)bh * Lk * D);

  const int q_last = min(q0 + BM, Lq) - 1;
  const int kv_end = CAUSAL ? min(Lk, q_last + off + 1) : Lk;
  const int nkv = (kv_end + BN - 1) / BN;  // tiles the workgroup streams
  const int wq0 = q0 + 32 * w;             // first query of this wave
  const int w_key_end = CAUSAL ? min(Lk, min(wq0 + 31, Lq - 1) + off + 1) : Lk;
  // Tiles [0, w_nkv) are computed by this wave; tiles [0, j_mask) hold no
  // masked key for it (the causal diagonal band and the Lk tail do).
  const int w_nkv = __builtin_amdgcn_readfirstlane(wq0 < Lq ? (w_key_end + BN - 1) / BN : 0);
  int j_mask = w_nkv;
  if (CAUSAL) {
    const int first_bad = wq0 + off - BN + 2;  // first kv0 whose last key passes the diagonal
    j_mask = min(j_mask, first_bad <= 0 ? 0 : (first_bad + BN - 1) / BN);
  }
  if (Lk % BN) j_mask = min(j_mask, Lk / BN);
  j_mask = __builtin_amdgcn_readfirstlane(j_mask);

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

  // DMA of one K or V tile (DmaPlan); rows past Lk read row Lk-1 and the V
  // slots of those rows are zeroed once the DMA has landed.  Offsets are
  // biased for dma_run.
  using KP = typename Slots<D, BF16>::KP;
  using VP = typename Slots<D, BF16>::VP;
  unsigned k_src[KP::N];
  unsigned v_src[VP::N];
#pragma unroll
  for (int i = 0; i < KP::N; ++i)
    k_src[i] = dma_src_offset<D>(KP::inst(i, w), lane, T::KSPR) + kDmaBias - KP::pos_in_run(i) * 1024u;
#pragma unroll
  for (int i = 0; i < VP::N; ++i)
    v_src[i] = dma_src_offset<D>(VP::inst(i, w), lane, T::VSPR) + kDmaBias - VP::pos_in_run(i) * 1024u;
  // Global base of a tile lowered by the DMA bias (the sum with every lane
  // offset is inside the tile).
  auto biased = [](const char* p) {
    return reinterpret_cast<const char*>(reinterpret_cast<uintptr_t>(p) - kDmaBias);
  };
  // full_tag: the caller knows the tile lies entirely before Lk.
  auto dma_k = [&](char* buf, int kv0, auto full_tag) {
    const char* g = biased(Kb + (size_t)kv0 * (D * 2));
    if (decltype(full_tag)::value || kv0 + BN <= Lk)
      dma_tile_whole<KP>(g, buf, k_src, w);
    else
      dma_tile_ragged<D, KP>(g, buf, k_src, w, Lk - kv0);
  };
  auto dma_v = [&](char* buf, int kv0, auto full_tag) {
    const char* g = biased(Vb + (size_t)kv0 * (D * 2));
    if (decltype(full_tag)::value || kv0 + BN <= Lk)
      dma_tile_whole<VP>(g, buf, v_src, w);
    else
      dma_tile_ragged<D, VP>(g, buf, v_src, w, Lk - kv0);
  };
  const std::integral_constant<bool, false> maybe_ragged{};
  auto land = [&](char* vbuf, int kv0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (kv0 + BN > Lk) {
#pragma unroll
      for (int i = 0; i < VP::N; ++i) {
        if (i < VP::U || w < VP::X) {
          const int slot = VP::inst(i, w) * 64 + lane;
          if (kv0 + slot / T::VSPR >= Lk) *reinterpret_cast<u32x4*>(vbuf + slot * 16) = u32x4{0u, 0u, 0u, 0u};
        }
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
  // bf16: sum over tiles of the rounding error (fp32 weight minus its bf16
  // value) of the row's largest weight of the tile, half in each lane of
  // the row.  The value product takes the rounded weights, so O is divided
  // by l_run - e_run: the dominant weight then has the same rounding in the
  // numerator and the denominator.  LSE keeps the unrounded sum.
  float e_run = 0.f;
  float m_cur = -INFINITY;  // maximum (base-2 scaled) of the tile whose weights come next

  // Tile row read by this lane for S^T: bits 2 and 3 of n swapped, so the
  // accumulator register r of block blk holds key 32 blk + 16 (r/8) + 8 h + r%8.
  const int prow = (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1);
  const int g = lane >> 4, li = lane & 15;

  // ---- building blocks of one tile ----
  // S^T = K Q^T for the 64 keys of a K tile (two 32-key blocks, 16 MFMAs).
  // The two blocks alternate so consecutive MFMAs never wait on each other.
  auto scores = [&](f32x16 (&s)[2], const char* Ks) {
    const char* kp = Ks + prow * T::KPITCH + 16 * h;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int t = 0; t < T::KSTEPS; ++t)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        s[blk] = mfma32<BF16>(*reinterpret_cast<const s16x8*>(kp + 32 * blk * T::KPITCH + 32 * t), qreg[t],
                              s[blk]);
  };
  // Keys past Lk and (causal) past the diagonal get score -inf; returns the
  // bit mask of the live ones.
  auto mask_scores = [&](f32x16 (&s)[2], int kv0) -> unsigned {
    // Per-lane key offset and query made opaque here, so the per-element
    // bounds are not hoisted out of the tile loop (registers).
    int hk = 8 * h, q = qi;
    asm volatile("" : "+v"(hk), "+v"(q));
    unsigned live = 0u;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * blk + 16 * (r >> 3) + hk + (r & 7);
        const bool ok = key < Lk && (!CAUSAL || key <= q + off);
        live |= (ok ? 1u : 0u) << (16 * blk + r);
        if (!ok) s[blk][r] = -INFINITY;
      }
    return live;
  };
  // Row maximum of a tile in base-2 scaled units (-inf if no live key).
  auto row_max = [&](const f32x16 (&s)[2]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk][r]);
    mx = halves_max(mx);
    return (mx == -INFINITY) ? -INFINITY : mx * c;
  };
  // The guide's running maximum d_k = max(d_{k-1}, max of chunk k), with a
  // lag: the reference d moves to the new maximum only when a tile's
  // maximum exceeds it by more than kTau (base 2); then O~ and s get the
  // correction exp(d_old - d_new).  Otherwise d stays, the weights
  // exp(a - d) are at most 2^kTau, and O~ / s is unchanged in real
  // arithmetic (the correction holds for any reference).  The branch is
  // taken by the whole wave if any of its rows needs it.
  auto advance_max = [&](float m_tile) {
    const bool grow = m_tile > m_ref + kTau;
    if (__any(grow)) {
      const float m_new = grow ? m_tile : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      m_ref = m_new;
      l_run *= alpha;
      if constexpr (BF16) e_run *= alpha;
#pragma unroll
      for (int i = 0; i < T::DBLK; ++i) oacc[i] *= alpha;
    }
  };
  // Rounding error of the largest weight of a tile with maximum m_tile,
  // weights taken against m_use (half of it: both lanes of the row add it).
  auto add_round_error = [&](float m_tile, float m_use) {
    if constexpr (BF16) {
      const float wmax = __builtin_amdgcn_exp2f(m_tile - m_use);
      const float wr = __builtin_bit_cast(float, (unsigned)round16<true>(wmax) << 16);
      e_run += 0.5f * (wmax - wr);
    }
  };
  // P = exp(a - d), rounded to the MFMA type for the value product; the
  // denominator sums the fp32 weights (exact LSE).
  auto probs = [&](const f32x16 (&s)[2], s16x8 (&pb)[4], unsigned live, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int blk = st >> 1, r = 8 * (st & 1) + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][r], c, -m_use));
        if constexpr (MASK) p = ((live >> (16 * blk + r)) & 1u) ? p : 0.f;
        pb[st][e] = (short)round16<BF16>(p);
        psum = st || e ? psum + p : p;  // the first weight starts the sum
      }
    }
    if constexpr (!BF16) {
      if (!weights_bounded(psum, m_ref)) move_reference<BF16, D, MASK>(s, pb, oacc, c, live, m_ref, l_run, psum);
    }
    l_run += psum;
  };
  // O^T += V^T P^T; V^T fragments via transposed LDS reads.
  auto pv = [&](const s16x8 (&pb)[4], const char* Vs) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
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

  // ---- prologue: K_0, V_0, K_1 in LDS; scores of tile 0 ----
  dma_k(kb0, 0, maybe_ragged);
  dma_v(vb0, 0, maybe_ragged);
  if (nkv > 1) dma_k(kb1, BN, maybe_ragged);
  land(vb0, 0);
  __syncthreads();
  f32x16 sa[2], sb[2];
  unsigned live_a = 0xffffffffu, live_b = 0xffffffffu;
  if (w_nkv > 0) {
    scores(sa, kb0);
    if (j_mask == 0) live_a = mask_scores(sa, 0);
    m_cur = row_max(sa);
    advance_max(m_cur);
  }
  __syncthreads();  // kb0 is refilled with K_2 in step 0

  // ---- step j: holds the scores of tile j (sc), computes those of tile j+1 (sn) ----
  //   phase A: S_{j+1} = K_{j+1} Q^T on MFMA, overlapped with P_j on VALU
  //   phase B: O += V_j^T P_j on MFMA, overlapped with the max of S_{j+1}
  //   then the running-maximum update for tile j+1 (rarely taken branch).
  // FAST: tiles j and j+1 both computed by this wave and unmasked.
  // PAR: the parity of j, when the caller knows it at compile time (0 or 1),
  // otherwise -1; with a known parity every LDS buffer is a fixed array.
  auto step = [&](int j, f32x16 (&sc)[2], unsigned live_c, f32x16 (&sn)[2], unsigned& live_n,
                  auto fast_tag, auto par_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    const bool odd = PAR < 0 ? (j & 1) != 0 : PAR == 1;
    char* kn = odd ? kb0 : kb1;   // K_{j+1}
    char* vc = odd ? vb1 : vb0;   // V_j
    char* kf = odd ? kb1 : kb0;   // receives K_{j+2}
    char* vf = odd ? vb0 : vb1;   // receives V_{j+1}
    // In FAST steps tiles j+1 and j+2 < j_mask <= Lk / BN are whole.
    if constexpr (!FAST) {
      if (j + 2 < nkv) dma_k(kf, (j + 2) * BN, std::integral_constant<bool, false>{});
      if (j + 1 < nkv) dma_v(vf, (j + 1) * BN, fast_tag);
    }
    const bool do_cur = FAST || j < w_nkv;
    const bool do_next = FAST || j + 1 < w_nkv;
    s16x8 pb[4];
    float m_next = -INFINITY;
    if constexpr (FAST) {
      float mx;
      fast_step<BF16, D>(kn + prow * T::KPITCH + 16 * h,
                         vc + (8 * h + (li >> 2)) * T::VPITCH + (16 * (g & 1) + 4 * (li & 3)) * 2, qreg, sc,
                         sn, oacc, c, m_ref, l_run, mx, biased(Kb + (size_t)(j + 2) * BN * (D * 2)), kf, k_src,
                         biased(Vb + (size_t)(j + 1) * BN * (D * 2)), vf, v_src, w);
      if constexpr (BF16) {
        mx = halves_max(mx);
        m_next = (mx == -INFINITY) ? -INFINITY : mx * c;
      }
    } else {
      // Fences between the phases keep the operand reads of one phase from
      // being hoisted into the previous one (register pressure).
      if (do_next) scores(sn, kn);
      __builtin_amdgcn_sched_barrier(0);
      if (do_cur) probs(sc, pb, live_c, std::integral_constant<bool, true>{});
      __builtin_amdgcn_sched_barrier(0);
      if (do_cur) pv(pb, vc);
      __builtin_amdgcn_sched_barrier(0);
      if (do_next) {
        live_n = mask_scores(sn, (j + 1) * BN);
        if constexpr (BF16) m_next = row_max(sn);
      }
    }
    if constexpr (BF16) {
      if (do_cur) add_round_error(m_cur, (m_ref == -INFINITY) ? 0.f : m_ref);
      if (do_next) advance_max(m_next);
      m_cur = do_next ? m_next : -INFINITY;
    }
    if (j + 1 < nkv) land(vf, (j + 1) * BN);
    __syncthreads();
  };

  // Fast steps j also need K_{j+2} to exist and be whole (its DMA is issued
  // unclamped inside the step).
  const int k_whole_end = min(nkv, Lk / BN);
  int j = 0;
  for (; j + 2 < j_mask && j + 3 < k_whole_end; j += 2) {
    step(j, sa, 0xffffffffu, sb, live_b, std::integral_constant<bool, true>{},
         std::integral_constant<int, 0>{});
    step(j + 1, sb, 0xffffffffu, sa, live_a, std::integral_constant<bool, true>{},
         std::integral_constant<int, 1>{});
  }
  if (j > 0) live_a = 0xffffffffu;  // tile j < j_mask: no masked key
  for (; j < nkv; ++j) {
    step(j, sa, live_a, sb, live_b, std::integral_constant<bool, false>{}, std::integral_constant<int, -1>{});
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) sa[blk] = sb[blk];
    live_a = live_b;
  }

  // ---- epilogue: O = O~ / s, lse = ln 2 (d + log2 s) ----
  // O goes through LDS (this wave's 32 rows, padded pitch) so that the
  // global stores are whole 16-byte chunks of consecutive rows.  Every wave
  // has passed the last barrier of the loop, so the V buffers are free.
  constexpr int OPITCH = D * 2 + 16;
  static_assert(2 * 32 * OPITCH <= T::VBYTES, "two waves' rows of O fit in one V buffer");
  char* ob = (w < 2 ? vb0 : vb1) + (w & 1) * 32 * OPITCH;
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
      *reinterpret_cast<uint2*>(ob + n * OPITCH + d * 2) = make_uint2(lo, hi);
    }
  if (h == 0 && qi < Lq) LSE[(size_t)bh * Lq + qi] = (m_ref + log2f(l_tot)) * kLn2;
  __syncthreads();
  constexpr int ROWS = 64 / T::CPR;  // rows per 64-lane store
#pragma unroll
  for (int i = 0; i < 32 / ROWS; ++i) {
    const int row = ROWS * i + lane / T::CPR, chunk = lane % T::CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ob + row * OPITCH + chunk * 16);
    if (wq0 + row < Lq)
      *reinterpret_cast<u32x4*>(O + ((size_t)bh * Lq + wq0 + row) * D + chunk * 8) = v;
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
