// Building blocks shared by the 16-bit prefill kernels on gfx950: MFMA
// wrappers, cross-half reductions, transposed LDS reads and the K/V tile
// DMA (HBM -> LDS without a VGPR round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace attn {
namespace mt {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;  // key rows per tile

template <int D>
struct Tile {
  // LDS rows are padded so that every read address is a lane base plus an
  // immediate offset, and both read patterns are bank-conflict-free:
  //  K: pitch = D*2 + 16 B (an odd number of 16-byte slots): 16 lanes
  //     reading one 16-byte chunk of 16 consecutive rows hit 16 different
  //     4-bank groups (ds_read_b128).
  //  V: pitch = D*2 + 64 B (4 mod 16 slots): the 4 rows x 64 B of one
  //     half-wave transposed read (ds_read_b64_tr_b16) hit disjoint banks.
  static constexpr int CPR = D / 8;             // 16-byte data chunks per row
  static constexpr int KSPR = CPR + 1;          // K slots per row (1 pad slot)
  static constexpr int VSPR = CPR + 4;          // V slots per row (4 pad slots)
  static constexpr int KPITCH = KSPR * 16;
  static constexpr int VPITCH = VSPR * 16;
  static constexpr int KBYTES = BN * KPITCH;
  static constexpr int VBYTES = BN * VPITCH;
  static constexpr int KINST = BN * KSPR / 64;  // 64-lane DMA instructions per K tile
  static constexpr int VINST = BN * VSPR / 64;  // ... per V tile
  static constexpr int KSTEPS = D / 16;         // MFMA k-steps of Q K^T
  static constexpr int DBLK = D / 32;           // 32-wide blocks of the output
  static_assert(BN * KSPR % 64 == 0 && BN * VSPR % 64 == 0, "whole DMA instructions");
};

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
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
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false,
                                            false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false,
                                            false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const char*)p;
}

// K/V tiles go HBM -> LDS by DMA (global_load_lds_dwordx4): one instruction
// moves 64 lanes x 16 B into 1 KB of consecutive LDS, here a run of 16-byte
// slots of the padded tile.  Lane l of DMA instruction i fills slot 64 i + l
// (row = slot / slots-per-row, chunk = the rest).
//
// One global_load_lds_dwordx4 moves 16 bytes per lane from global memory to
// LDS at M0 + 16 * lane; its immediate offset is added to BOTH addresses.
// A wave issues a run of up to four instructions of consecutive LDS
// kilobytes under one M0 value with offsets 0, 1024, 2048, 3072; the global
// base passed in SGPRs is lowered by kDmaBias so that every per-lane offset
// (source offset + kDmaBias - offset of the instruction in its run) stays
// non-negative.  Written as inline assembly so that the compiler's LGKM wait
// model does not count the DMA: with the builtin, every wait for an LDS read
// becomes a wait for all outstanding LDS traffic including this DMA.
// Completion is awaited explicitly with s_waitcnt vmcnt(0).
constexpr unsigned kDmaBias = 4096u;

// gbase and m0 must be wave-uniform (SGPR operands).
template <int G>
__device__ __forceinline__ void dma_run(const char* gbase, const unsigned* voff, unsigned m0) {
  static_assert(G >= 1 && G <= 4, "one M0 run holds 1 to 4 instructions");
  // Wave-uniform by contract; readfirstlane keeps it in an SGPR even where
  // the compiler computed it in a VGPR (free when it already is an SGPR).
  m0 = __builtin_amdgcn_readfirstlane(m0);
  if constexpr (G == 1)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %0\n"
                 :
                 : "s"(gbase), "s"(m0), "v"(voff[0])
                 : "memory", "m0");
  else if constexpr (G == 2)
    asm volatile(
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %0\n\t"
        "global_load_lds_dwordx4 %3, %0 offset:1024\n"
        :
        : "s"(gbase), "s"(m0), "v"(voff[0]), "v"(voff[1])
        : "memory", "m0");
  else if constexpr (G == 3)
    asm volatile(
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %0\n\t"
        "global_load_lds_dwordx4 %3, %0 offset:1024\n\tglobal_load_lds_dwordx4 %4, %0 offset:2048\n"
        :
        : "s"(gbase), "s"(m0), "v"(voff[0]), "v"(voff[1]), "v"(voff[2])
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %0\n\t"
        "global_load_lds_dwordx4 %3, %0 offset:1024\n\tglobal_load_lds_dwordx4 %4, %0 offset:2048\n\t"
        "global_load_lds_dwordx4 %5, %0 offset:3072\n"
        :
        : "s"(gbase), "s"(m0), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3])
        : "memory", "m0");
}

// Run of g instructions, g known once loops are unrolled.
__device__ __forceinline__ void dma_run_n(int g, const char* gbase, const unsigned* voff, unsigned m0) {
  switch (g) {
    case 1: dma_run<1>(gbase, voff, m0); break;
    case 2: dma_run<2>(gbase, voff, m0); break;
    case 3: dma_run<3>(gbase, voff, m0); break;
    default: dma_run<4>(gbase, voff, m0); break;
  }
}

// Per-wave DMA plan of one tile with INST instructions spread over NWV
// issuing waves: wave w issues the U = INST / NWV instructions
// w U .. w U + U - 1 (consecutive LDS kilobytes), in runs of at most RUN,
// and, when INST % NWV != 0, waves w < INST % NWV issue instruction U NWV + w
// as a run of one.  Index i of a wave's list: i < U: instruction w U + i;
// i == U: the extra one.
template <int INST, int RUN, int NWV>
struct DmaPlan {
  static constexpr int U = INST / NWV;
  static constexpr int X = INST % NWV;
  static constexpr int N = U + (X ? 1 : 0);  // list length (the extra may be idle)
  static constexpr int RUNS = (U + RUN - 1) / RUN;
  static constexpr int run_first(int r) { return r * RUN; }
  static constexpr int run_len(int r) { return (r + 1) * RUN <= U ? RUN : U - r * RUN; }
  static constexpr int pos_in_run(int i) { return i < U ? i % RUN : 0; }
  __device__ static int inst(int i, int w) { return i < U ? w * U + i : U * NWV + w; }
};

// Byte offset, within one tile of the source tensor, of the chunk that lane
// `lane` fetches for DMA instruction `inst` of a tile with `spr` slots per
// row; pad slots fetch chunk 0 of their row again (in bounds, never read).
template <int D>
__device__ __forceinline__ unsigned dma_src_offset(int inst, int lane, int spr) {
  const int slot = inst * 64 + lane;
  const int row = slot / spr;
  const int chunk = slot - row * spr;
  return (unsigned)row * (D * 2) + (unsigned)(chunk < D / 8 ? chunk : 0) * 16;
}

// Issue a wave's DMA for one whole tile (every row before Lk).  voff holds
// the biased per-lane offsets of the wave's list; gbase = tile - kDmaBias.
template <class P>
__device__ __forceinline__ void dma_tile_whole(const char* gbase, char* dst, const unsigned* voff, int w) {
#pragma unroll
  for (int r = 0; r < P::RUNS; ++r)
    dma_run_n(P::run_len(r), gbase, voff + P::run_first(r), lds_addr(dst + P::inst(P::run_first(r), w) * 1024));
  if constexpr (P::X != 0) {
    if (w < P::X) dma_run<1>(gbase, voff + P::U, lds_addr(dst + P::inst(P::U, w) * 1024));
  }
}

// Ragged tile: rows at or past `rows_left` read row rows_left - 1 instead
// (in bounds); one instruction per run.
template <int D, class P>
__device__ __forceinline__ void dma_tile_ragged(const char* gbase, char* dst, const unsigned* voff, int w,
                                                int rows_left) {
#pragma unroll
  for (int i = 0; i < P::N; ++i) {
    if (i < P::U || w < P::X) {
      unsigned off = voff[i];
      asm volatile("" : "+v"(off));  // not hoisted out of the tile loop
      off -= kDmaBias - P::pos_in_run(i) * 1024u;
      const int row = (int)(off / (D * 2));
      const unsigned o = row < rows_left ? off : (unsigned)(rows_left - 1) * (D * 2) + off % (D * 2);
      const unsigned vo = o + kDmaBias;
      dma_run<1>(gbase, &vo, lds_addr(dst + P::inst(i, w) * 1024));
    }
  }
}

}  // namespace mt
}  // namespace attn
