// Swizzled 64-row LDS tiles (read along rows and across rows without bank
// conflicts), their DMA, and small compile-time helpers shared by the
// backward kernels and the masked / dropout forward.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "mfma_tile.hpp"

namespace attn {
namespace st {

using namespace mt;

constexpr int BQ = 64;  // rows per LDS tile

template <int D>
struct SwzTile {
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static constexpr int PITCH = D * 2;     // bytes per row (no padding)
  static constexpr int BYTES = BQ * PITCH;
  static constexpr int INST = BYTES / 1024;  // 64-lane DMA instructions per tile
  static constexpr int PER_WAVE = INST / 4;
  static_assert(INST % 4 == 0, "tile DMA splits evenly over 4 waves");
  // Chunk permutation of row r (depends on r mod 16 only).
  //  D = 128 (one row spans all 64 banks): bits 0-1 of r go to bits 2-3 of
  //   the chunk, bits 2-3 of r to bits 0-1.  16 consecutive rows: 16
  //   distinct chunks.  4 consecutive rows (r mod 4 = 0..3): 4 distinct
  //   4-chunk groups.
  //  D = 64 (two rows per 64 banks, bit 0 of r picks the half): bit 1 of r
  //   goes to bit 2 of the chunk, bits 2-3 of r to bits 0-1.
  __device__ static int swz(int r) {
    if constexpr (D == 128)
      return ((r & 3) << 2) | ((r >> 2) & 3);
    else
      return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
};

// A wave-uniform pointer, made visibly uniform (an SGPR pair) for the DMA's
// scalar base operand: some kernels' uniformity analysis leaves such a
// pointer in VGPRs.  No code when it already is in SGPRs.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

// DMA of one 64-row tile (row 0 at `src`) into swizzled LDS.  Rows at or
// past rows_left (>= 1) fetch row rows_left - 1 instead (in bounds; their
// results are discarded or zero-weighted).  `src` must be wave-uniform.
template <int D>
__device__ __forceinline__ void dma_swz_tile(const char* src_any, char* dst, int w, int lane, int rows_left) {
  using T = SwzTile<D>;
  const char* src = uniform_ptr(src_any);
#pragma unroll
  for (int i = 0; i < T::PER_WAVE; ++i) {
    const int inst = w * T::PER_WAVE + i;
    const int slot = inst * 64 + lane;
    const int row = slot / T::CPR, pc = slot % T::CPR;
    const int r = row < rows_left ? row : rows_left - 1;
    const unsigned off = (unsigned)r * (D * 2) + 16u * (unsigned)(pc ^ T::swz(row));
    dma_run<1>(src, &off, lds_addr(dst + inst * 1024));
  }
}

__device__ __forceinline__ void land_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Bit-permuted row read by lane n for products over D: bits 2 and 3 of n
// swapped, so that accumulator register r of the 32 x 32 result holds row
// 16 (r / 8) + 8 h + r % 8 -- the rows of the next product's k-steps.
__device__ __forceinline__ int perm_row(int n) { return (n & 0x13) | ((n & 4) << 1) | ((n & 8) >> 1); }

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled.
template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

}  // namespace st
}  // namespace attn
