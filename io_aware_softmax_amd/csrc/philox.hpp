// Philox4x32-10 counter-based generator on the device (Salmon, Moraes, Dror,
// Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011, section 3.2
// and table 2) and the dropout keep rule built on it.
//
// One round multiplies counter words 0 and 2 by M0 and M1 (full 64-bit
// products), then outputs (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1,
// lo(M0 x0)); the key is bumped by the Weyl constants between rounds.
//
// Dropout: the weight of (batch-head bh, query i, key j) is kept iff word
// (j mod 4) of Philox4x32-10(counter = (j / 4, i, bh, offset),
// key = (seed low, seed high)) is >= the threshold floor(p 2^32).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace attn {

struct PhiloxKey {
  unsigned k0, k1;
};

__device__ __forceinline__ uint4 philox4x32_10(uint4 x, PhiloxKey key) {
  constexpr unsigned M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr unsigned W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  unsigned k0 = key.k0, k1 = key.k1;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    // Full 64-bit products: one v_mad_u64_u32 each instead of a
    // v_mul_hi_u32 / v_mul_lo_u32 pair; each three-way XOR is one
    // v_bitop3_b32 (truth table 0x96) instead of two v_xor_b32.
    const uint64_t p0 = (uint64_t)M0 * x.x;
    const uint64_t p1 = (uint64_t)M1 * x.z;
    x = make_uint4(__builtin_amdgcn_bitop3_b32((unsigned)(p1 >> 32), x.y, k0, 0x96), (unsigned)p1,
                   __builtin_amdgcn_bitop3_b32((unsigned)(p0 >> 32), x.w, k1, 0x96), (unsigned)p0);
  }
  return x;
}

// Keep bits of keys j0 .. j0 + 7 (j0 a multiple of 8) for query i: bit e is
// key j0 + e.
__device__ __forceinline__ unsigned dropout_keep8(PhiloxKey key, unsigned j0, unsigned i, unsigned bh,
                                                  unsigned offset, unsigned thr) {
  const uint4 a = philox4x32_10(make_uint4(j0 >> 2, i, bh, offset), key);
  const uint4 b = philox4x32_10(make_uint4((j0 >> 2) + 1, i, bh, offset), key);
  return (a.x >= thr ? 1u : 0u) | (a.y >= thr ? 2u : 0u) | (a.z >= thr ? 4u : 0u) | (a.w >= thr ? 8u : 0u) |
         (b.x >= thr ? 16u : 0u) | (b.y >= thr ? 32u : 0u) | (b.z >= thr ? 64u : 0u) | (b.w >= thr ? 128u : 0u);
}

// Keep bit of one (query i, key j).
__device__ __forceinline__ bool dropout_keep1(PhiloxKey key, unsigned j, unsigned i, unsigned bh, unsigned offset,
                                              unsigned thr) {
  const uint4 a = philox4x32_10(make_uint4(j >> 2, i, bh, offset), key);
  const unsigned w = (j & 2) ? ((j & 1) ? a.w : a.z) : ((j & 1) ? a.y : a.x);
  return w >= thr;
}

}  // namespace attn
