// Philox4x32-10 counter-based generator on the device (Salmon, Moraes, Dror,
// Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011, section 3.2
// and table 2) and the dropout keep rule built on it.
//
// One round multiplies counter words 0 and 2 by M0 and M1 (full 64-bit
// products), then outputs (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1,
// lo(M0 x0)); the key is bumped by the Weyl constants between rounds.
//
// Dropout: the weight of (batch-head bh, query i, key j) is kept iff the
// 16-bit half (j mod 2; 0 the low half) of word ((j mod 8) / 2) of
// Philox4x32-10(counter = (j / 8, i, bh, offset), key = (seed low, seed
// high)) is >= floor(p 2^16).  One block serves 8 consecutive keys.  The
// threshold travels shifted: thr = floor(p 2^16) << 16, so a high half is
// kept iff word >= thr and a low half iff (word << 16) >= thr.
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

// Keep bits of the 8 keys of one block: bit e is key 8 (block) + e.
__device__ __forceinline__ unsigned keep_bits8(uint4 a, unsigned thr) {
  return ((a.x << 16) >= thr ? 1u : 0u) | (a.x >= thr ? 2u : 0u) | ((a.y << 16) >= thr ? 4u : 0u) |
         (a.y >= thr ? 8u : 0u) | ((a.z << 16) >= thr ? 16u : 0u) | (a.z >= thr ? 32u : 0u) |
         ((a.w << 16) >= thr ? 64u : 0u) | (a.w >= thr ? 128u : 0u);
}

// Keep bits of keys j0 .. j0 + 7 (j0 a multiple of 8) for query i: bit e is
// key j0 + e.
__device__ __forceinline__ unsigned dropout_keep8(PhiloxKey key, unsigned j0, unsigned i, unsigned bh,
                                                  unsigned offset, unsigned thr) {
  return keep_bits8(philox4x32_10(make_uint4(j0 >> 3, i, bh, offset), key), thr);
}

}  // namespace attn
