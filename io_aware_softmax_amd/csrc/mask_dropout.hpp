// Reading a general attention mask and drawing dropout keep bits inside the
// fused tile (the comfyai.app chapter "6.3 FlashAttention", section 6.3.3,
// "Kernel Fusion": scores, scale, mask, softmax, dropout and the value
// product in one kernel).  The mask kind is a template argument: each kernel
// is instantiated once per (mask kind, dropout), so a variant does only its
// own per-element work.
#pragma once

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "attn_internal.hpp"
#include "philox.hpp"

namespace attn {

// Element offset of the (b, h) slab of a [mask_b, mask_h, Lq, Lk] mask
// (axes of size 1 broadcast).
__device__ __forceinline__ size_t mask_slab(const MaskDropout& md, int bh, int Lq, int Lk) {
  const int b = bh / md.H, h = bh % md.H;
  const int slab = (md.mask_b == 1 ? 0 : b) * md.mask_h + (md.mask_h == 1 ? 0 : h);
  return (size_t)slab * Lq * Lk;
}

// Terms of keys j0 .. j0 + 7 of one query row (idx = slab + i Lk + j0) for a
// mask of kind KIND (0 none, 1 boolean, 2 additive), in base-2 units and
// shifted by `off` (a kept key gets off, an additive term off + log2(e) m);
// keys at or past Lk get -inf.  `vec` (wave-uniform: Lk % 8 == 0 and all 8 keys before Lk) selects
// one 8-byte (boolean) or two 16-byte (additive) loads; otherwise 8 element
// loads, each from an index clamped into the row so that no load depends on
// a lane condition.
template <int KIND>
__device__ __forceinline__ void mask_terms8_kind(const MaskDropout& md, size_t idx, int j0, int Lk, bool vec,
                                                 float (&t)[8], float off = 0.f) {
  if constexpr (KIND == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = j0 + e < Lk ? off : -INFINITY;
    return;
  } else {
    if (vec) {
      if constexpr (KIND == 1) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const unsigned char*>(md.mask) + idx);
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (((e < 4 ? u.x : u.y) >> (8 * (e & 3))) & 0xffu) ? off : -INFINITY;
      } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(md.mask) + idx);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(md.mask) + idx + 4);
        t[0] = __builtin_fmaf(a.x, kLog2e, off); t[1] = __builtin_fmaf(a.y, kLog2e, off);
        t[2] = __builtin_fmaf(a.z, kLog2e, off); t[3] = __builtin_fmaf(a.w, kLog2e, off);
        t[4] = __builtin_fmaf(b.x, kLog2e, off); t[5] = __builtin_fmaf(b.y, kLog2e, off);
        t[6] = __builtin_fmaf(b.z, kLog2e, off); t[7] = __builtin_fmaf(b.w, kLog2e, off);
      }
      return;
    }
    size_t ie[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ie[e] = j0 + e < Lk ? idx + e : idx - j0;  // key 0 of the row: in bounds
    if constexpr (KIND == 1) {
      const unsigned char* m8 = static_cast<const unsigned char*>(md.mask);
      unsigned char v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = m8[ie[e]];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = (j0 + e < Lk && v[e] != 0) ? off : -INFINITY;
    } else {
      const float* m32 = static_cast<const float*>(md.mask);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = m32[ie[e]];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = j0 + e < Lk ? __builtin_fmaf(v[e], kLog2e, off) : -INFINITY;
    }
  }
}

}  // namespace attn
