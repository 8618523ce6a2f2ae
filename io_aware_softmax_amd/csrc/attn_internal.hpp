// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace attn {

// log2(e): scores are moved to base 2 so that exp becomes one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;        // B * H
  int Lq;
  int Lk;
  float c;       // |scale| * log2(e)
  bool neg;      // scale < 0: q is negated on load (exact)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* part_o;  // [BH, splits, D] normalised partial outputs
  float* part_m;  // [BH, splits] partial maxima, base-2 scaled-score units
  float* part_l;  // [BH, splits] partial denominators
  int BH;
  int H;
  int Lk;              // keys per (b, h) in memory (the row stride of k and v)
  const int* seqlens;  // device [B] lengths (clamped to [0, Lk]) or nullptr: all Lk
  int splits;
  int keys_per_split;  // used when seqlens == nullptr
  float c;
  bool neg;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* stats;  // workspace: per 64-query tile, lse * log2(e) [64] then Dv [64]
  int BH;
  int Lq;
  int Lk;
  float c;       // scale * log2(e) (signed)
  float scale;
};

// General mask and dropout of the fused tile (forward and backward).
struct MaskDropout {
  const void* mask;  // [mask_b, mask_h, Lq, Lk] uint8 (kind 1) or float32 (kind 2); nullptr for kind 0
  int kind;          // 0 none, 1 boolean (nonzero = attend), 2 additive (float32, -inf = excluded)
  int mask_b;        // 1 (broadcast over batch) or B
  int mask_h;        // 1 (broadcast over heads) or H
  int H;             // heads: bh = b * H + h
  bool dropout;      // p > 0
  unsigned thr;      // floor(p 2^16) << 16: a 16-bit Philox half h is kept iff (h << 16) >= thr
  float rp;          // 1 / (1 - p)
  unsigned k0, k1;   // Philox key: the seed's low and high words
  unsigned offset;   // Philox counter word 3
};

// Workgroups of `kernel` (block threads, static LDS only) that device `dev`
// holds resident at once: compute units times workgroups per unit.  Cached.
hipError_t resident_workgroups(int dev, const void* kernel, int block, int* out);

// Tiled one-pass prefill on MFMA for 16-bit inputs (dtype 1 = f16, 2 = bf16).
hipError_t launch_prefill_mfma(int dtype, int D, bool causal, const PrefillArgs& a, hipStream_t s);
// Two-group (ping-pong) variant of the 16-bit prefill, D = 64 or 128.
hipError_t launch_prefill_pp(int dtype, int D, bool causal, const PrefillArgs& a, hipStream_t s);
// Key ranges of a split prefill: query tile qt (256 rows) of every
// (batch, head) has ranges[qt] contiguous, balanced, non-empty ranges of its
// 64-key tiles; item[t] = (qt << 5) | range lists the `items` ranges of one
// (batch, head), heaviest tiles first.  Passed by value to the kernels.
constexpr int kSplitMaxItems = 256;
constexpr int kSplitMaxTiles = 128;
constexpr int kSplitMaxRanges = 32;
struct PrefillSplitPlan {
  int items;       // ranges per (batch, head)
  int max_ranges;  // largest ranges[qt]: the partial buffers' leading extent
  unsigned short item[kSplitMaxItems];
  unsigned char ranges[kSplitMaxTiles];
};
// The same (D = 128) with the keys of every query tile cut as `plan` says (partials in
// part_o [max_ranges, BH, Lq, 128] and part_l [max_ranges, BH, Lq] fp32),
// then merged.
hipError_t launch_prefill_pp_split(int dtype, bool causal, const PrefillArgs& a, const PrefillSplitPlan& plan,
                                   float* part_o, float* part_l, hipStream_t s);
// Plans the split on a part with `cus` compute units; false: do not split.
// Automatic (forced == 0): only shapes with at most cus / 2 query tiles; the
// ranges hold about R key tiles each, R the smallest value (>= 8) for which
// one range per workgroup covers the shape.  forced > 0: that many ranges
// for every tile, capped at 16 and so that no range is empty.
bool prefill_pp_plan_splits(int BH, int Lq, int Lk, bool causal, int cus, int forced, PrefillSplitPlan* plan);
// The same algorithm with fp32 inputs on the fp32 MFMA.
hipError_t launch_prefill_f32(int D, bool causal, const PrefillArgs& a, hipStream_t s);
// Forward with a general mask and / or dropout (16-bit dtypes).
hipError_t launch_prefill_ex(int dtype, int D, bool causal, const PrefillArgs& a, const MaskDropout& md,
                             hipStream_t s);
// Attention backward (16-bit dtypes): stats, dK/dV and dQ kernels on stream s;
// md == nullptr: no mask and no dropout.
hipError_t launch_bwd(int dtype, int D, bool causal, const BwdArgs& a, hipStream_t s,
                      const MaskDropout* md = nullptr);
// Bytes of BwdArgs::stats for B * H = BH and Lq queries.
size_t bwd_workspace_bytes(int BH, int Lq);
// Split-KV decode: partials then combine, both on stream s.
hipError_t launch_decode(int dtype, int D, const DecodeArgs& a, hipStream_t s);

}  // namespace attn
