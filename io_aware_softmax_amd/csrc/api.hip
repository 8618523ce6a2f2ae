// C ABI of the attention forward and backward: argument validation, kernel
// dispatch and the stream-ordered workspaces.  Declarations and the
// contract are in include/attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_internal.hpp"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_hip_msg[192] = "";
thread_local char g_status_msg[256] = "";

int hip_fail(hipError_t e) {
  std::snprintf(g_hip_msg, sizeof(g_hip_msg), "%s (%s)", hipGetErrorString(e), hipGetErrorName(e));
  return ATTN_ERR_HIP;
}

size_t elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Launch-size limit: grid size times block size must fit 32 bits.
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 24) - 1;

// Everything that does not need the device; returns ATTN_OK or an error.
int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
             int H, int Lq, int Lk, int D, int causal, float scale, int dtype) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || D <= 0) return ATTN_ERR_DIM;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED_D;
  const int64_t BH = int64_t(B) * H;
  if (BH > INT32_MAX || int64_t(Lq) * D > INT32_MAX || int64_t(Lk) * D > INT32_MAX)
    return ATTN_ERR_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (causal && Lq > Lk) return ATTN_ERR_CAUSAL_SHAPE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if ((mis & 15u) || (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
  const size_t es = elem_bytes(dtype);
  const size_t nq = size_t(BH) * Lq * D * es, nk = size_t(BH) * Lk * D * es;
  const size_t nl = size_t(BH) * Lq * sizeof(float);
  if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nk) || overlaps(o, nq, v, nk) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nk) ||
      overlaps(o, nq, lse, nl))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

// ATTN_PREFILL_KERNEL=single forces the single-group 16-bit prefill kernel
// everywhere, =two the two-group kernel also at D = 64 (tests compare the
// kernels); read on every call.  0: the library's choice.
int prefill_variant() {
  const char* e = std::getenv("ATTN_PREFILL_KERNEL");
  if (e == nullptr) return 0;
  if (std::strcmp(e, "single") == 0) return 1;
  if (std::strcmp(e, "two") == 0) return 2;
  return 0;
}

// Key ranges of the two-group prefill: ATTN_PREFILL_SPLITS=n forces n per
// query tile (1 = never split; capped so that no range is empty), else the
// library plans them from the shape and the device's compute-unit count.
hipError_t prefill_split_plan(int BH, int Lq, int Lk, bool causal, attn::PrefillSplitPlan* plan, bool* split) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const char* env = std::getenv("ATTN_PREFILL_SPLITS");
  const int forced = (env != nullptr && *env != '\0') ? std::max(1, std::atoi(env)) : 0;
  *split = attn::prefill_pp_plan_splits(BH, Lq, Lk, causal, cus, forced, plan);
  return hipSuccess;
}

int auto_splits(int64_t BH, int Lk) {
  // Aim for about 16 workgroups per CU of the 256-CU part, but keep at least
  // 256 keys per range so the per-range epilogue stays negligible.
  const int64_t target = 4096;
  int64_t s = (target + BH - 1) / BH;
  const int64_t by_len = (int64_t(Lk) + 255) / 256;
  if (s > by_len) s = by_len;
  if (s > ATTN_MAX_SPLITS) s = ATTN_MAX_SPLITS;
  if (s < 1) s = 1;
  return int(s);
}

// Bytes of split partials a decode call needs: [BH * splits] rows of D
// floats (the normalised partial outputs), then the maxima and the sums.
size_t decode_workspace_bytes(int64_t BH, int splits, int D) {
  return size_t(BH) * splits * (size_t(D) + 2) * sizeof(float);
}

// The decode kernels on a given workspace of decode_workspace_bytes().
hipError_t launch_decode_on(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                            int H, int Lk, int D, float scale, int splits, hipStream_t stream, int dtype,
                            const int* seqlens, void* ws) {
  const size_t nparts = size_t(BH) * splits;
  attn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.part_o = static_cast<float*>(ws);
  a.part_m = a.part_o + nparts * D;
  a.part_l = a.part_m + nparts;
  a.BH = int(BH);
  a.H = H;
  a.Lk = Lk;
  a.seqlens = seqlens;
  a.splits = splits;
  a.keys_per_split = int((int64_t(Lk) + splits - 1) / splits);
  a.c = std::fabs(scale) * attn::kLog2e;
  a.neg = scale < 0.f;
  return attn::launch_decode(dtype, D, a, stream);
}

int run_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Lk, int D, float scale, int splits, hipStream_t stream, int dtype,
               const int* seqlens = nullptr) {
  const int64_t BH = int64_t(B) * H;
  if (splits == 0) splits = auto_splits(BH, Lk);
  if (BH * splits > kMaxWorkgroups) return ATTN_ERR_DIM;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, decode_workspace_bytes(BH, splits, D), stream);
  if (e != hipSuccess) return hip_fail(e);
  e = launch_decode_on(q, k, v, o, lse, BH, H, Lk, D, scale, splits, stream, dtype, seqlens, ws);
  const hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return ATTN_OK;
}

// Scratch of attn_decode_fwd_noalloc: the split partials live in this
// fixed device array instead of a stream-ordered allocation.  Every device
// the library runs on holds its own copy until the process ends.  In host
// code the array's name is only a host-side stand-in: its device address
// comes from hipGetSymbolAddress, once per device, with that device
// current, and only that address is passed to kernels.
__device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the
// first call per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

// Checks and packs the mask / dropout arguments shared by attn_fwd_ex and
// attn_bwd_ex.  `outs` / `out_n`: the call's output buffers, which must not
// overlap the mask.
int make_mask_dropout(const void* mask, int mask_kind, int mask_b, int mask_h, float dropout_p,
                      unsigned long long seed, unsigned offset, int B, int H, int Lq, int Lk,
                      const void* const* outs, const size_t* out_n, int n_outs, attn::MaskDropout* md) {
  if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_BOOL && mask_kind != ATTN_MASK_ADD)
    return ATTN_ERR_MASK;
  if (!(dropout_p >= 0.f && dropout_p < 1.f)) return ATTN_ERR_DROPOUT;  // also rejects NaN
  md->mask = nullptr;
  md->kind = mask_kind;
  md->mask_b = md->mask_h = 1;
  md->H = H;
  if (mask_kind != ATTN_MASK_NONE) {
    if (mask == nullptr) return ATTN_ERR_NULL;
    if ((mask_b != 1 && mask_b != B) || (mask_h != 1 && mask_h != H)) return ATTN_ERR_MASK;
    if (reinterpret_cast<uintptr_t>(mask) & 15u) return ATTN_ERR_ALIGN;
    const size_t nm = size_t(mask_b) * mask_h * Lq * Lk * (mask_kind == ATTN_MASK_BOOL ? 1 : 4);
    for (int i = 0; i < n_outs; ++i)
      if (overlaps(outs[i], out_n[i], mask, nm)) return ATTN_ERR_ALIAS;
    md->mask = mask;
    md->mask_b = mask_b;
    md->mask_h = mask_h;
  }
  md->dropout = dropout_p > 0.f;
  const double thr = std::floor(double(dropout_p) * 65536.0);
  md->thr = (thr >= 65535.0 ? 0xFFFFu : unsigned(thr)) << 16;
  md->rp = float(1.0 / (1.0 - double(dropout_p)));
  md->k0 = unsigned(seed & 0xFFFFFFFFull);
  md->k1 = unsigned(seed >> 32);
  md->offset = offset;
  return ATTN_OK;
}

// The backward behind attn_bwd and attn_bwd_ex (md: mask / dropout or NULL).
int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
            void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int D, int causal, float scale,
            hipStream_t s, int dtype, const attn::MaskDropout* md) {
  if (!dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  // The forward's checks cover q, k, v, o, lse, the sizes, scale and causal.
  int st = validate(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_F32) return ATTN_ERR_DTYPE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                        reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if (mis & 15u) return ATTN_ERR_ALIGN;
  const int64_t BH = int64_t(B) * H;
  const size_t es = elem_bytes(dtype);
  const size_t nq = size_t(BH) * Lq * D * es, nk = size_t(BH) * Lk * D * es;
  const size_t nl = size_t(BH) * Lq * sizeof(float);
  // Outputs must not overlap any input or each other.
  const void* in[6] = {q, k, v, o, dout, lse};
  const size_t in_n[6] = {nq, nk, nk, nq, nq, nl};
  void* out[3] = {dq, dk, dv};
  const size_t out_n[3] = {nq, nk, nk};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], out_n[i], in[j], in_n[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(out[i], out_n[i], out[j], out_n[j])) return ATTN_ERR_ALIAS;
  }
  if (BH * ((int64_t(Lk) + 127) / 128) > kMaxWorkgroups || BH * ((int64_t(Lq) + 63) / 64) > kMaxWorkgroups)
    return ATTN_ERR_DIM;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, attn::bwd_workspace_bytes(int(BH), Lq), s);
  if (e != hipSuccess) return hip_fail(e);
  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.stats = static_cast<float*>(ws);
  a.BH = int(BH);
  a.Lq = Lq;
  a.Lk = Lk;
  a.c = scale * attn::kLog2e;
  a.scale = scale;
  e = attn::launch_bwd(dtype, D, causal != 0, a, s, md);
  const hipError_t ef = hipFreeAsync(ws, s);
  if (e != hipSuccess) return hip_fail(e);
  if (ef != hipSuccess) return hip_fail(ef);
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Lq, int Lk, int D, int causal, float scale, void* stream,
                         int dtype) {
  const int st = validate(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Lq == 1) return run_decode(q, k, v, o, lse, B, H, Lk, D, scale, 0, s, dtype);
  attn::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.Lq = Lq;
  a.Lk = Lk;
  a.c = std::fabs(scale) * attn::kLog2e;
  a.neg = scale < 0.f;
  const int64_t nqt = (int64_t(Lq) + 127) / 128;
  if (int64_t(a.BH) * nqt > kMaxWorkgroups) return ATTN_ERR_DIM;
  // 16-bit inputs at D = 128 with a nonzero scale take the two-group kernel;
  // D = 64 (softmax-bound: half the products per score) and scale 0 (whose
  // masked keys need explicit zero weights) take the single-group kernel.
  hipError_t e;
  if (dtype == ATTN_F32) {
    e = attn::launch_prefill_f32(D, causal != 0, a, s);
  } else if (D == 64 && a.c > 0.f && prefill_variant() == 2) {
    e = attn::launch_prefill_pp(dtype, 64, causal != 0, a, s);
  } else if (D == 128 && a.c > 0.f && prefill_variant() != 1) {
    // Shapes with fewer query tiles than the part has compute units (one
    // head, short chunks) cut each tile's keys into ranges, merged after.
    attn::PrefillSplitPlan plan;
    bool split = false;
    e = prefill_split_plan(a.BH, Lq, Lk, causal != 0, &plan, &split);
    if (e != hipSuccess) return hip_fail(e);
    if (split) {
      const size_t rows = size_t(a.BH) * Lq;
      const size_t ranges = size_t(plan.max_ranges);
      const size_t bytes = ranges * rows * (size_t(D) + 1) * sizeof(float);
      void* ws = nullptr;
      e = hipMallocAsync(&ws, bytes, s);
      if (e != hipSuccess) return hip_fail(e);
      float* part_o = static_cast<float*>(ws);
      e = attn::launch_prefill_pp_split(dtype, causal != 0, a, plan, part_o, part_o + ranges * rows * D, s);
      const hipError_t ef = hipFreeAsync(ws, s);
      if (e == hipSuccess) e = ef;
    } else {
      e = attn::launch_prefill_pp(dtype, 128, causal != 0, a, s);
    }
  } else {
    e = attn::launch_prefill_mfma(dtype, D, causal != 0, a, s);
  }
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

ATTN_EXPORT int attn_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Lk, int D, float scale, int num_splits,
                                void* stream, int dtype) {
  const int st = validate(q, k, v, o, lse, B, H, 1, Lk, D, 0, scale, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  return run_decode(q, k, v, o, lse, B, H, Lk, D, scale, num_splits, static_cast<hipStream_t>(stream),
                    dtype);
}

ATTN_EXPORT int attn_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                        int B, int H, int Lk, int D, float scale, int num_splits,
                                        void* stream, int dtype) {
  const int st = validate(q, k, v, o, lse, B, H, 1, Lk, D, 0, scale, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  const int64_t BH = int64_t(B) * H;
  const int splits = num_splits == 0 ? auto_splits(BH, Lk) : num_splits;
  if (BH * splits > kMaxWorkgroups) return ATTN_ERR_DIM;
  if (decode_workspace_bytes(BH, splits, D) > size_t(ATTN_NOALLOC_SCRATCH_BYTES)) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  e = launch_decode_on(q, k, v, o, lse, BH, H, Lk, D, scale, splits, static_cast<hipStream_t>(stream), dtype,
                       nullptr, ws);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

ATTN_EXPORT int attn_decode_varlen_fwd(const void* q, const void* k, const void* v, void* o,
                                       float* lse, const int* seqlens, int B, int H, int Lk_max,
                                       int D, float scale, int num_splits, void* stream,
                                       int dtype) {
  if (seqlens == nullptr) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(seqlens) & 3u) return ATTN_ERR_ALIGN;
  const int st = validate(q, k, v, o, lse, B, H, 1, Lk_max, D, 0, scale, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SPLITS;
  const size_t no = size_t(B) * H * D * elem_bytes(dtype), nl = size_t(B) * H * sizeof(float);
  if (overlaps(o, no, seqlens, size_t(B) * sizeof(int)) || overlaps(lse, nl, seqlens, size_t(B) * sizeof(int)))
    return ATTN_ERR_ALIAS;
  return run_decode(q, k, v, o, lse, B, H, Lk_max, D, scale, num_splits,
                    static_cast<hipStream_t>(stream), dtype, seqlens);
}

ATTN_EXPORT int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk,
                         int D, int causal, float scale, void* stream, int dtype) {
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Lq, Lk, D, causal, scale,
                 static_cast<hipStream_t>(stream), dtype, nullptr);
}

ATTN_EXPORT int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int H, int Lq, int Lk, int D, int causal, float scale, const void* mask,
                            int mask_kind, int mask_b, int mask_h, float dropout_p,
                            unsigned long long seed, unsigned offset, void* stream, int dtype) {
  const int st = validate(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_F32) return ATTN_ERR_DTYPE;
  const size_t es = elem_bytes(dtype);
  const void* outs[2] = {o, lse};
  const size_t out_n[2] = {size_t(B) * H * Lq * D * es, size_t(B) * H * Lq * sizeof(float)};
  attn::MaskDropout md;
  const int sm = make_mask_dropout(mask, mask_kind, mask_b, mask_h, dropout_p, seed, offset, B, H, Lq, Lk,
                                   outs, out_n, 2, &md);
  if (sm != ATTN_OK) return sm;
  if (mask_kind == ATTN_MASK_NONE && !md.dropout)
    return attn_fwd(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, stream, dtype);
  if (int64_t(B) * H * ((int64_t(Lq) + 127) / 128) > kMaxWorkgroups) return ATTN_ERR_DIM;
  attn::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.Lq = Lq;
  a.Lk = Lk;
  a.c = std::fabs(scale) * attn::kLog2e;
  a.neg = scale < 0.f;
  const hipError_t e = attn::launch_prefill_ex(dtype, D, causal != 0, a, md, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

ATTN_EXPORT int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk,
                            int D, int causal, float scale, const void* mask, int mask_kind, int mask_b,
                            int mask_h, float dropout_p, unsigned long long seed, unsigned offset,
                            void* stream, int dtype) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  // Sizes first (the mask's extent below needs them valid).
  int st = validate(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  const size_t es = elem_bytes(dtype);
  const void* outs[3] = {dq, dk, dv};
  const size_t out_n[3] = {size_t(B) * H * Lq * D * es, size_t(B) * H * Lk * D * es,
                           size_t(B) * H * Lk * D * es};
  attn::MaskDropout md;
  st = make_mask_dropout(mask, mask_kind, mask_b, mask_h, dropout_p, seed, offset, B, H, Lq, Lk, outs, out_n, 3,
                         &md);
  if (st != ATTN_OK) return st;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Lq, Lk, D, causal, scale,
                 static_cast<hipStream_t>(stream), dtype, &md);
}

ATTN_EXPORT int attn_decode_auto_splits(int B, int H, int Lk, int D) {
  if (B <= 0 || H <= 0 || Lk <= 0 || D <= 0) return ATTN_ERR_DIM;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED_D;
  if (int64_t(B) * H > INT32_MAX) return ATTN_ERR_DIM;
  return auto_splits(int64_t(B) * H, Lk);
}

ATTN_EXPORT int attn_prefill_split_plan(int B, int H, int Lq, int Lk, int causal, int num_cus, int forced,
                                        int* ranges, int* items) {
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || num_cus <= 0 || forced < 0) return ATTN_ERR_DIM;
  if (ranges == nullptr || items == nullptr) return ATTN_ERR_NULL;
  if (int64_t(B) * H > INT32_MAX) return ATTN_ERR_DIM;
  const int nqt = (Lq + 255) / 256;
  attn::PrefillSplitPlan plan;
  if (attn::prefill_pp_plan_splits(B * H, Lq, Lk, causal != 0, num_cus, forced, &plan)) {
    for (int qt = 0; qt < nqt; ++qt) ranges[qt] = plan.ranges[qt];
    *items = plan.items;
  } else {
    for (int qt = 0; qt < nqt; ++qt) ranges[qt] = 1;
    *items = nqt;
  }
  return ATTN_OK;
}

ATTN_EXPORT const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_DIM: return "a dimension is <= 0 or a size exceeds the index range";
    case ATTN_ERR_UNSUPPORTED_D: return "head dimension must be 64 or 128";
    case ATTN_ERR_DTYPE: return "unsupported dtype (ATTN_F32, ATTN_F16 or ATTN_BF16; attn_bwd: ATTN_F16 or ATTN_BF16)";
    case ATTN_ERR_SCALE: return "scale is NaN or infinite";
    case ATTN_ERR_CAUSAL_SHAPE: return "causal attention requires Lq <= Lk";
    case ATTN_ERR_SPLITS: return "num_splits must be in [0, ATTN_MAX_SPLITS]";
    case ATTN_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case ATTN_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_MASK: return "mask_kind is not an attn_mask_kind_t, or mask_b / mask_h is not 1 or B / H";
    case ATTN_ERR_DROPOUT: return "dropout_p must be in [0, 1)";
    case ATTN_ERR_WORKSPACE:
      return "the call needs more than ATTN_NOALLOC_SCRATCH_BYTES of split partials (fewer splits or a smaller batch)";
    case ATTN_ERR_HIP:
      std::snprintf(g_status_msg, sizeof(g_status_msg), "HIP error: %s", g_hip_msg);
      return g_status_msg;
    default: return "unknown status";
  }
}
