// Measurement probes for the costs the attention kernels are designed
// around on gfx950 (not part of the library): per-wave issue cost of the
// softmax's VALU instructions and of one 32x32x16 bf16 MFMA, how much a
// stream of MFMAs on one wave slows a VALU stream on the other wave of the
// same SIMD, per-wave LDS read throughput for the two read forms the
// kernels use (ds_read_b128 and ds_read_b64_tr_b16), and the HBM read rate
// of a plain stream of 16-byte loads, ordinary and nontemporal.
//
// Every workgroup reserves 96 KB of LDS, so at most one runs per compute
// unit; the grid is 256 workgroups.  Each wave times its own loop with
// s_memtime (shader clock) and s_memrealtime (100 MHz) and writes the two
// 64-bit counts to out[block, wave, 0..1]; the host prints the mean cycles
// per instruction (or per read), the shader clock they imply and the
// launch's event time.  Nothing else is written: results feed an empty asm,
// and the only other store sits behind a condition the data never meets.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGrid = 256;
constexpr int kIter = 512;
constexpr int kLdsBytes = 96 * 1024;

enum Stream { kExp, kFma, kAdd, kCvt, kMax3, kMfma, kSoftmaxMix, kLdsB128, kLdsTr };

// 64 instructions per call, 8 independent chains.
__device__ __forceinline__ void exp64(float (&x)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("v_exp_f32 %0, %0" : "+v"(x[c]));
}
__device__ __forceinline__ void fma64(float (&x)[8], float a, float b) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[c]) : "v"(a), "v"(b));
}
__device__ __forceinline__ void add64(float (&x)[8], float a) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("v_add_f32 %0, %0, %1" : "+v"(x[c]) : "v"(a));
}
__device__ __forceinline__ void cvt64(float (&x)[8], unsigned (&p)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(p[c]) : "v"(x[c]), "v"(x[(c + 1) & 7]));
}
__device__ __forceinline__ void max64(float (&x)[8], float a, float b) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x[c]) : "v"(a), "v"(b));
}

// One softmax tile of one lane as the two-group kernel runs it at D = 128:
// 32 x (fma, exp, add) and 16 packs = 112 instructions.
__device__ __forceinline__ void softmax_mix(float (&x)[8], float (&s)[2], unsigned (&p)[8], float a, float b) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float t;
      asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(t) : "v"(x[c]), "v"(a), "v"(b));
      asm volatile("v_exp_f32 %0, %0" : "+v"(t));
      asm volatile("v_add_f32 %0, %0, %1" : "+v"(s[c & 1]) : "v"(t));
      x[c] = t;
    }
#pragma unroll
    for (int c = 0; c < 8; c += 2) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(p[c]) : "v"(x[c]), "v"(x[c + 1]));
  }
}

// 16 MFMAs on 4 independent accumulators.
__device__ __forceinline__ void mfma16(f32x16 (&acc)[4], bf16x8 a, bf16x8 b) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
}

// 16 distinct reads in flight per round: b128 over a 16 KB window (one per
// pair of waves), transposed b64 over an 8 KB window per wave.  16 lanes x
// 16 B (or 8 lanes x 8 B) cover all banks once: conflict free.
__device__ __forceinline__ void lds_b128(const char* lds, int base, int lane) {
  u32x4 r[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] = *reinterpret_cast<const u32x4*>(lds + base + j * 1024 + 16 * lane);
  asm volatile("" ::"v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]), "v"(r[4]), "v"(r[5]), "v"(r[6]), "v"(r[7]),
               "v"(r[8]), "v"(r[9]), "v"(r[10]), "v"(r[11]), "v"(r[12]), "v"(r[13]), "v"(r[14]), "v"(r[15]));
}
__device__ __forceinline__ void lds_tr(char* lds, int base, int lane) {
  s16x4 r[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    r[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(lds + base + j * 512 + 8 * lane));
  asm volatile("" ::"v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]), "v"(r[4]), "v"(r[5]), "v"(r[6]), "v"(r[7]),
               "v"(r[8]), "v"(r[9]), "v"(r[10]), "v"(r[11]), "v"(r[12]), "v"(r[13]), "v"(r[14]), "v"(r[15]));
}

// Waves below `split` run stream A, the others stream B.
template <int A, int B>
__global__ __launch_bounds__(512) void probe(unsigned long long* out, float* sink, int split) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nw = blockDim.x >> 6;
  for (int i = tid; i < kLdsBytes / 16; i += blockDim.x) reinterpret_cast<u32x4*>(lds)[i] = u32x4{unsigned(i), 1u, 2u, 3u};
  __syncthreads();
  const int mode = w < split ? A : B;
  float x[8], s[2] = {0.f, 0.f};
  unsigned p[8] = {};
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = -1.0f - 0.01f * c - 1e-6f * lane;
  const float a = 0.5f, b = -0.25f;
  f32x16 acc[4] = {};
  bf16x8 fa, fb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    fa[e] = __bf16(0.001f * (lane + e));
    fb[e] = __bf16(0.002f * (lane - e));
  }
  // Read windows inside the first 64 KB: [16 KB * (w & 3), + 16 KB) for b128,
  // [8 KB * (w & 7), + 8 KB) for the transposed reads.
  const int base = mode == kLdsB128 ? (w & 3) * 16384 : (w & 7) * 8192;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < kIter; ++it) {
    switch (mode) {
      case kExp: exp64(x); break;
      case kFma: fma64(x, a, b); break;
      case kAdd: add64(x, a); break;
      case kCvt: cvt64(x, p); break;
      case kMax3: max64(x, a, b); break;
      case kMfma: mfma16(acc, fa, fb); break;
      case kSoftmaxMix: softmax_mix(x, s, p, a, b); break;
      case kLdsB128: lds_b128(lds, base, lane); break;
      case kLdsTr: lds_tr(lds, base, lane); break;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float keep = s[0] + s[1];
#pragma unroll
  for (int c = 0; c < 8; ++c) keep += x[c] + float(p[c]);
#pragma unroll
  for (int c = 0; c < 4; ++c) keep += acc[c][0];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[2 * (blockIdx.x * nw + w)] = t1 - t0;
    out[2 * (blockIdx.x * nw + w) + 1] = r1 - r0;
  }
  if (keep == 1234.5f) sink[tid] = keep;  // never met for these inputs; keeps the work alive
}

// Reads n 16-byte vectors of `src` once (grid-stride, U loads in flight per
// lane), ordinary or nontemporal loads, and folds them into one word per
// thread; the only store sits behind a condition the data (all zero) never
// meets.
template <bool NT, int U>
__global__ __launch_bounds__(256) void hbm_read(const u32x4* __restrict__ src, size_t n, unsigned* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= NT ? __builtin_nontemporal_load(src + i) : src[i];
  if ((acc.x | acc.y | acc.z | acc.w) == 0x5a5a5a5au) sink[threadIdx.x] = acc.x;
}

template <bool NT, int U>
double hbm_rate(const u32x4* buf, size_t n, unsigned* sink) {
  const int grid = 256 * 16;  // 16 workgroups of 256 threads per compute unit
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) std::exit(1);
  for (int r = 0; r < 3; ++r) hbm_read<NT, U><<<grid, 256>>>(buf, n, sink);  // warm-up
  (void)hipEventRecord(e0, nullptr);
  constexpr int kReps = 5;
  for (int r = 0; r < kReps; ++r) hbm_read<NT, U><<<grid, 256>>>(buf, n, sink);
  (void)hipEventRecord(e1, nullptr);
  if (hipDeviceSynchronize() != hipSuccess) {
    std::fprintf(stderr, "hbm probe failed: %s\n", hipGetErrorString(hipGetLastError()));
    std::exit(2);
  }
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return double(n) * 16.0 * kReps / (ms * 1e-3) / 1e12;
}

const char* kNames[] = {"v_exp_f32", "v_fma_f32", "v_add_f32", "v_cvt_pk_bf16_f32", "v_max3_f32",
                        "v_mfma_f32_32x32x16_bf16", "softmax tile (112 VALU)", "ds_read_b128", "ds_read_b64_tr_b16"};
// Instructions (or reads) per loop iteration of each stream.
const int kPerIter[] = {64, 64, 64, 64, 64, 16, 112, 16, 16};

struct Result {
  double a, b;  // mean cycles per instruction of the A and B waves
  double ghz;   // shader clock: s_memtime cycles over s_memrealtime time, mean over waves
  double ms;    // event time of the timed launch
};

template <int A, int B>
Result run(int threads, int split) {
  const int nw = threads / 64;
  unsigned long long* out = nullptr;
  float* sink = nullptr;
  if (hipMalloc(&out, 2 * sizeof(unsigned long long) * kGrid * nw) != hipSuccess ||
      hipMalloc(&sink, sizeof(float) * threads) != hipSuccess) {
    std::fprintf(stderr, "hipMalloc failed\n");
    std::exit(1);
  }
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&probe<A, B>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess) {
    std::fprintf(stderr, "hipFuncSetAttribute failed\n");
    std::exit(1);
  }
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) std::exit(1);
  probe<A, B><<<kGrid, threads, kLdsBytes>>>(out, sink, split);  // warm-up
  (void)hipEventRecord(e0, nullptr);
  probe<A, B><<<kGrid, threads, kLdsBytes>>>(out, sink, split);
  (void)hipEventRecord(e1, nullptr);
  if (hipDeviceSynchronize() != hipSuccess) {
    std::fprintf(stderr, "probe failed: %s\n", hipGetErrorString(hipGetLastError()));
    std::exit(2);
  }
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  static unsigned long long h[2 * kGrid * 8];
  if (hipMemcpy(h, out, 2 * sizeof(unsigned long long) * kGrid * nw, hipMemcpyDeviceToHost) != hipSuccess) std::exit(3);
  double sa = 0, sb = 0, cyc = 0, ticks = 0;
  int na = 0, nb = 0;
  for (int g = 0; g < kGrid; ++g)
    for (int w = 0; w < nw; ++w) {
      const double c = double(h[2 * (g * nw + w)]);
      cyc += c;
      ticks += double(h[2 * (g * nw + w) + 1]);
      if (w < split) { sa += c; ++na; }
      else { sb += c; ++nb; }
    }
  (void)hipFree(out);
  (void)hipFree(sink);
  Result r;
  r.a = na ? sa / na / kIter / kPerIter[A] : 0.0;
  r.b = nb ? sb / nb / kIter / kPerIter[B] : 0.0;
  r.ghz = ticks > 0 ? cyc / ticks * 0.1 : 0.0;
  r.ms = ms;
  return r;
}

template <int A>
void alone(int waves_per_simd) {
  const Result r = run<A, A>(256 * waves_per_simd, 8);
  std::printf("%-26s alone, %d wave(s) per SIMD: %6.2f cycles per instruction per wave  (clock %.2f GHz, %.3f ms)\n",
              kNames[A], waves_per_simd, r.a, r.ghz, r.ms);
}

}  // namespace

int main() {
  std::printf("# gfx950 probe: 256 workgroups, one per compute unit, %d iterations per wave, s_memtime cycles\n", kIter);
  alone<kExp>(1);
  alone<kFma>(1);
  alone<kAdd>(1);
  alone<kCvt>(1);
  alone<kMax3>(1);
  {
    const Result r = run<kMfma, kMfma>(256, 8);
    const double flops = 256.0 * 4 * kIter * 16 * 32768.0;
    std::printf("%-26s alone, 1 wave(s) per SIMD: %6.2f cycles per instruction per wave  (clock %.2f GHz, %.3f ms = %.0f TFLOP/s)\n",
                kNames[kMfma], r.a, r.ghz, r.ms, flops / (r.ms * 1e-3) / 1e12);
  }
  alone<kSoftmaxMix>(1);
  // Two waves per SIMD (waves w and w + 4 of an 8-wave workgroup share a SIMD).
  {
    const Result r = run<kMfma, kSoftmaxMix>(512, 4);
    std::printf("co-issue: waves 0-3 MFMA %.2f cycles per MFMA, waves 4-7 softmax tile %.2f cycles per VALU instruction"
                "  (clock %.2f GHz, %.3f ms)\n", r.a, r.b, r.ghz, r.ms);
  }
  {
    const Result r = run<kSoftmaxMix, kSoftmaxMix>(512, 4);
    std::printf("two softmax waves per SIMD: %.2f cycles per VALU instruction per wave  (clock %.2f GHz, %.3f ms)\n",
                r.a, r.ghz, r.ms);
  }
  {
    const Result r = run<kMfma, kMfma>(512, 4);
    // 256 workgroups x 8 waves x kIter x 16 MFMAs of 32 x 32 x 16 x 2 flops.
    const double flops = 256.0 * 8 * kIter * 16 * 32768.0;
    // The waves of a SIMD take the matrix pipe in turn, so only the launch
    // time is meaningful here.
    std::printf("two MFMA waves per SIMD: %.3f ms = %.0f TFLOP/s (clock %.2f GHz)\n", r.ms,
                flops / (r.ms * 1e-3) / 1e12, r.ghz);
  }
  alone<kLdsB128>(1);
  alone<kLdsB128>(2);
  alone<kLdsTr>(1);
  alone<kLdsTr>(2);
  {
    const size_t bytes = size_t(8) << 30;
    const size_t n = bytes / 16;
    u32x4* buf = nullptr;
    unsigned* sink = nullptr;
    if (hipMalloc(&buf, bytes) != hipSuccess || hipMalloc(&sink, 256 * sizeof(unsigned)) != hipSuccess ||
        hipMemset(buf, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      std::fprintf(stderr, "hbm buffer setup failed\n");
      std::exit(1);
    }
    std::printf("HBM read of 8 GiB, 16-byte loads, 4 in flight per lane: ordinary %.2f TB/s, nontemporal %.2f TB/s\n",
                hbm_rate<false, 4>(buf, n, sink), hbm_rate<true, 4>(buf, n, sink));
    std::printf("HBM read of 8 GiB, 16-byte loads, 8 / 16 in flight per lane: ordinary %.2f / %.2f TB/s, "
                "nontemporal %.2f / %.2f TB/s\n",
                hbm_rate<false, 8>(buf, n, sink), hbm_rate<false, 16>(buf, n, sink), hbm_rate<true, 8>(buf, n, sink),
                hbm_rate<true, 16>(buf, n, sink));
    (void)hipFree(buf);
    (void)hipFree(sink);
  }
  return 0;
}
