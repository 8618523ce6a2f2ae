// Single-query attention (decode, Lq = 1) by split-KV, for fp32/fp16/bf16.
//
// The decode phase emits one token at a time (quidproquo.cc guide,
// slide 5), so each (batch, head) has one query against Lk cached keys.  The
// work is a memory-bound stream over K and V; one workgroup per (b, h) would
// leave most of the chip idle, so the keys of each (b, h) are cut into
// `splits` contiguous ranges that run as independent workgroups.
//
// decode_split_kernel: one workgroup per (b*h, range p), flattened.  Each wave streams
// its keys with 16-byte loads (LPK lanes cover one key row; a wave load
// covers KPI keys), reduces the partial dot products across the LPK lanes
// with DPP, and runs the guide's recurrence ("Mechanism: run with the wrong
// answer, then correct it": d_k = max(d_{k-1}, chunk max),
// s_k = s_{k-1} exp(d_{k-1} - d_k) + sum exp(a_i - d_k), output rescaled the
// same way) on its own (d, s, O~) state.  The states of the KPI key lanes and
// of the 4 waves are merged with the same correction, and the range writes
// d_p (base 2), s_p and the normalised O_p = O~ / s_p.
//
// decode_combine_kernel: one workgroup per (b, h) merges the ranges as the
// chunks of the guide's output correction:
//   d = max_p d_p,  s = sum_p s_p exp(d_p - d),
//   O = sum_p O_p (s_p / s) exp(d_p - d),  lse = d + ln s.
// Empty ranges (s_p = 0) are skipped; a (b, h) with no key at all gets
// O = 0 and lse = -inf (the empty sum).
//
// With per-sequence lengths (a KV cache whose rows past a sequence's length
// are unused), the same kernels run over the first seqlens[b] keys of each
// (b, h), cut into `splits` ranges of that length.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "attn_internal.hpp"

namespace attn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int NWAVE = NT / 64;
constexpr int UNROLL = 8;  // key loads per lane per tensor in flight per iteration

// Storage types: 0 = f32, 1 = f16, 2 = bf16.
template <int DT> struct Elem;
template <> struct Elem<0> {
  static constexpr int PER16 = 4;  // elements per 16-byte load
  __device__ static void unpack(const u32x4& x, float* f) {
    // Copy each element to a scalar first: bit-casting a vector element
    // lvalue directly is miscompiled (every lane reads element 0).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned u = x[i];
      f[i] = __builtin_bit_cast(float, u);
    }
  }
  __device__ static void store(void* o, int idx, float v) { static_cast<float*>(o)[idx] = v; }
};
template <> struct Elem<1> {
  static constexpr int PER16 = 8;
  __device__ static void unpack(const u32x4& x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(x[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(x[i] >> 16));
    }
  }
  __device__ static void store(void* o, int idx, float v) {
    static_cast<_Float16*>(o)[idx] = (_Float16)v;
  }
};
template <> struct Elem<2> {
  static constexpr int PER16 = 8;
  __device__ static void unpack(const u32x4& x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, x[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, x[i] & 0xffff0000u);
    }
  }
  __device__ static void store(void* o, int idx, float v) {
    static_cast<__bf16*>(o)[idx] = (__bf16)v;
  }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// Sum over groups of LANES consecutive lanes (LANES in {4, 8, 16, 32});
// every lane of the group ends with the group sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xb1>(x);  // quad_perm [1,0,3,2]: pairs
  x += dpp<0x4e>(x);  // quad_perm [2,3,0,1]: quads
  if constexpr (LANES >= 8) x += dpp<0x141>(x);   // row_half_mirror: 8 lanes
  if constexpr (LANES >= 16) x += dpp<0x140>(x);  // row_mirror: 16 lanes
  if constexpr (LANES >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Merge state (m2, l2, o2) into (m, l, o): the guide's correction with the
// larger maximum as the new reference.  States with l = 0 are empty.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2, const float* o2) {
  const float mn = fmaxf(m, m2);
  const float mu = (mn == -INFINITY) ? 0.f : mn;
  const float a1 = __builtin_amdgcn_exp2f(m - mu);
  const float a2 = __builtin_amdgcn_exp2f(m2 - mu);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = mn;
}

template <int DT, int D>
__global__ __launch_bounds__(NT) void decode_split_kernel(
    const u32x4* __restrict__ Q, const u32x4* __restrict__ K, const u32x4* __restrict__ V,
    float* __restrict__ part_o, float* __restrict__ part_m, float* __restrict__ part_l, int Lk,
    int keys_per_split, int splits, float c, float qsign, const int* __restrict__ seqlens, int H) {
  using E = Elem<DT>;
  constexpr int EPL = E::PER16;       // elements per lane per key
  constexpr int LPK = D / EPL;        // lanes per key row
  constexpr int KPI = 64 / LPK;       // keys per wave load
  constexpr int KPW = KPI * UNROLL;   // keys per wave per iteration
  constexpr int KPB = KPW * NWAVE;    // keys per workgroup per iteration
  constexpr int ROW16 = D / EPL;      // 16-byte chunks per row

  __shared__ float sm_o[NWAVE][D];
  __shared__ float sm_m[NWAVE], sm_l[NWAVE];

  const int split = blockIdx.x % splits;
  const int bh = blockIdx.x / splits;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kq = lane / LPK, dl = lane % LPK;

  // Keys of this (b, h): all Lk, or the first seqlens[b] of them (a KV
  // cache with ragged lengths), cut into `splits` equal ranges.
  int len = Lk, kps = keys_per_split;
  if (seqlens != nullptr) {
    len = min(max(seqlens[bh / H], 0), Lk);
    kps = (len + splits - 1) / splits;
  }
  const int kb = min(len, split * kps);
  const int ke = min(len, kb + kps);

  // Query slice, pre-multiplied by |scale| log2(e) (and the sign of scale).
  float qf[EPL];
  E::unpack(Q[(size_t)bh * ROW16 + dl], qf);
#pragma unroll
  for (int i = 0; i < EPL; ++i) qf[i] *= c * qsign;

  const u32x4* Kh = K + (size_t)bh * Lk * ROW16;
  const u32x4* Vh = V + (size_t)bh * Lk * ROW16;

  float m_run = -INFINITY, l_run = 0.f;
  float o[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) o[i] = 0.f;

  for (int base = kb + w * KPW; base < ke; base += KPB) {
    // Every K/V byte is read exactly once: nontemporal loads stream past the
    // caches (measured on the part: a plain 8 GiB read reaches 6.0-6.1 TB/s
    // with ordinary 16-byte loads and 6.4-6.6 TB/s with nontemporal ones).
    u32x4 kx[UNROLL], vx[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + kq + KPI * u;
      kx[u] = key < ke ? __builtin_nontemporal_load(Kh + (size_t)key * ROW16 + dl) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = base + kq + KPI * u;
      vx[u] = key < ke ? __builtin_nontemporal_load(Vh + (size_t)key * ROW16 + dl) : u32x4{0u, 0u, 0u, 0u};
    }
    float sc[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float kf[EPL];
      E::unpack(kx[u], kf);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc = __builtin_fmaf(qf[i], kf[i], acc);
      acc = group_sum<LPK>(acc);
      sc[u] = (base + kq + KPI * u < ke) ? acc : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) mx = fmaxf(mx, sc[u]);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] *= alpha;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float p = __builtin_amdgcn_exp2f(sc[u] - m_use);
      psum += p;
      float vf[EPL];
      E::unpack(vx[u], vf);
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i] = __builtin_fmaf(p, vf[i], o[i]);
    }
    l_run = l_run * alpha + psum;
  }

  // Merge the KPI key lanes of the wave (lanes dl, dl + LPK, ...).
#pragma unroll
  for (int sh = LPK; sh < 64; sh <<= 1) {
    const float m2 = __shfl_xor(m_run, sh);
    const float l2 = __shfl_xor(l_run, sh);
    float o2[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) o2[i] = __shfl_xor(o[i], sh);
    merge_state<EPL>(m_run, l_run, o, m2, l2, o2);
  }
  if (kq == 0) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) sm_o[w][dl * EPL + i] = o[i];
    if (dl == 0) {
      sm_m[w] = m_run;
      sm_l[w] = l_run;
    }
  }
  __syncthreads();
  if (tid < D) {
    float m = sm_m[0], l = sm_l[0], acc = sm_o[0][tid];
#pragma unroll
    for (int ww = 1; ww < NWAVE; ++ww) merge_state<1>(m, l, &acc, sm_m[ww], sm_l[ww], &sm_o[ww][tid]);
    const size_t pi = (size_t)bh * splits + split;
    part_o[pi * D + tid] = l > 0.f ? acc / l : 0.f;
    if (tid == 0) {
      part_m[pi] = m;
      part_l[pi] = l;
    }
  }
}

template <int DT, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, void* __restrict__ O, float* __restrict__ LSE, int splits) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* pm = part_m + (size_t)bh * splits;
  const float* pl = part_l + (size_t)bh * splits;
  float dmax = -INFINITY;
  for (int p = 0; p < splits; ++p)
    if (pl[p] > 0.f) dmax = fmaxf(dmax, pm[p]);
  const float du = (dmax == -INFINITY) ? 0.f : dmax;
  float s = 0.f;
  for (int p = 0; p < splits; ++p)
    if (pl[p] > 0.f) s += pl[p] * __builtin_amdgcn_exp2f(pm[p] - du);
  const float inv_s = 1.f / s;
  float acc = 0.f;
  for (int p = 0; p < splits; ++p)
    if (pl[p] > 0.f)
      acc += part_o[((size_t)bh * splits + p) * D + d] * (pl[p] * inv_s) * __builtin_amdgcn_exp2f(pm[p] - du);
  Elem<DT>::store(O, bh * D + d, acc);
  if (d == 0) LSE[bh] = (dmax + log2f(s)) * kLn2;
}

template <int DT, int D>
hipError_t launch_dt(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<DT, D>), dim3(a.splits * a.BH), dim3(NT), 0, s,
                     static_cast<const u32x4*>(a.q), static_cast<const u32x4*>(a.k),
                     static_cast<const u32x4*>(a.v), a.part_o, a.part_m, a.part_l, a.Lk,
                     a.keys_per_split, a.splits, a.c, a.neg ? -1.f : 1.f, a.seqlens, a.H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<DT, D>), dim3(a.BH), dim3(D), 0, s, a.part_o, a.part_m,
                     a.part_l, a.o, a.lse, a.splits);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_d(int D, const DecodeArgs& a, hipStream_t s) {
  return D == 64 ? launch_dt<DT, 64>(a, s) : launch_dt<DT, 128>(a, s);
}

}  // namespace

hipError_t launch_decode(int dtype, int D, const DecodeArgs& a, hipStream_t s) {
  switch (dtype) {
    case 0: return launch_d<0>(D, a, s);
    case 1: return launch_d<1>(D, a, s);
    default: return launch_d<2>(D, a, s);
  }
}

}  // namespace attn
