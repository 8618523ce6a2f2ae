// Tiled one-pass attention forward for fp32 inputs on the gfx950 fp32 MFMA.
//
// Same method and loop structure as the fp16/bf16 kernel (the online
// softmax of the quidproquo.cc guide, "Mechanism: run with the wrong answer,
// then correct it", fused per tile as in the comfyai.app chapter "6.3
// FlashAttention", section 6.3.3), with every operand in fp32:
// v_mfma_f32_32x32x2_f32 computes S^T = K_j Q^T and O^T += V_j^T P^T, so the
// weights P are never rounded below fp32.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows, 32-key
// tiles): lane (n, h) of a wave owns query n of the wave's 32 rows; for the
// fp32 MFMA, lane half h supplies the k-th element with k = h, and the D
// columns are split so that half h walks columns [h D/2, (h+1) D/2), which
// makes its K reads 16-byte vectors.  V stays row-major in LDS: the A
// operand of the P V product is one fp32 per lane, 32 consecutive columns of
// one key row per half-wave.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

#include "attn_internal.hpp"

namespace attn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 32;
constexpr int NT = 256;

template <int D>
struct TileF {
  // K: rows 4 banks apart (16 lanes x 16 B reads from 16 rows are disjoint).
  // V: rows 8 banks apart, so the two half-waves (rows m and m + 4) use
  // disjoint 32-bank halves.
  static constexpr int KPITCH = D * 4 + 16;
  static constexpr int VPITCH = D * 4 + 32;
  static constexpr int KBYTES = BN * KPITCH;
  static constexpr int STAGE = KBYTES + BN * VPITCH;
  static constexpr int CHUNKS = BN * D / 4 / NT;
  static constexpr int HALF = D / 2;
  static constexpr int DBLK = D / 32;
};

__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void prefill_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Lq, int Lk, int nqt, float c,
    float qsign) {
  using T = TileF<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;

  const int total = BH * nqt;
  const int wg = blockIdx.x;
  const int logical = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
  const int bh = logical / nqt;
  const int qt = CAUSAL ? nqt - 1 - logical % nqt : logical % nqt;
  const int q0 = qt * BM;
  const int off = Lk - Lq;

  const float* Qh = Q + (size_t)bh * Lq * D;
  const float* Kh = K + (size_t)bh * Lk * D;
  const float* Vh = V + (size_t)bh * Lk * D;

  const int q_last = min(q0 + BM, Lq) - 1;
  const int kv_end = CAUSAL ? min(Lk, q_last + off + 1) : Lk;
  const int nkv = (kv_end + BN - 1) / BN;
  const int wq0 = q0 + 32 * w;
  const bool wave_live = wq0 < Lq;
  const int w_key_end = CAUSAL ? min(Lk, min(wq0 + 31, Lq - 1) + off + 1) : Lk;

  // Q^T fragment: lane (n, h) holds Q[qi][h D/2 + t], t < D/2.
  const int qi = wq0 + n;
  float qreg[T::HALF];
#pragma unroll
  for (int t4 = 0; t4 < T::HALF / 4; ++t4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (qi < Lq) x = *reinterpret_cast<const f32x4*>(Qh + (size_t)qi * D + h * T::HALF + 4 * t4);
#pragma unroll
    for (int e = 0; e < 4; ++e) qreg[4 * t4 + e] = x[e] * qsign;
  }

  f32x4 kst[T::CHUNKS], vst[T::CHUNKS];
  auto gload = [&](int kv0) {
#pragma unroll
    for (int u = 0; u < T::CHUNKS; ++u) {
      const int ci = tid + NT * u;
      const int row = ci / (D / 4), col = ci % (D / 4);
      const int key = kv0 + row;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < Lk) {
        kx = *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + col * 4);
        vx = *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + col * 4);
      }
      kst[u] = kx;
      vst[u] = vx;
    }
  };
  auto sstore = [&](int stage) {
    char* base = smem + stage * T::STAGE;
#pragma unroll
    for (int u = 0; u < T::CHUNKS; ++u) {
      const int ci = tid + NT * u;
      const int row = ci / (D / 4), col = ci % (D / 4);
      *reinterpret_cast<f32x4*>(base + row * T::KPITCH + col * 16) = kst[u];
      *reinterpret_cast<f32x4*>(base + T::KBYTES + row * T::VPITCH + col * 16) = vst[u];
    }
  };

  f32x16 oacc[T::DBLK];
#pragma unroll
  for (int i = 0; i < T::DBLK; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (nkv > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const int kv0 = j * BN;
    if (j + 1 < nkv) gload(kv0 + BN);

    if (wave_live && kv0 < w_key_end) {
      const char* Ks = smem + (j & 1) * T::STAGE;
      const char* Vs = Ks + T::KBYTES;

      // S^T = K_j Q^T: A = K[m][h D/2 + t], B = Q[n][h D/2 + t].
      f32x16 sacc = f32x16{};
      const char* kp = Ks + n * T::KPITCH + h * T::HALF * 4;
#pragma unroll
      for (int t4 = 0; t4 < T::HALF / 4; ++t4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(kp + 16 * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qreg[4 * t4 + e], sacc, 0, 0, 0);
      }

      // Register r of lane (n, h) holds the score of key kv0 + 8(r/4) + 4h + r%4.
      const bool need_mask = (kv0 + BN > Lk) || (CAUSAL && kv0 + BN - 1 > wq0 + off);
      unsigned live = 0xffffu;
      if (need_mask) {
        live = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool ok = key < Lk && (!CAUSAL || key <= qi + off);
          live |= (ok ? 1u : 0u) << r;
          if (!ok) sacc[r] = -INFINITY;
        }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
      mx = halves_max(mx);
      const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
      const float m_new = fmaxf(m_run, m_tile);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      float p[16];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -m_use));
        if (need_mask && !((live >> r) & 1u)) x = 0.f;
        p[r] = x;
        psum += x;
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < T::DBLK; ++i) oacc[i] *= alpha;

      // O^T += V_j^T P^T, one key pair (k = h) per MFMA.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < T::DBLK; ++db) {
          const float a = *reinterpret_cast<const float*>(Vs + key * T::VPITCH + (32 * db + n) * 4);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[r], oacc[db], 0, 0, 0);
        }
      }
    }

    if (j + 1 < nkv) sstore((j + 1) & 1);
    __syncthreads();
  }

  const float l_tot = halves_sum(l_run);
  if (wave_live && qi < Lq) {
    const float inv = 1.f / l_tot;
    float* Oq = O + (size_t)bh * Lq * D + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < T::DBLK; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * db + 8 * jj + 4 * h;
        const f32x4 val = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv,
                           oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv};
        *reinterpret_cast<f32x4*>(Oq + d) = val;
      }
    if (h == 0) LSE[(size_t)bh * Lq + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  const int nqt = (a.Lq + BM - 1) / BM;
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3(a.BH * nqt), dim3(NT), 0, s,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.BH, a.Lq,
                     a.Lk, nqt, a.c, a.neg ? -1.f : 1.f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(int D, bool causal, const PrefillArgs& a, hipStream_t s) {
  if (D == 64) return causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
  return causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
}

}  // namespace attn
