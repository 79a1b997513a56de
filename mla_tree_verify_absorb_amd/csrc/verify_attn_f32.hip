// Tree-verify attention, absorbed MLA form, float32 arithmetic on float32 or
// bf16 inputs (bf16 widened exactly on load).
//
// What is computed (page "The Moment of Proof: Validating a Native CUDA
// Speculative Decoding Engine", section "Input Knowledge Required": MLA in
// absorb form and a draft tree verified under a custom mask): for each
// request b, node i and head h, the scores of the latent query against the
// request's cached latent rows and the node's visible tree rows, an online
// softmax over them, the softmax-weighted sum of the latent rows and the
// natural log-sum-exp.
//
// This kernel serves the float32 workloads (the pages' tiny FP32 model has
// kv_lora 64 with 4 heads) and bf16 inputs at dims other than the MFMA
// kernel's (512, 64): small, launch-latency-bound shapes where MFMA tiles
// would sit mostly empty.  One workgroup per (request, node); each
// wave takes one head at a time.  Keys are visited in chunks of 64, one key
// per lane for the score (q staged in LDS), then the chunk's probabilities
// are broadcast and every lane accumulates its own output dimensions from
// coalesced row reads.  Any Dl <= 512 and Dr <= 512.
#include <cmath>

#include "ddtree_internal.h"

namespace ddtree {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxDl = 512;
constexpr int kMaxDq = 1024;   // Dl + Dr
constexpr int kMaxT = kMaxDl / 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t bits) { return __builtin_bit_cast(float, (uint32_t)bits << 16); }

template <typename T>
__global__ void __launch_bounds__(kWaves * 64) verify_attn_generic_kernel(AttnArgs a) {
  __shared__ float s_q[kWaves][kMaxDq];
  const int bi = blockIdx.x;            // b * N + i
  const int b = bi / a.N;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int Dl = a.Dl, Dr = a.Dr;
  const int W = (a.N + 31) >> 5;

  const T* q_lat = static_cast<const T*>(a.q_lat);
  const T* q_rope = static_cast<const T*>(a.q_rope);
  const T* ckv = static_cast<const T*>(a.ckv);
  const T* krope = static_cast<const T*>(a.krope);
  const T* ckv_t = static_cast<const T*>(a.ckv_tree);
  const T* krope_t = static_cast<const T*>(a.krope_tree);
  const uint32_t* mrow = a.mask + (int64_t)bi * W;

  const int64_t p0 = a.prefix_offsets[b];
  int64_t L = a.prefix_offsets[b + 1] - p0;
  if (L < 0) L = 0;
  const int64_t total = L + a.N;

  for (int h = wave; h < a.H; h += kWaves) {
    const int64_t row = (int64_t)bi * a.H + h;
    for (int d = lane; d < Dl; d += 64) s_q[wave][d] = widen(q_lat[row * Dl + d]);
    for (int d = lane; d < Dr; d += 64) s_q[wave][Dl + d] = widen(q_rope[row * Dr + d]);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

    float m = -INFINITY, l = 0.f;
    float acc[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) acc[t] = 0.f;

    for (int64_t k0 = 0; k0 < total; k0 += 64) {
      // --- score of key k0 + lane ---
      const int64_t kk = k0 + lane;
      float s = -INFINITY;
      if (kk < total) {
        const T* crow;
        const T* rrow;
        bool vis = true;
        if (kk < L) {
          crow = ckv + (p0 + kk) * a.ld_ckv;
          rrow = krope + (p0 + kk) * a.ld_krope;
        } else {
          const int node = (int)(kk - L);
          vis = (mrow[node >> 5] >> (node & 31)) & 1u;
          crow = ckv_t + ((int64_t)b * a.N + node) * a.ld_ckv_tree;
          rrow = krope_t + ((int64_t)b * a.N + node) * a.ld_krope_tree;
        }
        if (vis) {
          float dot = 0.f;
          for (int d = 0; d < Dl; ++d) dot = fmaf(s_q[wave][d], widen(crow[d]), dot);
          for (int d = 0; d < Dr; ++d) dot = fmaf(s_q[wave][Dl + d], widen(rrow[d]), dot);
          s = dot * a.scale;
        }
      }
      // --- online softmax update ---
      const float cmax = wave_max(s);
      const float m_new = fmaxf(m, cmax);
      if (m_new == -INFINITY) continue;            // nothing visible yet (wave-uniform)
      const float alpha = expf(m - m_new);         // m = -inf gives 0
      const float p = (s == -INFINITY) ? 0.f : expf(s - m_new);
      l = l * alpha + wave_sum(p);
      m = m_new;
#pragma unroll
      for (int t = 0; t < kMaxT; ++t) acc[t] *= alpha;
      // --- accumulate the chunk's weighted latent rows, lane = output dims ---
      const int nk = (int)((total - k0) < 64 ? (total - k0) : 64);
      for (int j = 0; j < nk; ++j) {
        const float pj = __shfl(p, j, 64);
        if (pj == 0.f) continue;                   // wave-uniform
        const int64_t kj = k0 + j;
        const T* crow = (kj < L) ? ckv + (p0 + kj) * a.ld_ckv
                                 : ckv_t + ((int64_t)b * a.N + (kj - L)) * a.ld_ckv_tree;
#pragma unroll
        for (int t = 0; t < kMaxT; ++t) {
          const int d = lane + 64 * t;
          if (d < Dl) acc[t] = fmaf(pj, widen(crow[d]), acc[t]);
        }
      }
    }
    const float inv_l = 1.f / l;
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
      const int d = lane + 64 * t;
      if (d < Dl) a.o[row * Dl + d] = acc[t] * inv_l;
    }
    if (lane == 0) a.lse[row] = m + logf(l);
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_verify_attn_generic(const AttnArgs& a, bool bf16, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(verify_attn_generic_kernel<uint16_t>, dim3(a.B * a.N), dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(verify_attn_generic_kernel<float>, dim3(a.B * a.N), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ddtree
