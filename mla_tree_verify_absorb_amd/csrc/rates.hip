// Achievable-rate probes for MI355X (gfx950): the rate the chip sustains on a
// back-to-back bf16 MFMA loop and on a read-only HBM stream, measured on the
// box next to the attention and accept kernels so that their fractions can be
// read against the clock and memory the chip actually holds under load.  Not
// part of the verify path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ddtree_rates.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;   // independent accumulators per wave

// Every wave issues kChains independent v_mfma_f32_32x32x16_bf16 per iteration
// (32768 flop each); the accumulators are summed and stored once so that the
// loop stays live.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(1e-3f * (float)((lane + k) & 7));
    b[k] = (__bf16)(1e-3f * (float)((lane * 3 + k) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// Reads n16 16-byte words with nontemporal loads: workgroup g reads the
// contiguous span [g * per, (g + 1) * per), 8 loads in flight per thread.
// Whole spans per workgroup keep each one's requests inside few DRAM pages; a
// grid-stride walk (every load of a thread one grid apart) measured 10-20%
// slower.  One XOR per workgroup thread is stored so that the loads stay live.
constexpr int kStreamThreads = 256;
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                     int64_t per, uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  constexpr int T = kStreamThreads;
  const int64_t start = (int64_t)blockIdx.x * per;
  const int64_t end = start + per < n16 ? start + per : n16;
  int64_t c = start + threadIdx.x;
  uint32_t x = 0;
  for (; c + (U - 1) * T < end; c += U * T) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + c + u * T);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; c < end; c += T) {
    const u32x4 v = __builtin_nontemporal_load(src + c);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * T + threadIdx.x] = x;
}

}  // namespace

extern "C" {

int64_t ddtree_rates_mfma_loop_flops(int32_t workgroups, int32_t iters) {
  return (int64_t)workgroups * 4 * iters * kChains * (2LL * 32 * 32 * 16);
}

int ddtree_rates_mfma_loop(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || iters < 1 || !sink) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int ddtree_rates_stream_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15) || workgroups < 1)
    return -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kStreamThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), n16, (n16 + workgroups - 1) / workgroups, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
