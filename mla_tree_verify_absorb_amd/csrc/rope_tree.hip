// NeoX rotary embedding of the tree nodes' rotary queries and keys at their
// positions (cache length + depth), in place, just before verification.
//
// The engine rotates with NeoX rotary embeddings and computes the angle in
// double precision (page "The Moment of Truth: Validating a Custom CUDA
// Inference Engine for Kimi K2.6", section "What the Output Tells Us"); node
// positions are cache length plus depth as int64 (page "The Build That Proved
// It: Compiling the Native DDTree Speculative Decoding Engine", section "The
// Thinking Process Visible in Reasoning").  NeoX pairs element i with element
// i + Dr/2: out[i] = x[i] cos a_i - x[i + Dr/2] sin a_i, out[i + Dr/2] =
// x[i + Dr/2] cos a_i + x[i] sin a_i, a_i = position * inv_freq[i].  The caller
// supplies inv_freq, so any frequency scaling folds in there.
//
// One workgroup per tree node: its Dr/2 angles and their sine and cosine are
// computed once in float64 (LDS), then applied to the node's H query rows and
// its key row.  The rotation itself is also done in float64 and rounded once
// to the storage type (float32; bf16 through float32, round to nearest even).
#include <cmath>

#include "ddtree_internal.h"

namespace ddtree {
namespace {

__device__ __forceinline__ double load_elem(const void* p, int64_t i, bool bf16) {
  if (bf16) {
    const uint16_t u = static_cast<const uint16_t*>(p)[i];
    return (double)__uint_as_float((uint32_t)u << 16);
  }
  return (double)static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_elem(void* p, int64_t i, double v, bool bf16) {
  const float f = (float)v;
  if (bf16) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);   // round to nearest even (inputs are finite)
    static_cast<uint16_t*>(p)[i] = (uint16_t)(u >> 16);
  } else {
    static_cast<float*>(p)[i] = f;
  }
}

__global__ void __launch_bounds__(256) rope_tree_kernel(RopeArgs a) {
  __shared__ double s_cos[kMaxRopeDim / 2], s_sin[kMaxRopeDim / 2];
  const int node = blockIdx.x;   // b * N + i
  const int half = a.Dr / 2;
  const int64_t pos = a.positions[node];
  for (int t = threadIdx.x; t < half; t += blockDim.x) {
    double sn, cs;
    sincos((double)pos * a.inv_freq[t], &sn, &cs);
    s_cos[t] = cs;
    s_sin[t] = sn;
  }
  __syncthreads();
  const int rows = (a.q_rope ? a.H : 0) + (a.krope_tree ? 1 : 0);
  for (int idx = threadIdx.x; idx < rows * half; idx += blockDim.x) {
    const int r = idx / half, t = idx - r * half;
    void* base;
    int64_t off;
    if (a.q_rope && r < a.H) {
      base = a.q_rope;
      off = ((int64_t)node * a.H + r) * a.Dr;
    } else {
      base = a.krope_tree;
      off = (int64_t)node * a.ld_krope_tree;
    }
    const double x1 = load_elem(base, off + t, a.bf16), x2 = load_elem(base, off + t + half, a.bf16);
    const double c = s_cos[t], s = s_sin[t];
    store_elem(base, off + t, x1 * c - x2 * s, a.bf16);
    store_elem(base, off + t + half, x2 * c + x1 * s, a.bf16);
  }
}

}  // namespace

hipError_t launch_rope_tree(const RopeArgs& a, hipStream_t stream) {
  const int64_t nodes = (int64_t)a.B * a.N;
  if (nodes == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_tree_kernel, dim3((unsigned)nodes), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ddtree
