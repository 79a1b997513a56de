// Greedy tree accept: the target's argmax per tree node, then the longest
// root path whose draft tokens match the greedy choices.
//
// Tokens along the longest matching path are accepted (page "The Moment of
// Proof: Validating a Native CUDA Speculative Decoding Engine", section
// "Input Knowledge Required"; greedy acceptance and path selection: page "The
// Moment of Proof: Running the Native DDTree Speculative Decoding Engine",
// section "Input Knowledge Required"; the longest prefix matching the
// target's greedy choices: page "The Build That Proved It: Compiling the
// Native DDTree Speculative Decoding Engine", section "The Output Knowledge
// Created").
//
// accept_argmax: one 512-thread workgroup per logits row streams the row
// with 16-byte nontemporal loads (10 in flight per thread) and keeps (max,
// first index) per thread: a thread visits its elements in increasing index
// order, so a strict comparison keeps the first of equal values with one
// compare per element.  Waves reduce with shuffles, the block through LDS,
// both with an explicit lowest-index tie rule, so the result does not depend
// on the reduction order.  NaN never compares greater and is never chosen.
// accept_path: one workgroup per request, one thread per node; each thread
// walks its ancestor chain once (bounded by N) to decide whether its root path
// matches and to record its ancestors as a bitmask; the deepest matching node
// (smallest index on ties) is found with an LDS max over a packed (depth,
// -index) key, and the nodes in the terminal's bitmask place themselves by
// depth.
#include <climits>

#include "ddtree_internal.h"

namespace ddtree {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kArgmaxThreads = 512;
constexpr int kUnroll = 10;

struct ValIdx {
  float v;
  int i;
};

__device__ __forceinline__ void take_if_better(ValIdx& best, float v, int i) {
  // strictly greater, or equal with a smaller index
  if (v > best.v || (v == best.v && i < best.i)) {
    best.v = v;
    best.i = i;
  }
}

// a thread's own scan: indices only grow, so equal values keep the earlier one
__device__ __forceinline__ void take_if_greater(ValIdx& best, float v, int i) {
  if (v > best.v) {
    best.v = v;
    best.i = i;
  }
}

template <bool kVec>
__global__ void __launch_bounds__(kArgmaxThreads) argmax_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                                int32_t* __restrict__ out) {
  const int64_t row = blockIdx.x;
  const float* p = logits + row * ld;
  const int tid = threadIdx.x;
  // start from (-inf, the thread's first index), so a row of -inf gives its first index
  ValIdx best{-__builtin_inff(), INT_MAX};

  if (kVec) {
    const int nvec = V >> 2;
    best.i = tid < nvec ? tid << 2 : ((nvec << 2) + tid < V ? (nvec << 2) + tid : INT_MAX);
    const f32x4* p4 = reinterpret_cast<const f32x4*>(p);
    int c = tid;
    // main loop: kUnroll independent 16-byte loads in flight per thread
    for (; c + (kUnroll - 1) * kArgmaxThreads < nvec; c += kUnroll * kArgmaxThreads) {
      f32x4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(p4 + c + u * kArgmaxThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int base = (c + u * kArgmaxThreads) << 2;
        take_if_greater(best, x[u].x, base);
        take_if_greater(best, x[u].y, base + 1);
        take_if_greater(best, x[u].z, base + 2);
        take_if_greater(best, x[u].w, base + 3);
      }
    }
    for (; c < nvec; c += kArgmaxThreads) {
      const f32x4 x = p4[c];
      const int base = c << 2;
      take_if_greater(best, x.x, base);
      take_if_greater(best, x.y, base + 1);
      take_if_greater(best, x.z, base + 2);
      take_if_greater(best, x.w, base + 3);
    }
    for (int e = (nvec << 2) + tid; e < V; e += kArgmaxThreads) take_if_greater(best, p[e], e);
  } else {
    best.i = tid < V ? tid : INT_MAX;
    for (int e = tid; e < V; e += kArgmaxThreads) take_if_greater(best, p[e], e);
  }

  // wave reduction
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(best.v, off, 64);
    const int oi = __shfl_xor(best.i, off, 64);
    take_if_better(best, ov, oi);
  }
  __shared__ float s_v[kArgmaxThreads / 64];
  __shared__ int s_i[kArgmaxThreads / 64];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    s_v[wave] = best.v;
    s_i[wave] = best.i;
  }
  __syncthreads();
  if (tid == 0) {
    ValIdx r{s_v[0], s_i[0]};
    for (int w = 1; w < kArgmaxThreads / 64; ++w) take_if_better(r, s_v[w], s_i[w]);
    out[row] = r.i;
  }
}

__global__ void __launch_bounds__(256) accept_path_kernel(const int32_t* __restrict__ tokens,
                                                          const int32_t* __restrict__ parents,
                                                          const int32_t* __restrict__ tstar, int N,
                                                          int32_t* __restrict__ accept_len,
                                                          int32_t* __restrict__ accept_nodes,
                                                          int32_t* __restrict__ commit_tokens) {
  constexpr int kWords = 256 / 32;
  __shared__ int s_par[256];
  __shared__ int s_tok[256];
  __shared__ int s_ts[256];
  __shared__ uint32_t s_anc[256][kWords + 1];   // node's ancestors-or-self (padded row: no bank conflicts)
  __shared__ unsigned s_key;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)b * N;
  if (tid < N) {
    s_par[tid] = parents[base + tid];
    s_tok[tid] = tokens[base + tid];
    s_ts[tid] = tstar[base + tid];
  }
  if (tid == 0) s_key = 0u;
  __syncthreads();

  // One walk up the ancestor chain of node tid: is every draft token on its root
  // path equal to its parent's argmax, how deep is it, and which nodes are on it.
  int valid = 0, d = 0;
  uint32_t anc[kWords];
#pragma unroll
  for (int w = 0; w < kWords; ++w) anc[w] = 0u;
  if (tid < N) {
    valid = 1;
    int k = tid;
    while (true) {
#pragma unroll
      for (int w = 0; w < kWords; ++w) anc[w] |= (k >> 5) == w ? 1u << (k & 31) : 0u;
      if (k == 0 || d >= N) break;
      const int p = s_par[k];
      if (p < 0 || p >= k) {        // not a tree: reject (bounded walk either way)
        valid = 0;
        break;
      }
      if (s_tok[k] != s_ts[p]) valid = 0;
      k = p;
      ++d;
    }
#pragma unroll
    for (int w = 0; w < kWords; ++w) s_anc[tid][w] = anc[w];
    if (valid) atomicMax(&s_key, ((unsigned)d << 16) | (0xFFFFu - (unsigned)tid));
  }
  __syncthreads();
  const unsigned key = s_key;
  const int len = (int)(key >> 16);
  const int term = (int)(0xFFFFu - (key & 0xFFFFu));

  if (tid < N) {
    if (tid > len) {
      accept_nodes[base + tid] = -1;
      commit_tokens[base + tid] = -1;
    }
    // node tid is on the accepted path iff it is an ancestor-or-self of the terminal
    if ((s_anc[term][tid >> 5] >> (tid & 31)) & 1u) {
      accept_nodes[base + d] = tid;
      if (d >= 1) commit_tokens[base + d - 1] = s_tok[tid];
    }
  }
  if (tid == 0) {
    accept_len[b] = len;
    commit_tokens[base + len] = s_ts[term];
  }
}

}  // namespace

hipError_t launch_accept(const float* logits, int64_t ld_logits, const int32_t* tokens, const int32_t* parents, int B,
                         int N, int V, int32_t* target_argmax, int32_t* accept_len, int32_t* accept_nodes,
                         int32_t* commit_tokens, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const int rows = B * N;
  const bool vec = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (ld_logits % 4 == 0);
  if (vec)
    hipLaunchKernelGGL(argmax_kernel<true>, dim3(rows), dim3(kArgmaxThreads), 0, stream, logits, ld_logits, V,
                       target_argmax);
  else
    hipLaunchKernelGGL(argmax_kernel<false>, dim3(rows), dim3(kArgmaxThreads), 0, stream, logits, ld_logits, V,
                       target_argmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_path_kernel, dim3(B), dim3(256), 0, stream, tokens, parents, target_argmax, N, accept_len,
                     accept_nodes, commit_tokens);
  return hipGetLastError();
}

}  // namespace ddtree
