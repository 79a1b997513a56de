// Visibility mask of a draft tree: ancestor-or-self bitmask, depth, positions.
//
// The mask is the custom attention mask under which the draft tree is
// verified in one forward (page "The Moment of Proof: Validating a Native CUDA
// Speculative Decoding Engine", sections "Input Knowledge Required" and
// "Output Knowledge Created"); positions are cache length + depth, int64
// (page "The Build That Proved It: Compiling the Native DDTree Speculative
// Decoding Engine", section "The Thinking Process Visible in Reasoning").
//
// One workgroup of 256 threads per request, one thread per node.  The parent
// array is validated first (root parent -1, every other parent an earlier
// node), so each thread's pointer chase strictly decreases and ends within
// N steps.  A thread builds its own mask row in LDS, then the block writes
// the rows out with coalesced stores.
#include "ddtree_internal.h"

namespace ddtree {
namespace {

constexpr int kMaxN = 256;
constexpr int kMaxW = kMaxN / 32;

__global__ void __launch_bounds__(256) build_mask_kernel(const int32_t* __restrict__ parents, int N,
                                                         const int64_t* __restrict__ prefix_offsets,
                                                         uint32_t* __restrict__ mask, int32_t* __restrict__ depth,
                                                         int64_t* __restrict__ positions,
                                                         int32_t* __restrict__ tree_ok) {
  __shared__ int32_t s_parent[kMaxN];
  __shared__ uint32_t s_mask[kMaxN][kMaxW + 1];   // +1 word of padding against bank conflicts
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int W = (N + 31) >> 5;

  int bad = 0;
  if (tid < N) {
    const int p = parents[(int64_t)b * N + tid];
    s_parent[tid] = p;
    bad = (tid == 0) ? (p != -1) : (p < 0 || p >= tid);
  }
  const int any_bad = __syncthreads_or(bad);

  int64_t L = 0;
  if (prefix_offsets != nullptr) L = prefix_offsets[b + 1] - prefix_offsets[b];

  int d = -1;
  if (tid < N) {
    for (int w = 0; w < W; ++w) s_mask[tid][w] = 0u;
    if (!any_bad) {
      int k = tid;
      int steps = 0;
      while (k >= 0 && steps <= tid) {       // parent[k] < k: at most tid + 1 visits
        s_mask[tid][k >> 5] |= 1u << (k & 31);
        k = s_parent[k];
        ++steps;
      }
      d = steps - 1;
    }
    depth[(int64_t)b * N + tid] = d;
    if (positions != nullptr) positions[(int64_t)b * N + tid] = any_bad ? (int64_t)-1 : L + d;
  }
  __syncthreads();
  // coalesced write of the N x W mask words of this request
  uint32_t* out = mask + (int64_t)b * N * W;
  for (int e = tid; e < N * W; e += blockDim.x) out[e] = s_mask[e / W][e % W];
  if (tid == 0) tree_ok[b] = any_bad ? 0 : 1;
}

}  // namespace

hipError_t launch_build_mask(const int32_t* parents, int B, int N, const int64_t* prefix_offsets, uint32_t* mask,
                             int32_t* depth, int64_t* positions, int32_t* tree_ok, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(build_mask_kernel, dim3(B), dim3(256), 0, stream, parents, N, prefix_offsets, mask, depth,
                     positions, tree_ok);
  return hipGetLastError();
}

}  // namespace ddtree
