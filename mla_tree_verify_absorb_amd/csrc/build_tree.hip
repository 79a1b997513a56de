// Best-first draft-tree builder on the GPU.
//
// The engine builds the draft tree on the GPU best-first, in place of a
// per-request CPU heap (page "The Moment of Proof: Validating a Native CUDA
// Speculative Decoding Engine", opening and section "Output Knowledge
// Created").  Depth d (1..D) offers K proposals (token, log-probability),
// non-increasing along K; any node at depth d-1 may take any of them as a
// child, with score = parent score + log-probability (float32, root 0).  Nodes
// are taken in order of the key (score descending, then depth, parent index,
// proposal rank ascending) until N exist; taking node (p, d, j) puts its next
// sibling (p, d, j+1) and its first child (new node, d+1, 0) on the frontier.
//
// One 64-thread workgroup (a single wave) per request.  The frontier lives in
// LDS as 64-bit keys, larger = better: the score's order-preserving bit
// pattern above 24 bits of (depth, parent, rank), inverted so that smaller
// tuples rank higher.  Each step is a wave-wide max over the frontier (DPP
// within 16-lane rows, then readlane); the key itself carries the taken
// node's depth, parent and rank.  Slots are appended and never reused (at
// most 2N - 1).  Tokens are looked up once, after the loop.
#include <cmath>

#include "../../include/ddtree.h"
#include "ddtree_internal.h"

namespace ddtree {
namespace {

constexpr int kSlots = 2 * DDTREE_MAX_NODES;

__device__ __forceinline__ uint32_t score_code(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);   // -0 -> +0, so equal scores get equal codes
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float code_score(uint32_t c) {
  return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

__device__ __forceinline__ uint64_t make_key(float s, int d, int p, int j) {
  const uint32_t tie = 0xFFFFFFu - (((uint32_t)d << 16) | ((uint32_t)p << 8) | (uint32_t)j);
  return ((uint64_t)score_code(s) << 32) | tie;
}


// Max over the wave's 64 lanes of a 64-bit value: DPP row shifts within each 16-lane
// row, then the four row maxima through readlane (scalar compares).
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  // lanes whose source is outside the row keep their own value (bound_ctrl off, old = v)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0x111>(v));   // row_shr:1
  v = max_u64(v, dpp_u64<0x112>(v));   // row_shr:2
  v = max_u64(v, dpp_u64<0x114>(v));   // row_shr:4
  v = max_u64(v, dpp_u64<0x118>(v));   // row_shr:8 -> lane 15 of each row holds the row's max
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r + 15);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r + 15);
    m = max_u64(m, ((uint64_t)hi << 32) | lo);
  }
  return m;
}

__global__ void __launch_bounds__(64) build_tree_kernel(int N, int D, int K, const int32_t* __restrict__ root_tokens,
                                                         const int32_t* __restrict__ cand_tokens,
                                                         const float* __restrict__ cand_logp, int32_t* parents,
                                                         int32_t* tokens, int32_t* depth, float* scores) {
  __shared__ float s_logp[DDTREE_MAX_DEPTH * DDTREE_MAX_PROPOSALS];
  __shared__ uint64_t s_key[kSlots];
  __shared__ float s_score[DDTREE_MAX_NODES];
  __shared__ int s_par[DDTREE_MAX_NODES], s_rank[DDTREE_MAX_NODES], s_dep[DDTREE_MAX_NODES];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t cbase = (int64_t)b * D * K;
  for (int e = lane; e < D * K; e += 64) s_logp[e] = cand_logp[cbase + e];
  for (int e = lane; e < kSlots; e += 64) s_key[e] = 0ull;   // 0 = empty (every real key is larger)
  if (lane == 0) {
    s_score[0] = 0.f;
    s_par[0] = -1;
    s_rank[0] = 0;
    s_dep[0] = 0;
  }
  __syncthreads();
  if (lane == 0) s_key[0] = make_key(0.f + s_logp[0], 1, 0, 0);
  int count = 1;   // slots used (uniform)
  __syncthreads();

  for (int n = 1; n < N; ++n) {
    // every slot past `count` holds 0, so the lane reads all of its slots at once
    // (independent LDS reads, one round trip) instead of looping up to `count`
    uint64_t keys[kSlots / 64];
#pragma unroll
    for (int i = 0; i < kSlots / 64; ++i) keys[i] = s_key[lane + 64 * i];
    uint64_t mine = 0ull;
    int mine_slot = -1;
#pragma unroll
    for (int i = 0; i < kSlots / 64; ++i) {
      if (keys[i] > mine) {
        mine = keys[i];
        mine_slot = lane + 64 * i;
      }
    }
    // best > 0: the frontier cannot run dry before N nodes (the host checks the candidate tree's size)
    const uint64_t best = wave_max_u64(mine);
    const uint32_t tie = 0xFFFFFFu - (uint32_t)(best & 0xFFFFFFu);
    const int d = (int)(tie >> 16), p = (int)((tie >> 8) & 0xFFu), j = (int)(tie & 0xFFu);
    const float s = code_score((uint32_t)(best >> 32));
    if (mine_slot >= 0 && mine == best) s_key[mine_slot] = 0ull;   // keys are unique: one lane owns it
    if (lane == 0) {
      s_score[n] = s;
      s_par[n] = p;
      s_rank[n] = j;
      s_dep[n] = d;
      // the next sibling (same parent) and the first child join the frontier
      int c = count;
      if (j + 1 < K) s_key[c++] = make_key(s_score[p] + s_logp[(d - 1) * K + j + 1], d, p, j + 1);
      if (d < D) s_key[c++] = make_key(s + s_logp[d * K], d + 1, n, 0);
    }
    count += (j + 1 < K) + (d < D);
    __syncthreads();
  }
  const int64_t obase = (int64_t)b * N;
  for (int i = lane; i < N; i += 64) {
    parents[obase + i] = s_par[i];
    tokens[obase + i] = i == 0 ? root_tokens[b] : cand_tokens[cbase + (int64_t)(s_dep[i] - 1) * K + s_rank[i]];
    if (depth) depth[obase + i] = s_dep[i];
    if (scores) scores[obase + i] = s_score[i];
  }
}

}  // namespace

hipError_t launch_build_tree(int B, int N, int D, int K, const int32_t* root_tokens, const int32_t* cand_tokens,
                             const float* cand_logp, int32_t* parents, int32_t* tokens, int32_t* depth, float* scores,
                             hipStream_t stream) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(build_tree_kernel, dim3(B), dim3(64), 0, stream, N, D, K, root_tokens, cand_tokens, cand_logp,
                     parents, tokens, depth, scores);
  return hipGetLastError();
}

}  // namespace ddtree
