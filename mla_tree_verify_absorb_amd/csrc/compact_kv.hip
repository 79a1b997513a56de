// Post-verify KV-cache compaction: the accepted path's latent rows move into the
// cache, root first, at positions L_b .. L_b + accept_len.
//
// The engine keeps a KV cache with post-verify compaction, which carries the
// accepted tokens into the following steps (page "The Moment of Proof:
// Validating a Native CUDA Speculative Decoding Engine", section "Output
// Knowledge Created"; page "The Build That Proved It: Compiling the Native
// DDTree Speculative Decoding Engine", section "The Output Knowledge Created").
//
// One workgroup per request.  A path that fits in 64 KB is read whole into LDS
// and then written, so the move is safe in place (tree rows living in the
// cache right after the prefix, row dest + i holding node i).  A longer path
// is moved one row at a time in path order with a barrier between rows; that
// is safe in place too, because a path's node indices grow with depth, so
// row dest + k never holds a row that a later step still has to read.  Rows
// are copied in 16-byte pieces when the row, both base pointers and both
// strides allow it, else in 4- or 2-byte pieces (staged parts start on 16-byte
// boundaries, so every piece size stays aligned in LDS).
#include "../../include/ddtree.h"
#include "ddtree_internal.h"

namespace ddtree {
namespace {

template <typename U>
__device__ __forceinline__ void copy_row(unsigned char* dst, const unsigned char* src, int64_t bytes, int tid) {
  const int64_t n = bytes / (int64_t)sizeof(U);
  U* d = reinterpret_cast<U*>(dst);
  const U* s = reinterpret_cast<const U*>(src);
  for (int64_t e = tid; e < n; e += blockDim.x) d[e] = s[e];
}

__device__ __forceinline__ void copy_row_any(unsigned char* dst, const unsigned char* src, int64_t bytes, int unit,
                                             int tid) {
  if (bytes <= 0) return;
  if (unit == 16)
    copy_row<uint4>(dst, src, bytes, tid);
  else if (unit == 4)
    copy_row<uint32_t>(dst, src, bytes, tid);
  else
    copy_row<uint16_t>(dst, src, bytes, tid);
}

constexpr int kStageBytes = 64 * 1024;   // LDS staging for short paths

// Flat copy of part (latent or rotary) of rows 0..last between global rows and the
// LDS stage: every (row, piece) pair is one work item, so all loads are in flight
// at once.  to_stage: tree rows -> stage; else stage -> cache rows.
template <typename U>
__device__ __forceinline__ void stage_part(bool to_stage, unsigned char* stage, int64_t stage_row, int64_t stage_off,
                                           const unsigned char* tree, int64_t ld_tree, unsigned char* cache,
                                           int64_t ld_cache, int64_t d0, const int* nodes, int b, int N, int last,
                                           int64_t bytes, int tid) {
  const int64_t pieces = bytes / (int64_t)sizeof(U);
  const int64_t total = (int64_t)(last + 1) * pieces;
  for (int64_t idx = tid; idx < total; idx += blockDim.x) {
    const int k = (int)(idx / pieces);
    const int64_t p = idx - (int64_t)k * pieces;
    const int s = nodes[k];
    if (s < 0 || s >= N) continue;
    U* st = reinterpret_cast<U*>(stage + k * stage_row + stage_off) + p;
    if (to_stage)
      *st = reinterpret_cast<const U*>(tree + ((int64_t)b * N + s) * ld_tree)[p];
    else
      reinterpret_cast<U*>(cache + (d0 + k) * ld_cache)[p] = *st;
  }
}

__device__ __forceinline__ void stage_part_any(int unit, bool to_stage, unsigned char* stage, int64_t stage_row,
                                               int64_t stage_off, const unsigned char* tree, int64_t ld_tree,
                                               unsigned char* cache, int64_t ld_cache, int64_t d0, const int* nodes,
                                               int b, int N, int last, int64_t bytes, int tid) {
  if (bytes <= 0) return;
  if (unit == 16)
    stage_part<uint4>(to_stage, stage, stage_row, stage_off, tree, ld_tree, cache, ld_cache, d0, nodes, b, N, last,
                      bytes, tid);
  else if (unit == 4)
    stage_part<uint32_t>(to_stage, stage, stage_row, stage_off, tree, ld_tree, cache, ld_cache, d0, nodes, b, N,
                         last, bytes, tid);
  else
    stage_part<uint16_t>(to_stage, stage, stage_row, stage_off, tree, ld_tree, cache, ld_cache, d0, nodes, b, N,
                         last, bytes, tid);
}

__global__ void __launch_bounds__(256) compact_kv_kernel(CompactArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char stage[kStageBytes];
  __shared__ int s_nodes[DDTREE_MAX_NODES];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t d0 = a.dest_rows[b];
  if (d0 < 0) return;
  int last = a.accept_len[b];
  if (last > a.N - 1) last = a.N - 1;
  if (last < 0) return;
  for (int k = tid; k <= last; k += blockDim.x) s_nodes[k] = a.accept_nodes[(int64_t)b * a.N + k];
  __syncthreads();
  // staged rows: latent part, then rotary part, each padded to 16 bytes
  const int64_t c_pad = (a.c_bytes + 15) & ~int64_t(15);
  const int64_t row_bytes = c_pad + ((a.r_bytes + 15) & ~int64_t(15));
  if ((int64_t)(last + 1) * row_bytes <= kStageBytes) {
    // Short path: every row is read into LDS before any is written, so the move
    // is also safe in place; all loads, then all stores, are in flight together.
    stage_part_any(a.c_unit, true, stage, row_bytes, 0, a.ckv_tree, a.ld_ckv_tree, nullptr, 0, d0, s_nodes, b, a.N,
                   last, a.c_bytes, tid);
    stage_part_any(a.r_unit, true, stage, row_bytes, c_pad, a.krope_tree, a.ld_krope_tree, nullptr, 0, d0, s_nodes, b,
                   a.N, last, a.r_bytes, tid);
    __syncthreads();
    stage_part_any(a.c_unit, false, stage, row_bytes, 0, nullptr, 0, a.ckv, a.ld_ckv, d0, s_nodes, b, a.N, last,
                   a.c_bytes, tid);
    stage_part_any(a.r_unit, false, stage, row_bytes, c_pad, nullptr, 0, a.krope, a.ld_krope, d0, s_nodes, b, a.N,
                   last, a.r_bytes, tid);
    return;
  }
  // Long path: one row at a time in path order (see above for why this is safe in place).
  for (int k = 0; k <= last; ++k) {
    const int s = s_nodes[k];
    if (s >= 0 && s < a.N) {
      const int64_t tree_row = (int64_t)b * a.N + s;
      copy_row_any(a.ckv + (d0 + k) * a.ld_ckv, a.ckv_tree + tree_row * a.ld_ckv_tree, a.c_bytes, a.c_unit, tid);
      copy_row_any(a.krope + (d0 + k) * a.ld_krope, a.krope_tree + tree_row * a.ld_krope_tree, a.r_bytes, a.r_unit,
                   tid);
    }
    __syncthreads();   // row dest + k is complete before a later row is read
  }
}

}  // namespace

hipError_t launch_compact_kv(const CompactArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(compact_kv_kernel, dim3(a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ddtree
