// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ddtree {

// ---- launchers (each enqueues on `stream`, returns the launch's hipError_t) ----

hipError_t launch_build_mask(const int32_t* parents, int B, int N, const int64_t* prefix_offsets, uint32_t* mask,
                             int32_t* depth, int64_t* positions, int32_t* tree_ok, hipStream_t stream);

hipError_t launch_accept(const float* logits, int64_t ld_logits, const int32_t* tokens, const int32_t* parents, int B,
                         int N, int V, int32_t* target_argmax, int32_t* accept_len, int32_t* accept_nodes,
                         int32_t* commit_tokens, hipStream_t stream);

struct AttnArgs {
  int B, N, H, Dl, Dr;
  const void* q_lat;
  const void* q_rope;
  const void* ckv;
  int64_t ld_ckv;
  const void* krope;
  int64_t ld_krope;
  const int64_t* prefix_offsets;
  const void* ckv_tree;
  int64_t ld_ckv_tree;
  const void* krope_tree;
  int64_t ld_krope_tree;
  const uint32_t* mask;
  float scale;
  int splits;          // >= 1 (uniform schedule)
  int balanced;        // 1: band schedule (row blocks per request a multiple or a divisor of kBandRowBlocks)
  float* o;
  float* lse;
  // Partial records, one per row of a KV split or a band piece (MFMA kernel, Dl = 512):
  //   part_o   [records][Dl] fp16: the row's unnormalised output scaled by a power of two,
  //            in the chunk order of partial_chunk_dim (verify_attn_bf16.hip)
  //   part_aux [records] {lse2, k}, log2 units: the record adds 2^lse2 to the merged
  //            exp-sum and 2^k times its fp16 values to the merged numerator
  // uniform schedule, splits > 1: [splits][B*N*H] records; band schedule: [slots][kRowsPerBlock]
  // with slots = 2 * band_windows * (row blocks per band)
  void* part_o;
  float2* part_aux;
  int* band_edges;     // band schedule: [band_windows][4] (after part_aux): [0] the total column
                       // count (int64) and the window count, [e] edge e's cut descriptor
  int band_windows;    // band schedule: most windows (host bound from the longest prefix; the
                       // kernel uses fewer when the columns run short)
};

// bf16 MFMA kernel for (Dl, Dr) = (512, 64)
constexpr int kMfmaDl = 512;
constexpr int kMfmaDr = 64;
constexpr int kRowsPerBlock = 128;   // query rows (node, head) per workgroup
constexpr int kKeysPerTile = 32;     // latent KV rows per LDS tile
// Band schedule: R row blocks of one request form a band (R = 32, one per CU of
// an XCD, when a request has a multiple of 32 row blocks; R = all of them when
// that count divides 32).  The bands' KV tile columns are cut into at most 256 / R
// equal windows, 32 / R per XCD, and each workgroup of a window keeps at most one
// piece at each window edge.
constexpr int kBandRowBlocks = 32;
constexpr int kBandXcds = 8;
constexpr int kBandWorkgroups = kBandXcds * kBandRowBlocks;   // 256, one per CU
constexpr int kBandMinWindowColumns = 8;   // fewest KV tile columns in a window
constexpr int64_t kMaxBf16RowStride = int64_t(1) << 24;   // elements; keeps tile row offsets in 32 bits
constexpr int kPartialRecordBytes = kMfmaDl * 2 + 8;       // fp16 values + {lse2, k}

// KV-cache compaction (byte addressing; strides in bytes)
struct CompactArgs {
  int B, N;
  const unsigned char* ckv_tree;
  int64_t ld_ckv_tree;
  const unsigned char* krope_tree;
  int64_t ld_krope_tree;
  const int32_t* accept_len;
  const int32_t* accept_nodes;
  unsigned char* ckv;
  int64_t ld_ckv;
  unsigned char* krope;
  int64_t ld_krope;
  const int64_t* dest_rows;
  int64_t c_bytes, r_bytes;   // bytes per latent / rotary row
  int c_unit, r_unit;         // copy piece: 16, 4 or 2 bytes
};

hipError_t launch_verify_attn_bf16(const AttnArgs& a, hipStream_t stream);
// fp32 arithmetic for fp32 or bf16 inputs, any Dl <= 512, Dr <= 512
hipError_t launch_verify_attn_generic(const AttnArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_compact_kv(const CompactArgs& a, hipStream_t stream);
// NeoX rotary embedding at tree positions
constexpr int kMaxRopeDim = 512;
struct RopeArgs {
  int B, N, H, Dr;
  bool bf16;
  void* q_rope;              // [B, N, H, Dr] dense, or null
  void* krope_tree;          // rows (b, i) at krope_tree + (b*N + i) * ld_krope_tree, or null
  int64_t ld_krope_tree;     // elements
  const int64_t* positions;  // [B, N]
  const double* inv_freq;    // [Dr / 2]
};
hipError_t launch_rope_tree(const RopeArgs& a, hipStream_t stream);
hipError_t launch_build_tree(int B, int N, int D, int K, const int32_t* root_tokens, const int32_t* cand_tokens,
                             const float* cand_logp, int32_t* parents, int32_t* tokens, int32_t* depth, float* scores,
                             hipStream_t stream);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_band_combine(const AttnArgs& a, hipStream_t stream);

}  // namespace ddtree
