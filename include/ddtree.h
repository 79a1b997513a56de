/*
 * ddtree.h -- C ABI of the MI355X (gfx950) DDTree tree-verify library.
 *
 * The library implements the data-parallel hot path of verifying a draft
 * tree in one target forward: the visibility mask built from a parent array,
 * the tree-verify MLA attention in absorbed form over the shared latent KV
 * cache prefix plus each node's own ancestors, and the greedy tree accept.
 *
 * Pages cited (titles of the source pages):
 *   [Validating] "The Moment of Proof: Validating a Native CUDA Speculative Decoding Engine"
 *   [Running]    "The Moment of Proof: Running the Native DDTree Speculative Decoding Engine"
 *   [Build]      "The Build That Proved It: Compiling the Native DDTree Speculative Decoding Engine"
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device memory owned by the caller; the
 *     library allocates nothing, keeps no state between calls and is safe to
 *     call from several host threads (the one exception is the per-GPU scratch
 *     of ddtree_verify_attn_noalloc, described there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns; nothing synchronises.
 *   - Arrays are dense row-major (C order) unless a leading dimension (ld_*,
 *     in elements) is given for their rows.
 *   - The return value is a ddtree_status.  Arguments are validated on the
 *     host before anything is enqueued; an invalid call enqueues nothing.
 *     DDTREE_ERR_HIP reports a failed launch (hipGetLastError).  Problems that
 *     depend on device data (a malformed tree) are reported on the device
 *     through tree_ok.
 *   - Outputs must not overlap inputs or each other (checked where the
 *     extents are known on the host); a buffer whose extent runs past the top
 *     of the address space is DDTREE_ERR_INVALID_ARG.
 *   - Row strides (ld_*) and max_prefix_len above DDTREE_MAX_EXTENT are
 *     DDTREE_ERR_UNSUPPORTED, so that every extent the host computes fits in
 *     64 bits.
 *   - Tree layout: node 0 is the root (the last committed token), parent[0] =
 *     -1 and 0 <= parent[i] < i for i >= 1; at most DDTREE_MAX_NODES nodes.
 */
#ifndef DDTREE_H
#define DDTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDTREE_MAX_NODES 256
#define DDTREE_MAX_DEPTH 64      /* draft depths offered to ddtree_build_tree */
#define DDTREE_MAX_PROPOSALS 64  /* proposals per depth for ddtree_build_tree */
#define DDTREE_MAX_EXTENT ((int64_t)1 << 40) /* largest row stride (elements) and prefix length (rows) */

typedef enum {
  DDTREE_OK = 0,
  DDTREE_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment or overlapping buffers */
  DDTREE_ERR_UNSUPPORTED = -2, /* shape or dtype outside what the kernels implement */
  DDTREE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than ddtree_verify_attn_workspace_size */
  DDTREE_ERR_HIP = -4          /* the HIP runtime reported an error for a launch */
} ddtree_status;

typedef enum {
  DDTREE_F32 = 0,  /* float32 inputs, float32 arithmetic */
  DDTREE_BF16 = 1  /* bfloat16 inputs, bf16 MFMA products with float32 accumulation */
} ddtree_dtype;

/* Human-readable name of a status code (static storage). */
const char* ddtree_status_string(int status);

/* Digest of the sources and flags the library was built from (16 hex digits,
 * static storage): the binding compares it with the sources it ships with and
 * refuses a library built from other sources. */
const char* ddtree_build_digest(void);

/*
 * ddtree_build_mask -- ancestor-or-self visibility mask, depth and positions.
 *
 * Defines the custom attention mask under which a draft tree is verified in
 * one forward ([Validating] "Input Knowledge Required"; attention mask
 * construction in the decode loop: [Validating] "Output Knowledge Created"),
 * and positions = cache length + node depth as int64 ([Build] "The Thinking
 * Process Visible in Reasoning").
 *
 *   parents        device int32 [B, N]       parent array per request
 *   B, N           requests (>= 0) and nodes per request (1 .. DDTREE_MAX_NODES)
 *   prefix_offsets device int64 [B + 1] or NULL; L_b = offsets[b+1] - offsets[b]
 *                  (NULL: L_b = 0)
 *   mask           device uint32 [B, N, W], W = ceil(N / 32): bit k % 32 of word
 *                  k / 32 of row (b, i) is set iff node k is node i or one of
 *                  its ancestors
 *   depth          device int32 [B, N]       parent steps from node i to the root
 *   positions      device int64 [B, N] or NULL: L_b + depth
 *   tree_ok        device int32 [B]          1 if request b's parent array is a
 *                  valid tree, else 0; then its mask row words are 0 and its
 *                  depth and positions are -1
 */
int ddtree_build_mask(const int32_t* parents, int32_t B, int32_t N, const int64_t* prefix_offsets,
                      uint32_t* mask, int32_t* depth, int64_t* positions, int32_t* tree_ok, void* stream);

/*
 * ddtree_verify_attn -- tree-verify attention, MLA absorbed form.
 *
 * Every tree node's absorbed query attends to its request's cached latent
 * prefix plus the tree nodes its mask row makes visible ([Validating] "Input
 * Knowledge Required": the absorb form folds the key/value up-projections
 * into attention, and the draft tree is verified under a custom mask;
 * [Running] "Input Knowledge Required": verify attention with visibility
 * masking).  For request b, node i, head h and visible key j with latent row
 * c_j (Dl wide) and rotary key r_j (Dr wide, already rotated):
 *     s_j = softmax_scale * (q_lat[b,i,h] . c_j + q_rope[b,i,h] . r_j)
 *     o[b,i,h]   = sum_j softmax(s)_j * c_j   (latent output; the caller applies
 *                                              the value up-projection)
 *     lse[b,i,h] = ln sum_j exp(s_j)
 *
 *   dtype            DDTREE_BF16 at (Dl, Dr) = (512, 64): the MFMA kernel;
 *                    DDTREE_F32, and DDTREE_BF16 at other dims: the generic
 *                    kernel (float32 arithmetic), any Dl in 1..512, Dr in 0..512
 *   B, N, H          requests, nodes per request (<= DDTREE_MAX_NODES), heads
 *   q_lat            device [B, N, H, Dl], dense
 *   q_rope           device [B, N, H, Dr], dense
 *   ckv, ld_ckv      device packed prefix latent rows: row t at ckv + t*ld_ckv
 *   krope, ld_krope  device packed prefix rotary keys: row t at krope + t*ld_krope
 *                    (the usual fused cache [T, Dl+Dr] is krope = ckv + Dl, both
 *                    ld = Dl + Dr)
 *   prefix_offsets   device int64 [B + 1]: request b owns rows offsets[b] ..
 *                    offsets[b+1]-1 (lengths may be 0); the MFMA kernel indexes
 *                    rows with 32 bits, so offsets[B] < 2^32 (any cache that fits
 *                    in device memory: a latent row alone is 1 KB there)
 *   max_prefix_len   host value >= every L_b; only used to plan the KV split
 *   ckv_tree, ld_ckv_tree      device tree-node latent rows: node (b,i) at
 *                              ckv_tree + (b*N + i)*ld_ckv_tree
 *   krope_tree, ld_krope_tree  device tree-node rotary keys, same indexing
 *   mask             device uint32 [B, N, ceil(N/32)] from ddtree_build_mask
 *   softmax_scale    finite scale applied to q.k (e.g. 1/sqrt(qk head dim))
 *   num_splits       0 = automatic schedule; S > 0 = S uniform KV splits per
 *                    block of 128 query rows (flash-decoding).  Automatic: when
 *                    n_rb = ceil(N*H/128) is a multiple of 32 or divides 32,
 *                    the band schedule: a request's 128-row blocks are grouped
 *                    R at a time (R = 32, or R = n_rb), the groups' KV tiles
 *                    laid end to end and cut into at most 256/R equal ranges
 *                    of at least 8 tiles, R workgroups each, so that every CU
 *                    carries the same work however ragged the prefix lengths;
 *                    otherwise uniform splits (ddtree_verify_attn_auto_splits).
 *                    MFMA kernel only; the generic kernel ignores it.
 *   o                device float32 [B, N, H, Dl]
 *   lse              device float32 [B, N, H] (natural log)
 *   workspace        device scratch of workspace_bytes >=
 *                    ddtree_verify_attn_workspace_size(...) with the same shape,
 *                    max_prefix_len and num_splits (may be NULL when that size
 *                    is 0).  It holds one record per row of a split or band
 *                    piece: the row's output in fp16 under a power-of-two
 *                    scale plus two floats, 2*Dl + 8 bytes.  S splits take
 *                    S*B*N*H records, the band schedule 2*W*R*128 records plus
 *                    16*W bytes, with R row blocks per band and W <= 256/R
 *                    windows bounded from B, N, H and max_prefix_len (at most
 *                    67.6 MB for Dl 512; 4.2 MB for one 16-node, 8-head
 *                    request of 4096 tokens)
 * Outputs (o, lse, workspace) must not overlap the inputs, including the first
 * max_prefix_len rows at ckv and krope (checked; the host knows no more of the
 * cache's extent).
 * bf16 inputs on the MFMA kernel need 16-byte aligned base pointers and row
 * strides that are multiples of 8 elements (INVALID_ARG otherwise) and at most
 * 2^24 elements (UNSUPPORTED otherwise); on the generic kernel, 2-byte aligned
 * pointers.  B*N*H above INT32_MAX/4 and num_splits above 1024 are UNSUPPORTED.
 * Requests whose tree_ok is 0 give undefined o/lse.
 * The two sizing queries take any arguments: for a shape the call would refuse
 * they return 0 (workspace bytes) and 1 (split count).
 */
size_t ddtree_verify_attn_workspace_size(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                                         int64_t max_prefix_len, int32_t num_splits);

/* What num_splits = 0 selects for this shape: 0 for the band schedule, else the
 * uniform KV split count (>= 1). */
int32_t ddtree_verify_attn_auto_splits(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                                       int64_t max_prefix_len);

int ddtree_verify_attn(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                       const void* q_lat, const void* q_rope,
                       const void* ckv, int64_t ld_ckv, const void* krope, int64_t ld_krope,
                       const int64_t* prefix_offsets, int64_t max_prefix_len,
                       const void* ckv_tree, int64_t ld_ckv_tree, const void* krope_tree, int64_t ld_krope_tree,
                       const uint32_t* mask, float softmax_scale, int32_t num_splits,
                       float* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ddtree_verify_attn_noalloc -- ddtree_verify_attn that allocates nothing and
 * takes no workspace.
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results and errors are those of ddtree_verify_attn
 * (same kernels), without workspace / workspace_bytes.  The split partials live
 * in one device array inside the library, DDTREE_NOALLOC_SCRATCH_BYTES (72 MiB)
 * per GPU, held by every GPU the library runs on until the process ends (its
 * address is looked up once per device on the first call there).
 *   - A call whose ddtree_verify_attn_workspace_size(...) exceeds the scratch
 *     returns DDTREE_ERR_WORKSPACE and enqueues nothing (use ddtree_verify_attn
 *     with a workspace then).  The band schedule needs at most 67.6 MB, so
 *     it always fits; explicit split counts above 17 at 64 nodes x 64 heads do
 *     not.
 *   - Every call on a GPU shares that GPU's scratch, which keeps the last
 *     call's contents; nothing in it needs clearing (each call writes every
 *     byte it reads).  Calls that overlap on one GPU (on different streams, or
 *     from several host threads without ordering) race on it.
 *   - DDTREE_ERR_HIP also reports a failed lookup of the scratch's address.
 */
#define DDTREE_NOALLOC_SCRATCH_BYTES (72ull << 20)

int ddtree_verify_attn_noalloc(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                               const void* q_lat, const void* q_rope,
                               const void* ckv, int64_t ld_ckv, const void* krope, int64_t ld_krope,
                               const int64_t* prefix_offsets, int64_t max_prefix_len,
                               const void* ckv_tree, int64_t ld_ckv_tree, const void* krope_tree,
                               int64_t ld_krope_tree, const uint32_t* mask, float softmax_scale, int32_t num_splits,
                               float* o, float* lse, void* stream);

/*
 * ddtree_greedy_accept -- target argmax per node and the accepted path.
 *
 * The tokens along the longest root path whose draft tokens match the
 * target's greedy choices are accepted ([Validating] "Input Knowledge
 * Required"; [Running] "Input Knowledge Required": greedy token acceptance
 * and path selection; [Build] "The Output Knowledge Created": the longest
 * prefix matching the target's greedy choices).  Node i (i >= 1) is accepted
 * when its parent is accepted and tokens[b,i] == target_argmax[b,parent[i]];
 * the root is always accepted.  The accepted node of greatest depth is the
 * terminal (ties: smallest index).  Commit = the draft tokens of the path
 * after the root, then target_argmax of the terminal (the bonus token).
 *
 *   logits, ld_logits  device float32 rows [B*N] of V logits, row (b,i) at
 *                      logits + (b*N + i)*ld_logits (ld_logits >= V)
 *   tokens             device int32 [B, N] draft token per node (root unused)
 *   parents            device int32 [B, N] valid trees (ddtree_build_mask's tree_ok)
 *   B, N, V            requests, nodes (1 .. DDTREE_MAX_NODES), vocabulary (>= 1)
 *   target_argmax      device int32 [B, N]: first index of each row's maximum
 *                      (NaN logits are not supported)
 *   accept_len         device int32 [B]: accepted draft tokens (terminal depth)
 *   accept_nodes       device int32 [B, N]: path root..terminal, then -1
 *   commit_tokens      device int32 [B, N]: accept_len + 1 tokens, then -1
 */
int ddtree_greedy_accept(const float* logits, int64_t ld_logits, const int32_t* tokens, const int32_t* parents,
                         int32_t B, int32_t N, int32_t V, int32_t* target_argmax, int32_t* accept_len,
                         int32_t* accept_nodes, int32_t* commit_tokens, void* stream);

/*
 * ddtree_compact_kv -- move the accepted path's latent rows into the cache.
 *
 * After verification the engine compacts its KV cache so that the accepted
 * tokens carry into the following steps ([Validating] "Output Knowledge
 * Created": KV cache with post-verify compaction; [Build] "The Output
 * Knowledge Created").  The root (the last committed token) and the accepted
 * drafts become cache positions L_b .. L_b + accept_len[b]: for k = 0 ..
 * accept_len[b], cache row dest_rows[b] + k receives tree row
 * accept_nodes[b, k] (both the latent and the rotary part).  The bonus token
 * has no latent row yet; it is the next step's root.
 *
 * Rows are moved one at a time in path order.  Because node indices grow
 * along a path, the call is also correct in place, when node (b, i)'s tree
 * row is cache row dest_rows[b] + i: for example one call per request with
 * ckv_tree (krope_tree) pointing at the cache row of position L_b and
 * ld_ckv_tree = ld_ckv (ld_krope_tree = ld_krope).
 *
 *   dtype            DDTREE_F32 or DDTREE_BF16 (rows are copied bit for bit)
 *   B, N, Dl, Dr     requests, nodes per request (1 .. DDTREE_MAX_NODES), latent
 *                    and rotary widths (Dl >= 1, Dr >= 0)
 *   ckv_tree, krope_tree, ld_*_tree  device tree rows, node (b,i) at
 *                    ckv_tree + (b*N + i)*ld_ckv_tree (as in ddtree_verify_attn)
 *   accept_len       device int32 [B] from ddtree_greedy_accept (clamped to N-1)
 *   accept_nodes     device int32 [B, N] from ddtree_greedy_accept; entries
 *                    outside 0..N-1 are skipped
 *   dest_rows        device int64 [B]: cache row of position L_b of request b
 *                    (negative: request skipped)
 *   ckv, ld_ckv, krope, ld_krope  device cache rows, updated in place; the
 *                    caller provides room for accept_len + 1 rows per request
 * Pointers must be aligned to the element size.  The tree rows must not
 * overlap accept_len, accept_nodes or dest_rows (checked); the cache rows
 * written must not overlap them either (not checkable on the host).
 */
int ddtree_compact_kv(int32_t dtype, int32_t B, int32_t N, int32_t Dl, int32_t Dr, const void* ckv_tree,
                      int64_t ld_ckv_tree, const void* krope_tree, int64_t ld_krope_tree, const int32_t* accept_len,
                      const int32_t* accept_nodes, const int64_t* dest_rows, void* ckv, int64_t ld_ckv, void* krope,
                      int64_t ld_krope, void* stream);

/*
 * ddtree_build_tree -- grow each request's draft tree best-first on the GPU.
 *
 * The engine builds its draft trees on the GPU best-first, in place of a
 * per-request CPU heap ([Validating] opening and "Output Knowledge Created").
 * The pages give no further detail; the reading implemented here: depth d
 * (1..D) offers K proposals (token, log-probability), the log-probabilities
 * non-increasing along K.  Any node at depth d-1 may take any depth-d
 * proposal as a child; a node's score is its parent's score plus the
 * proposal's log-probability (float32 additions, root to leaf; the root scores
 * 0).  Nodes are taken in order of the key (score descending, then depth,
 * parent index, proposal rank ascending) until N nodes exist and are numbered
 * in that order, so parents precede children and the output is a valid tree
 * for ddtree_build_mask.  With log-probabilities <= 0 the result is the root
 * plus the N-1 best nodes of the whole candidate tree under that key.  The
 * ordering along K is a precondition (the kernel offers a node's proposals to
 * the frontier one rank at a time): with proposals out of order the result is
 * still a valid tree of N nodes, but not necessarily the best-first one.
 *
 *   B, N             requests (>= 0), nodes per tree (1 .. DDTREE_MAX_NODES)
 *   D, K             draft depths (1 .. DDTREE_MAX_DEPTH) and proposals per depth
 *                    (1 .. DDTREE_MAX_PROPOSALS); N must not exceed the candidate
 *                    tree's size 1 + K + K^2 + ... + K^D (UNSUPPORTED otherwise)
 *   root_tokens      device int32 [B]: node 0's token (the last committed token)
 *   cand_tokens      device int32 [B, D, K]: proposal tokens of depth d+1 at [b, d]
 *   cand_logp        device float32 [B, D, K]: their log-probabilities (NaN: undefined)
 *   parents, tokens  device int32 [B, N]: the tree (parent[0] = -1)
 *   depth            device int32 [B, N] or NULL
 *   scores           device float32 [B, N] or NULL: each node's score
 * Outputs must not overlap inputs or each other (checked).
 */
int ddtree_build_tree(int32_t B, int32_t N, int32_t D, int32_t K, const int32_t* root_tokens,
                      const int32_t* cand_tokens, const float* cand_logp, int32_t* parents, int32_t* tokens,
                      int32_t* depth, float* scores, void* stream);

/*
 * ddtree_rope_tree -- NeoX rotary embedding of the tree nodes at their positions.
 *
 * Rotates, in place, each tree node's rotary queries (all heads) and its
 * rotary key row at the node's position, cache length + depth as produced by
 * ddtree_build_mask ([Truth] "What the Output Tells Us": NeoX rotary
 * embeddings with the angle computed in double; [Build] "The Thinking Process
 * Visible in Reasoning": int64 positions).  Element i pairs with element
 * i + Dr/2; angle a_i = position * inv_freq[i] in float64;
 *   out[i] = x[i] cos a_i - x[i+Dr/2] sin a_i,
 *   out[i+Dr/2] = x[i+Dr/2] cos a_i + x[i] sin a_i,
 * computed in float64 and rounded once to the storage type.  Run it before
 * ddtree_verify_attn, whose rotary inputs are taken as already rotated.
 *
 *   dtype            DDTREE_F32 or DDTREE_BF16 (storage type of both arrays)
 *   B, N, H, Dr      requests, nodes (1 .. DDTREE_MAX_NODES), heads, rotary width
 *                    (even, 2 .. 512)
 *   q_rope           device [B, N, H, Dr] dense, rotated in place, or NULL
 *   krope_tree, ld_krope_tree  device rows (b, i) at krope_tree + (b*N + i)*ld,
 *                    rotated in place, or NULL
 *   positions        device int64 [B, N]
 *   inv_freq         device float64 [Dr/2]: the rotary frequencies (any scaling
 *                    of them is the caller's)
 * The rotated arrays must not overlap positions or inv_freq (checked).
 */
int ddtree_rope_tree(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dr, void* q_rope, void* krope_tree,
                     int64_t ld_krope_tree, const int64_t* positions, const double* inv_freq, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DDTREE_H */
