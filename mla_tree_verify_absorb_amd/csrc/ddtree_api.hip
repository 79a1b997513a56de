// C ABI entry points: host-side argument validation, KV split planning and
// kernel launches.  Every check runs before the first HIP call, so an invalid
// call enqueues nothing (and can be tested on a machine without a GPU).
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/ddtree.h"
#include "ddtree_internal.h"

using namespace ddtree;

namespace {

// Byte extents are computed with overflow checks: kBadExtent stands for one that
// does not fit in 64 bits, and a buffer whose extent is bad or runs past the top
// of the address space is rejected like an overlap.
constexpr uint64_t kBadExtent = UINT64_MAX;

uint64_t mul_ext(uint64_t a, uint64_t b) {
  uint64_t r;
  return __builtin_mul_overflow(a, b, &r) ? kBadExtent : r;
}

uint64_t add_ext(uint64_t a, uint64_t b) {
  uint64_t r;
  return __builtin_add_overflow(a, b, &r) ? kBadExtent : r;
}

// Bytes spanned by `rows` rows of `width` elements of `es` bytes, `ld` elements apart.
uint64_t rows_bytes(uint64_t rows, uint64_t ld, uint64_t width, uint64_t es) {
  if (rows == 0 || width == 0) return 0;
  return mul_ext(add_ext(mul_ext(rows - 1, ld), width), es);
}

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
  bool bad;           // the extent does not fit the address space
};

Range range_of(const void* p, uint64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  uintptr_t hi;
  const bool bad = bytes == kBadExtent || __builtin_add_overflow(lo, bytes, &hi);
  return bad ? Range{lo, lo, true} : Range{lo, hi, false};
}

bool overlaps(Range a, Range b) {
  if (a.bad || b.bad) return true;
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool any_overlap(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_in; ++i)
    if (ins[i].bad) return true;
  for (int i = 0; i < n_out; ++i) {
    if (outs[i].bad) return true;
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned_to(const void* p, unsigned n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1u)) == 0; }

// Largest copy piece (16, 4 or 2 bytes) that divides the row and both rows' addresses.
int copy_unit(const void* a, int64_t lda_bytes, const void* b, int64_t ldb_bytes, int64_t row_bytes) {
  const unsigned units[] = {16u, 4u};
  for (unsigned u : units)
    if (row_bytes % u == 0 && lda_bytes % u == 0 && ldb_bytes % u == 0 && aligned_to(a, u) && aligned_to(b, u))
      return (int)u;
  return 2;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// bf16 at (Dl, Dr) = (512, 64) runs on the MFMA kernel; every other supported
// case (fp32, bf16 at other dims) on the generic kernel, which never splits.
bool mfma_path(int dtype, int Dl, int Dr) { return dtype == DDTREE_BF16 && Dl == kMfmaDl && Dr == kMfmaDr; }

// KV splits per query block: enough workgroups to cover the 256 CUs once,
// while every split keeps at least 4 KV tiles (128 keys).
int auto_splits(bool mfma, int B, int N, int H, int64_t max_prefix_len) {
  if (!mfma || B <= 0 || N <= 0 || H <= 0) return 1;
  const int64_t n_rb = ceil_div((int64_t)N * H, kRowsPerBlock);
  const int64_t wg = (int64_t)B * n_rb;
  int64_t s = wg >= 256 ? 1 : ceil_div(256, wg);
  const int64_t max_tiles = ceil_div(max_prefix_len > 0 ? max_prefix_len : 0, kKeysPerTile) + ceil_div(N, kKeysPerTile);
  const int64_t cap = max_tiles / 4 > 1 ? max_tiles / 4 : 1;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

// The automatic schedule is the band schedule whenever a request's row blocks
// come in whole bands of kBandRowBlocks or divide it; 0 stands for it.
bool band_schedule_applies(bool mfma, int N, int H) {
  const int64_t n_rb = ceil_div((int64_t)N * H, kRowsPerBlock);
  return mfma && n_rb > 0 && (n_rb % kBandRowBlocks == 0 || kBandRowBlocks % n_rb == 0);
}

// Most windows the band schedule may use: 256 / R, fewer when even requests of
// max_prefix_len tokens leave under kBandMinWindowColumns columns a window.  The
// kernel takes the smaller of this and its own count from the true lengths, so
// a max_prefix_len below a true length costs balance, never correctness.
int band_windows_bound(int B, int N, int H, int64_t max_prefix_len) {
  const int64_t n_rb = ceil_div((int64_t)N * H, kRowsPerBlock);
  const int64_t rbb = n_rb % kBandRowBlocks == 0 ? kBandRowBlocks : n_rb;
  const int64_t per_band = ceil_div(max_prefix_len, kKeysPerTile) + ceil_div(N, kKeysPerTile);
  int64_t cols;
  if (__builtin_mul_overflow((int64_t)B * (n_rb / rbb), per_band, &cols)) cols = INT64_MAX;
  const int64_t w = cols / kBandMinWindowColumns;
  const int64_t most = kBandWorkgroups / rbb;
  return (int)(w < 1 ? 1 : (w > most ? most : w));
}

// Shapes the attention entry points take: B N H query rows within INT32_MAX / 4,
// a prefix bound within DDTREE_MAX_EXTENT and at most kMaxSplits explicit splits.
constexpr int kMaxSplits = 1024;

bool attn_shape_supported(int B, int N, int H, int64_t max_prefix_len, int num_splits) {
  int64_t rows;
  if (__builtin_mul_overflow((int64_t)B * N, (int64_t)H, &rows)) return false;
  return rows <= INT32_MAX / 4 && max_prefix_len <= DDTREE_MAX_EXTENT && num_splits <= kMaxSplits;
}

int auto_schedule(bool mfma, int B, int N, int H, int64_t max_prefix_len) {
  if (band_schedule_applies(mfma, N, H)) return 0;
  return auto_splits(mfma, B, N, H, max_prefix_len);
}

// Uniform split count (>= 1), or 0 for the band schedule.
int resolve_splits(bool mfma, int B, int N, int H, int64_t max_prefix_len, int num_splits) {
  if (!mfma) return 1;
  return num_splits > 0 ? num_splits : auto_schedule(mfma, B, N, H, max_prefix_len);
}

// Band schedule workspace, sized from the call: a workgroup (window, slot) keeps
// at most two partials (the band cut at its window's start and the one cut at
// its end), so windows * R * 2 partial slots of kRowsPerBlock rows (o then lse),
// then one 16-byte record per window (record 0: the column total and window
// count, record e: edge e's cut descriptor).
int band_part_slots(int N, int H, int windows) {
  const int64_t n_rb = ceil_div((int64_t)N * H, kRowsPerBlock);
  const int64_t rbb = n_rb % kBandRowBlocks == 0 ? kBandRowBlocks : n_rb;
  return (int)(2 * windows * rbb);
}

size_t workspace_bytes_for(bool mfma, int B, int N, int H, int Dl, int splits, int64_t max_prefix_len) {
  if (!mfma) return 0;
  if (splits == 0) {
    const int windows = band_windows_bound(B, N, H, max_prefix_len);
    return (size_t)band_part_slots(N, H, windows) * kRowsPerBlock * kPartialRecordBytes +
           (size_t)windows * 4 * sizeof(int);
  }
  if (splits == 1) return 0;
  const uint64_t rows = (uint64_t)B * N * H;
  return (size_t)(splits * rows * kPartialRecordBytes);
}

// ---- scratch of ddtree_verify_attn_noalloc ----
// One file-scope device array; each GPU the library runs on holds its own copy
// for the life of the process.  In host code `scratch` is only a stand-in
// symbol: its device address on a GPU comes from hipGetSymbolAddress, called
// once per device with that device current, and only that address is ever
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[DDTREE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`.
hipError_t scratch_for_stream(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

#ifndef DDTREE_SOURCE_DIGEST
#define DDTREE_SOURCE_DIGEST "unknown"
#endif

extern "C" {

const char* ddtree_build_digest(void) { return DDTREE_SOURCE_DIGEST; }

const char* ddtree_status_string(int status) {
  switch (status) {
    case DDTREE_OK: return "DDTREE_OK";
    case DDTREE_ERR_INVALID_ARG: return "DDTREE_ERR_INVALID_ARG";
    case DDTREE_ERR_UNSUPPORTED: return "DDTREE_ERR_UNSUPPORTED";
    case DDTREE_ERR_WORKSPACE: return "DDTREE_ERR_WORKSPACE";
    case DDTREE_ERR_HIP: return "DDTREE_ERR_HIP";
    default: return "DDTREE_UNKNOWN_STATUS";
  }
}

int ddtree_build_mask(const int32_t* parents, int32_t B, int32_t N, const int64_t* prefix_offsets, uint32_t* mask,
                      int32_t* depth, int64_t* positions, int32_t* tree_ok, void* stream) {
  if (B < 0 || N < 1) return DDTREE_ERR_INVALID_ARG;
  if (N > DDTREE_MAX_NODES) return DDTREE_ERR_UNSUPPORTED;
  if (B == 0) return DDTREE_OK;
  if (!parents || !mask || !depth || !tree_ok) return DDTREE_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)B * N;
  const uint64_t W = (uint64_t)(N + 31) / 32;
  const Range ins[] = {range_of(parents, n * 4), range_of(prefix_offsets, prefix_offsets ? ((uint64_t)B + 1) * 8 : 0)};
  const Range outs[] = {range_of(mask, n * W * 4), range_of(depth, n * 4), range_of(positions, positions ? n * 8 : 0),
                        range_of(tree_ok, (uint64_t)B * 4)};
  if (any_overlap(outs, 4, ins, 2)) return DDTREE_ERR_INVALID_ARG;
  hipError_t e = launch_build_mask(parents, B, N, prefix_offsets, mask, depth, positions, tree_ok,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP;
}

int32_t ddtree_verify_attn_auto_splits(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                                       int64_t max_prefix_len) {
  if (B <= 0 || N <= 0 || H <= 0 || max_prefix_len < 0 || !attn_shape_supported(B, N, H, max_prefix_len, 0))
    return 1;
  return auto_schedule(mfma_path(dtype, Dl, Dr), B, N, H, max_prefix_len);
}

size_t ddtree_verify_attn_workspace_size(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                                         int64_t max_prefix_len, int32_t num_splits) {
  if (B <= 0 || N <= 0 || H <= 0 || Dl <= 0 || num_splits < 0 || max_prefix_len < 0) return 0;
  if (!attn_shape_supported(B, N, H, max_prefix_len, num_splits)) return 0;
  const bool mfma = mfma_path(dtype, Dl, Dr);
  const int s = resolve_splits(mfma, B, N, H, max_prefix_len, num_splits);
  return workspace_bytes_for(mfma, B, N, H, Dl, s, max_prefix_len);
}

int ddtree_verify_attn(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr, const void* q_lat,
                       const void* q_rope, const void* ckv, int64_t ld_ckv, const void* krope, int64_t ld_krope,
                       const int64_t* prefix_offsets, int64_t max_prefix_len, const void* ckv_tree,
                       int64_t ld_ckv_tree, const void* krope_tree, int64_t ld_krope_tree, const uint32_t* mask,
                       float softmax_scale, int32_t num_splits, float* o, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  // ---- shapes ----
  if (dtype != DDTREE_F32 && dtype != DDTREE_BF16) return DDTREE_ERR_UNSUPPORTED;
  if (B < 0 || N < 1 || H < 1 || Dl < 1 || Dr < 0 || num_splits < 0 || max_prefix_len < 0)
    return DDTREE_ERR_INVALID_ARG;
  if (N > DDTREE_MAX_NODES) return DDTREE_ERR_UNSUPPORTED;
  const bool mfma = mfma_path(dtype, Dl, Dr);
  if (!mfma && (Dl > 512 || Dr > 512)) return DDTREE_ERR_UNSUPPORTED;
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
    return DDTREE_ERR_INVALID_ARG;
  if (!attn_shape_supported(B, N, H, max_prefix_len, num_splits)) return DDTREE_ERR_UNSUPPORTED;
  if (B == 0) return DDTREE_OK;
  // ---- pointers and strides ----
  if (!q_lat || !prefix_offsets || !ckv_tree || !mask || !o || !lse) return DDTREE_ERR_INVALID_ARG;
  if (Dr > 0 && (!q_rope || !krope_tree)) return DDTREE_ERR_INVALID_ARG;
  if (max_prefix_len > 0 && (!ckv || (Dr > 0 && !krope))) return DDTREE_ERR_INVALID_ARG;
  if (ld_ckv < Dl || ld_ckv_tree < Dl || ld_krope < Dr || ld_krope_tree < Dr) return DDTREE_ERR_INVALID_ARG;
  if (dtype == DDTREE_BF16 && !mfma) {
    // generic kernel: element loads only
    const uintptr_t any = reinterpret_cast<uintptr_t>(q_lat) | reinterpret_cast<uintptr_t>(q_rope) |
                          reinterpret_cast<uintptr_t>(ckv) | reinterpret_cast<uintptr_t>(krope) |
                          reinterpret_cast<uintptr_t>(ckv_tree) | reinterpret_cast<uintptr_t>(krope_tree);
    if (any & 1u) return DDTREE_ERR_INVALID_ARG;
  }
  if (mfma) {
    if (!aligned16(q_lat) || !aligned16(q_rope) || !aligned16(ckv) || !aligned16(krope) || !aligned16(ckv_tree) ||
        !aligned16(krope_tree) || !aligned16(o))
      return DDTREE_ERR_INVALID_ARG;
    if ((ld_ckv | ld_krope | ld_ckv_tree | ld_krope_tree) & 7) return DDTREE_ERR_INVALID_ARG;
    // the kernel forms byte offsets of a 32-key tile's rows in 32 bits
    if (ld_ckv > kMaxBf16RowStride || ld_krope > kMaxBf16RowStride || ld_ckv_tree > kMaxBf16RowStride ||
        ld_krope_tree > kMaxBf16RowStride)
      return DDTREE_ERR_UNSUPPORTED;
  }
  if (ld_ckv > DDTREE_MAX_EXTENT || ld_krope > DDTREE_MAX_EXTENT || ld_ckv_tree > DDTREE_MAX_EXTENT ||
      ld_krope_tree > DDTREE_MAX_EXTENT)
    return DDTREE_ERR_UNSUPPORTED;
  // ---- workspace ----
  const int splits = resolve_splits(mfma, B, N, H, max_prefix_len, num_splits);
  const size_t need = workspace_bytes_for(mfma, B, N, H, Dl, splits, max_prefix_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DDTREE_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return DDTREE_ERR_INVALID_ARG;
  // ---- aliasing (extents known on the host) ----
  const uint64_t rows = (uint64_t)B * N * H;
  const uint64_t es = dtype == DDTREE_BF16 ? 2 : 4;
  const uint64_t W = (uint64_t)(N + 31) / 32;
  const uint64_t tree_rows = (uint64_t)B * N;
  // The prefix cache's true extent (offsets[B] rows) lives on the device; the
  // host checks the first max_prefix_len rows at ckv and krope.
  const uint64_t mp = (uint64_t)max_prefix_len;
  const Range ins[] = {range_of(q_lat, rows * Dl * es),
                       range_of(q_rope, Dr ? rows * Dr * es : 0),
                       range_of(prefix_offsets, ((uint64_t)B + 1) * 8),
                       range_of(mask, tree_rows * W * 4),
                       range_of(ckv_tree, rows_bytes(tree_rows, ld_ckv_tree, Dl, es)),
                       range_of(krope_tree, rows_bytes(tree_rows, ld_krope_tree, Dr, es)),
                       range_of(ckv, rows_bytes(mp, ld_ckv, Dl, es)),
                       range_of(krope, rows_bytes(mp, ld_krope, Dr, es))};
  const Range outs[] = {range_of(o, rows * Dl * 4), range_of(lse, rows * 4), range_of(workspace, need)};
  if (any_overlap(outs, 3, ins, 8)) return DDTREE_ERR_INVALID_ARG;

  AttnArgs a;
  a.B = B;
  a.N = N;
  a.H = H;
  a.Dl = Dl;
  a.Dr = Dr;
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.ckv = ckv;
  a.ld_ckv = ld_ckv;
  a.krope = krope;
  a.ld_krope = ld_krope;
  a.prefix_offsets = prefix_offsets;
  a.ckv_tree = ckv_tree;
  a.ld_ckv_tree = ld_ckv_tree;
  a.krope_tree = krope_tree;
  a.ld_krope_tree = ld_krope_tree;
  a.mask = mask;
  a.scale = softmax_scale;
  a.splits = splits > 0 ? splits : 1;
  a.balanced = splits == 0 ? 1 : 0;
  a.o = o;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_aux = nullptr;
  a.band_edges = nullptr;
  a.band_windows = 0;
  if (splits != 1) {
    // records: fp16 values, then {lse2, k} pairs, then (band schedule) the edge descriptors
    uint64_t records = (uint64_t)splits * rows;
    if (splits == 0) {
      a.band_windows = band_windows_bound(B, N, H, max_prefix_len);
      records = (uint64_t)band_part_slots(N, H, a.band_windows) * kRowsPerBlock;
    }
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    a.part_o = ws;
    a.part_aux = reinterpret_cast<float2*>(ws + records * Dl * 2);
    if (splits == 0) a.band_edges = reinterpret_cast<int*>(a.part_aux + records);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (mfma) {
    e = launch_verify_attn_bf16(a, s);
    if (e == hipSuccess && splits > 1) e = launch_attn_combine(a, s);
    if (e == hipSuccess && splits == 0) e = launch_attn_band_combine(a, s);
  } else {
    e = launch_verify_attn_generic(a, dtype == DDTREE_BF16, s);
  }
  return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP;
}

int ddtree_verify_attn_noalloc(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dl, int32_t Dr,
                               const void* q_lat, const void* q_rope, const void* ckv, int64_t ld_ckv,
                               const void* krope, int64_t ld_krope, const int64_t* prefix_offsets,
                               int64_t max_prefix_len, const void* ckv_tree, int64_t ld_ckv_tree,
                               const void* krope_tree, int64_t ld_krope_tree, const uint32_t* mask,
                               float softmax_scale, int32_t num_splits, float* o, float* lse, void* stream) {
  // the size check comes first: a call too large for the scratch touches no device state
  const size_t need = ddtree_verify_attn_workspace_size(dtype, B, N, H, Dl, Dr, max_prefix_len, num_splits);
  if (need > DDTREE_NOALLOC_SCRATCH_BYTES) return DDTREE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && B > 0) {
    if (scratch_for_stream(static_cast<hipStream_t>(stream), &ws) != hipSuccess) return DDTREE_ERR_HIP;
  }
  return ddtree_verify_attn(dtype, B, N, H, Dl, Dr, q_lat, q_rope, ckv, ld_ckv, krope, ld_krope, prefix_offsets,
                            max_prefix_len, ckv_tree, ld_ckv_tree, krope_tree, ld_krope_tree, mask, softmax_scale,
                            num_splits, o, lse, ws, ws ? (size_t)DDTREE_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int ddtree_greedy_accept(const float* logits, int64_t ld_logits, const int32_t* tokens, const int32_t* parents,
                         int32_t B, int32_t N, int32_t V, int32_t* target_argmax, int32_t* accept_len,
                         int32_t* accept_nodes, int32_t* commit_tokens, void* stream) {
  if (B < 0 || N < 1 || V < 1 || ld_logits < V) return DDTREE_ERR_INVALID_ARG;
  if (N > DDTREE_MAX_NODES) return DDTREE_ERR_UNSUPPORTED;
  if ((int64_t)B * N > INT32_MAX || ld_logits > DDTREE_MAX_EXTENT) return DDTREE_ERR_UNSUPPORTED;
  if (B == 0) return DDTREE_OK;
  if (!logits || !tokens || !parents || !target_argmax || !accept_len || !accept_nodes || !commit_tokens)
    return DDTREE_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)B * N;
  const Range ins[] = {range_of(logits, rows_bytes(n, ld_logits, V, 4)), range_of(tokens, n * 4),
                       range_of(parents, n * 4)};
  const Range outs[] = {range_of(target_argmax, n * 4), range_of(accept_len, (uint64_t)B * 4),
                        range_of(accept_nodes, n * 4), range_of(commit_tokens, n * 4)};
  if (any_overlap(outs, 4, ins, 3)) return DDTREE_ERR_INVALID_ARG;
  hipError_t e = launch_accept(logits, ld_logits, tokens, parents, B, N, V, target_argmax, accept_len, accept_nodes,
                               commit_tokens, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP;
}

int ddtree_compact_kv(int32_t dtype, int32_t B, int32_t N, int32_t Dl, int32_t Dr, const void* ckv_tree,
                      int64_t ld_ckv_tree, const void* krope_tree, int64_t ld_krope_tree, const int32_t* accept_len,
                      const int32_t* accept_nodes, const int64_t* dest_rows, void* ckv, int64_t ld_ckv, void* krope,
                      int64_t ld_krope, void* stream) {
  if (dtype != DDTREE_F32 && dtype != DDTREE_BF16) return DDTREE_ERR_UNSUPPORTED;
  if (B < 0 || N < 1 || Dl < 1 || Dr < 0) return DDTREE_ERR_INVALID_ARG;
  if (N > DDTREE_MAX_NODES) return DDTREE_ERR_UNSUPPORTED;
  if (B == 0) return DDTREE_OK;
  if (!ckv_tree || !ckv || !accept_len || !accept_nodes || !dest_rows) return DDTREE_ERR_INVALID_ARG;
  if (Dr > 0 && (!krope_tree || !krope)) return DDTREE_ERR_INVALID_ARG;
  if (ld_ckv_tree < Dl || ld_ckv < Dl || (Dr > 0 && (ld_krope_tree < Dr || ld_krope < Dr)))
    return DDTREE_ERR_INVALID_ARG;
  if (ld_ckv_tree > DDTREE_MAX_EXTENT || ld_ckv > DDTREE_MAX_EXTENT || ld_krope_tree > DDTREE_MAX_EXTENT ||
      ld_krope > DDTREE_MAX_EXTENT)
    return DDTREE_ERR_UNSUPPORTED;
  const int64_t es = dtype == DDTREE_BF16 ? 2 : 4;
  if (!aligned_to(ckv_tree, (unsigned)es) || !aligned_to(ckv, (unsigned)es) ||
      (Dr > 0 && (!aligned_to(krope_tree, (unsigned)es) || !aligned_to(krope, (unsigned)es))))
    return DDTREE_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)B * N;
  const Range ctrl[] = {range_of(accept_len, (uint64_t)B * 4), range_of(accept_nodes, n * 4),
                        range_of(dest_rows, (uint64_t)B * 8)};
  const Range trees[] = {range_of(ckv_tree, rows_bytes(n, ld_ckv_tree, Dl, es)),
                         range_of(krope_tree, rows_bytes(n, ld_krope_tree, Dr, es))};
  // the tree rows (which may interleave, as views of one fused row) must not alias the path arrays
  for (const Range& c : ctrl)
    if (c.bad) return DDTREE_ERR_INVALID_ARG;
  for (const Range& t : trees)
    for (const Range& c : ctrl)
      if (overlaps(t, c)) return DDTREE_ERR_INVALID_ARG;
  CompactArgs a{};
  a.B = B;
  a.N = N;
  a.ckv_tree = static_cast<const unsigned char*>(ckv_tree);
  a.ld_ckv_tree = ld_ckv_tree * es;
  a.krope_tree = static_cast<const unsigned char*>(krope_tree);
  a.ld_krope_tree = ld_krope_tree * es;
  a.accept_len = accept_len;
  a.accept_nodes = accept_nodes;
  a.ckv = static_cast<unsigned char*>(ckv);
  a.ld_ckv = ld_ckv * es;
  a.krope = static_cast<unsigned char*>(krope);
  a.ld_krope = ld_krope * es;
  a.dest_rows = dest_rows;
  a.c_bytes = Dl * es;
  a.r_bytes = Dr * es;
  a.c_unit = copy_unit(ckv_tree, a.ld_ckv_tree, ckv, a.ld_ckv, a.c_bytes);
  a.r_unit = Dr > 0 ? copy_unit(krope_tree, a.ld_krope_tree, krope, a.ld_krope, a.r_bytes) : 2;
  hipError_t e = launch_compact_kv(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP;
}

int ddtree_build_tree(int32_t B, int32_t N, int32_t D, int32_t K, const int32_t* root_tokens,
                      const int32_t* cand_tokens, const float* cand_logp, int32_t* parents, int32_t* tokens,
                      int32_t* depth, float* scores, void* stream) {
  if (B < 0 || N < 1 || D < 1 || K < 1) return DDTREE_ERR_INVALID_ARG;
  if (N > DDTREE_MAX_NODES || D > DDTREE_MAX_DEPTH || K > DDTREE_MAX_PROPOSALS) return DDTREE_ERR_UNSUPPORTED;
  // the candidate tree must hold N nodes: 1 + K + ... + K^D (saturated)
  int64_t size = 1, level = 1;
  for (int d = 1; d <= D && size < N; ++d) {
    level = level * K > DDTREE_MAX_NODES ? DDTREE_MAX_NODES : level * K;
    size += level;
  }
  if (size < N) return DDTREE_ERR_UNSUPPORTED;
  if (B == 0) return DDTREE_OK;
  if (!root_tokens || !cand_tokens || !cand_logp || !parents || !tokens) return DDTREE_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)B * N, c = (uint64_t)B * D * K;
  const Range ins[] = {range_of(root_tokens, (uint64_t)B * 4), range_of(cand_tokens, c * 4),
                       range_of(cand_logp, c * 4)};
  const Range outs[] = {range_of(parents, n * 4), range_of(tokens, n * 4), range_of(depth, depth ? n * 4 : 0),
                        range_of(scores, scores ? n * 4 : 0)};
  if (any_overlap(outs, 4, ins, 3)) return DDTREE_ERR_INVALID_ARG;
  hipError_t e = launch_build_tree(B, N, D, K, root_tokens, cand_tokens, cand_logp, parents, tokens, depth, scores,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP;
}

int ddtree_rope_tree(int32_t dtype, int32_t B, int32_t N, int32_t H, int32_t Dr, void* q_rope, void* krope_tree,
                     int64_t ld_krope_tree, const int64_t* positions, const double* inv_freq, void* stream) {
  if (dtype != DDTREE_F32 && dtype != DDTREE_BF16) return DDTREE_ERR_UNSUPPORTED;
  if (B < 0 || N < 1 || H < 1 || Dr < 2 || (Dr & 1)) return DDTREE_ERR_INVALID_ARG;
  if (N > DDTREE_MAX_NODES || Dr > kMaxRopeDim) return DDTREE_ERR_UNSUPPORTED;
  // the kernel indexes nodes and a node's (H + 1) rotary rows of Dr elements in 32 bits
  if ((int64_t)B * N > INT32_MAX || ((int64_t)H + 1) * Dr > INT32_MAX ||
      (krope_tree && ld_krope_tree > DDTREE_MAX_EXTENT))
    return DDTREE_ERR_UNSUPPORTED;
  if (B == 0 || (!q_rope && !krope_tree)) return DDTREE_OK;
  if (!positions || !inv_freq) return DDTREE_ERR_INVALID_ARG;
  if (krope_tree && ld_krope_tree < Dr) return DDTREE_ERR_INVALID_ARG;
  const int64_t es = dtype == DDTREE_BF16 ? 2 : 4;
  if ((q_rope && !aligned_to(q_rope, (unsigned)es)) || (krope_tree && !aligned_to(krope_tree, (unsigned)es)))
    return DDTREE_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)B * N;
  const Range ins[] = {range_of(positions, n * 8), range_of(inv_freq, (uint64_t)(Dr / 2) * 8)};
  const Range outs[] = {range_of(q_rope, q_rope ? mul_ext(mul_ext(n, (uint64_t)H * Dr), es) : 0),
                        range_of(krope_tree, krope_tree ? rows_bytes(n, ld_krope_tree, Dr, es) : 0)};
  if (any_overlap(outs, 2, ins, 2)) return DDTREE_ERR_INVALID_ARG;
  RopeArgs a{};
  a.B = B;
  a.N = N;
  a.H = H;
  a.Dr = Dr;
  a.bf16 = dtype == DDTREE_BF16;
  a.q_rope = q_rope;
  a.krope_tree = krope_tree;
  a.ld_krope_tree = ld_krope_tree;
  a.positions = positions;
  a.inv_freq = inv_freq;
  hipError_t e = launch_rope_tree(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP;
}

}  // extern "C"
