// Tree-verify attention, absorbed MLA form, bf16 inputs on gfx950 MFMA.
//
// What is computed (page "The Moment of Proof: Validating a Native CUDA
// Speculative Decoding Engine", section "Input Knowledge Required": MLA in
// absorb form, the draft tree verified in one forward under a custom mask;
// page "The Moment of Proof: Running the Native DDTree Speculative Decoding
// Engine", section "Input Knowledge Required": verify attention with
// visibility masking): every (node, head) query row attends to its request's
// cached latent rows plus its visible tree rows; key = [c | r] (576 wide),
// value = c (512 wide); output o (float32, latent space) and the natural
// log-sum-exp of the scaled scores.
//
// Design (MI355X / gfx950):
//  * All H heads of all N tree nodes of a request read the same latent KV
//    stream, so (node, head) pairs are the rows of a dense contraction.  A
//    workgroup of 4 waves owns 128 rows; each wave 32 rows.
//  * The 32 rows' absorbed queries stay in VGPRs for the whole kernel (28
//    bf16x8 B-fragments, 112 VGPRs); the last 4 latent and the 4 rotary
//    k-steps are staged in LDS and read per tile.  A piece starts by copying
//    its queries into LDS with coalesced direct-to-LDS loads and reading the
//    fragments from there.
//  * KV tiles of 32 keys x 576 bf16 are copied HBM -> LDS with direct-to-LDS
//    16-byte loads into a 3-deep ring, with a 16-byte-chunk XOR swizzle that
//    keeps both read patterns below bank-conflict free.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = key rows read with
//    ds_read_b128, B = query fragments): each lane ends up holding 16 scores
//    of ONE query row, so the online-softmax statistics are per-lane scalars
//    and the row max needs a single cross-half exchange.
//  * O^T += V^T P^T on the same MFMA: V^T fragments come straight from the
//    row-major LDS tile through ds_read_b64_tr_b16 (transpose reads), and
//    the probabilities, rounded to bf16, are already in the B-operand layout
//    (no shuffle).  The 512 x 32 float32 accumulator (256 registers) again
//    holds one row per lane.  Probabilities use a fixed per-row reference
//    (the first visible tile's max, with 2^100 of headroom), so the
//    accumulators are never rescaled; a score beyond the headroom triggers
//    one rerun of the workgroup's tiles with the true row maximum.
//  * Software pipeline: iteration t runs the S^T MFMAs of tile t + 1, then
//    the O^T MFMAs of tile t, and computes the probabilities of tile t + 1
//    (one element per MFMA) in the shadow of the latter.  The first V^T
//    reads of tile t are issued during the last S^T MFMAs, and the first
//    O^T MFMAs ahead of the probability preparation (neither depends on
//    tile t + 1), so the MFMA pipe does not wait between the two streams.
//  * MFMAs are issued by inline asm to pin S^T to VGPRs and O^T to AGPRs;
//    LDS fragment reads run 3-4 MFMAs ahead; workgroups are mapped so that a
//    request's row blocks share one XCD's L2.
//  * On tiles of the slow path (tree tiles, a partial last prefix tile, a
//    row's first visible tile) P is applied as two bf16 terms, hi + lo, so
//    rows that see only a few keys keep about 16 bits of each weight; the
//    exp-sum adds exactly the bf16 values applied.
//  * Prefix tiles first, then tree tiles; the ancestor mask is one 32-bit
//    word per row per tree tile.
//  * Scheduling: the band schedule (below) balances ragged batches over the
//    CUs and keeps each XCD on one KV stream; otherwise long prefixes can be
//    split uniformly across workgroups (flash-decoding).  Partials are stored
//    as fp16 records under a per-row power-of-two scale and merged by a
//    combine kernel with the log-sum-exp weights.
#include <cmath>

#include "ddtree_internal.h"

namespace ddtree {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int DL = kMfmaDl;                 // 512
constexpr int DR = kMfmaDr;                 // 64

constexpr int KT = kKeysPerTile;            // 32 keys per tile
constexpr int C_ROW = DL * 2;               // 1024 bytes: latent part of one key in LDS
constexpr int R_ROW = DR * 2;               // 128 bytes: rotary part of one key in LDS
constexpr int R_OFF = KT * C_ROW;           // rotary region after the 32 latent rows
constexpr int TILE_BYTES = KT * (C_ROW + R_ROW);  // 36864
constexpr int NBUF = 3;
constexpr int ROWS = kRowsPerBlock;         // 128
constexpr int NWAVES = 4;
constexpr int C_LOADS_PER_WAVE = KT / NWAVES;   // 8 latent rows (1 KB each) per wave per tile
constexpr int LOADS_PER_WAVE = C_LOADS_PER_WAVE + 1;  // + one 1 KB slice of the rotary region
constexpr int MAXW = 8;                     // mask words per row (N <= 256)
constexpr float kHeadroomLog2 = 100.0f;     // scores may exceed a row's reference by 2^100
constexpr int kTwoTermMinFullTiles = 8;     // pieces with this many full prefix tiles take single P terms
constexpr int kPartialTopExp = 14;          // partial records: a row's largest |value| in [2^13, 2^14)
constexpr bf16x2 kBf16Ones = {(__bf16)1.0f, (__bf16)1.0f};

static_assert(KT * R_ROW == NWAVES * 1024, "rotary region must split into one 1 KB load per wave");
static_assert(LOADS_PER_WAVE == 9, "the copies are spread over the first 33 S^T MFMAs (one every fourth)");

// LDS layout of a tile.  Latent rows: key k at k * 1024, its 16-byte chunk p at
// 16 * (p >> 4) + ((p & 15) ^ swz(k)).  gfx950's LDS has 64 banks of 4 bytes.
// The key-fragment read (ds_read_b128) is served 16 lanes at a time: 16
// consecutive keys, one chunk, so swz must be a bijection on k & 15.  The
// transpose read (ds_read_b64_tr_b16) is served 32 lanes at a time: 4 keys of
// an aligned group of 4, each with 4 consecutive chunks of an aligned group of
// 4 (both 8-byte halves), so the 4 keys must land in 4 different chunk
// groups: (swz(k) >> 2) distinct over k & 3 (bank-conflict counters confirm
// that pass size).  swz(k) = ((k & 3) << 2) | ((k >> 2) & 3) does both, and
// swz(k + 8) = swz(k) ^ 2, swz(k + 16) = swz(k).  The rotary rows
// (8 chunks) are stored in pairs: keys 2 j and 2 j + 1 share the 256-byte row j,
// logical chunk (k & 1) * 8 + c at ((k & 1) * 8 + c) ^ (j & 7), which again
// spreads 16 consecutive keys over all 64 banks.
__device__ __forceinline__ int swz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }
__device__ __forceinline__ int pair_chunk(int key, int c) { return (((key & 1) << 3) | c) ^ ((key >> 1) & 7); }

// Hides a value from the optimiser (no code is emitted).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Direct-to-LDS 16-byte loads (global_load_lds_dwordx4, below) are written as
// inline asm so that the compiler does not treat them as LDS stores and
// serialise every later LDS read behind them; completion is tracked by the
// explicit vmcnt waits in the tile loop (vmcnt counts every vector memory op
// in issue order, so waits the compiler adds for its own loads stay correct).
// Each statement writes M0 and declares it clobbered.  M0 is a reserved register
// to the compiler, which does not keep values in it across statements (it
// writes M0 right before each instruction that reads it), so clang warns that
// the clobber is not needed for preservation; the warning is silenced here.  A
// compile-time test checks that no other instruction of the kernel reads or
// writes M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// Wait for every tile copy this wave has issued.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The direct-to-LDS copies of one tile (LDS layout above), 9 per wave.  Copy
// i < 8 loads latent key wave + 4 i with one 64-lane load (lane = physical
// chunk, so the lane fetches global chunk lane ^ swz(key)); copy 8 loads the
// 1 KB of the rotary region holding keys 8 wave .. 8 wave + 7 (pair rows
// 4 wave .. 4 wave + 3; lane = 16 * pair row + physical chunk).  Keys past the
// tile's valid count re-read its last valid row (masked later).  A CopyPlan
// holds the tile's row bases and strides (scalar) and its valid key count.
// The swizzle of key wave + 4 i is 4 wave + (i & 3), so the lane's chunk
// offset (lane ^ swz) * 16 is lw ^ 16 (i & 3), with lw = 16 lane ^ 64 wave
// (one v_xad_u32 per copy).  The rotary copy of a lane
// reads key rkey (clamped), 16-byte piece rpiece.  Lane values go through
// opaque() so that they are recomputed per copy instead of being kept in, or
// spilled from, registers across the tile loop.
struct CopyLanes {
  uint32_t lw;         // latent chunk offset of copy 0
  int rkey;            // rotary: the lane's key within the tile
  uint32_t rpiece;     // rotary: byte offset of the lane's 16 bytes within the key's rotary row
};
struct CopyPlan {
  const unsigned char* c;   // latent row of the tile's first key
  const unsigned char* r;   // rotary row of the tile's first key
  uint32_t cstride, rstride;  // row strides in bytes
  int count;                // valid keys (1..32)
};

// Row indices and byte strides fit in 32 bits for any cache that fits in device
// memory (a latent row holds 1 KB; row strides are checked below 2^24 elements on
// the host), so each row address is one 32 x 32 -> 64-bit scalar product.
__device__ __forceinline__ CopyPlan copy_plan(const AttnArgs& a, int b, int64_t p0, int64_t L, int n_pt, int t) {
  CopyPlan q;
  const unsigned char* cb;
  const unsigned char* rb;
  uint32_t row0, cs, rs;
  if (t < n_pt) {
    row0 = (uint32_t)p0 + (uint32_t)t * KT;
    cb = static_cast<const unsigned char*>(a.ckv);
    rb = static_cast<const unsigned char*>(a.krope);
    cs = (uint32_t)a.ld_ckv * 2u;
    rs = (uint32_t)a.ld_krope * 2u;
    const int rem = (int)L - t * KT;
    q.count = rem < KT ? rem : KT;
  } else {
    const int node0 = (t - n_pt) * KT;
    row0 = (uint32_t)(b * a.N + node0);
    cb = static_cast<const unsigned char*>(a.ckv_tree);
    rb = static_cast<const unsigned char*>(a.krope_tree);
    cs = (uint32_t)a.ld_ckv_tree * 2u;
    rs = (uint32_t)a.ld_krope_tree * 2u;
    const int rem = a.N - node0;
    q.count = rem < KT ? rem : KT;
  }
  row0 = __builtin_amdgcn_readfirstlane(row0);   // wave-uniform: keep the products scalar
  cs = __builtin_amdgcn_readfirstlane(cs);
  rs = __builtin_amdgcn_readfirstlane(rs);
  q.cstride = cs;
  q.rstride = rs;
  q.c = cb + (uint64_t)row0 * cs;
  q.r = rb + (uint64_t)row0 * rs;
  return q;
}

// The lane's address is formed inside the asm statement, between the M0 write
// and the load: that covers the one wait state an LDS DMA needs after M0 is
// written, and the compiler cannot precompute per-copy lane values (which it
// would keep in VGPRs across the tile loop).
// Latent copy: lane address (lw ^ xr) + rowoff, with xr = 16 (i & 3) an inline constant.
template <int XR>
__device__ __forceinline__ void lds_dma16_latent(uint32_t lds_base, const void* gbase, uint32_t lw, uint32_t rowoff) {
  uint32_t addr;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "v_xad_u32 %0, %2, %3, %4\n\t"
      "global_load_lds_dwordx4 %0, %5"
      : "=&v"(addr)
      : "s"(lds_base), "v"(lw), "i"(XR), "s"(rowoff), "s"(gbase)
      : "memory", "m0");
}
// Rotary copy: lane address rowoff + piece.
__device__ __forceinline__ void lds_dma16_rotary(uint32_t lds_base, const void* gbase, uint32_t rowoff, uint32_t piece) {
  uint32_t addr;
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "v_add_u32_e32 %0, %2, %3\n\t"
      "global_load_lds_dwordx4 %0, %4"
      : "=&v"(addr)
      : "s"(lds_base), "v"(rowoff), "v"(piece), "s"(gbase)
      : "memory", "m0");
}

#pragma clang diagnostic pop

template <int I>
__device__ __forceinline__ void issue_copy(const CopyPlan& q, const CopyLanes& cl, uint32_t lds_buf, int wave) {
  if constexpr (I < C_LOADS_PER_WAVE) {
    const int key = wave + NWAVES * I;
    const uint32_t kc = (uint32_t)min(key, q.count - 1);
    lds_dma16_latent<(I & 3) << 4>(lds_buf + key * C_ROW, q.c, cl.lw, kc * q.cstride);
  } else {
    const uint32_t kc = (uint32_t)min(opaque(cl.rkey), q.count - 1);
    lds_dma16_rotary(lds_buf + R_OFF + wave * 1024, q.r, kc * q.rstride, cl.rpiece);
  }
}

// Copy i of a tile, i a compile-time constant after unrolling.
__device__ __forceinline__ void issue_copy(const CopyPlan& q, const CopyLanes& cl, uint32_t lds_buf, int wave, int i) {
  switch (i) {
    case 0: issue_copy<0>(q, cl, lds_buf, wave); break;
    case 1: issue_copy<1>(q, cl, lds_buf, wave); break;
    case 2: issue_copy<2>(q, cl, lds_buf, wave); break;
    case 3: issue_copy<3>(q, cl, lds_buf, wave); break;
    case 4: issue_copy<4>(q, cl, lds_buf, wave); break;
    case 5: issue_copy<5>(q, cl, lds_buf, wave); break;
    case 6: issue_copy<6>(q, cl, lds_buf, wave); break;
    case 7: issue_copy<7>(q, cl, lds_buf, wave); break;
    default: issue_copy<8>(q, cl, lds_buf, wave); break;
  }
}

// Byte offset in a tile of the K fragment for latent k-step s (< 32): key lr,
// logical chunk 2 s + g; kbase = lr * 1024 + ((g ^ swz(lr)) << 4).
__device__ __forceinline__ int kaddr(int kbase, int s) { return (kbase ^ ((s & 7) << 5)) + (s >> 3) * 256; }

// V^T fragment of 16-key step ks and 32-dim block db: two transpose reads of
// 4 keys each (keys 16 ks + 4 g + 0..3 and 16 ks + 8 + 4 g + 0..3).  voff holds
// the lane's row and swizzled chunk for db = 0, first read, and voff_hi the
// same for the second read (8 keys on, whose swizzle differs in bit 1:
// (voff ^ 32) + 8 rows); db & 3 enters by XOR, db >> 2 and ks by offset, so
// both reads of every step are a per-tile base plus an immediate.
__device__ __forceinline__ bf16x8 load_vt(const unsigned char* buf, int voff, int voff_hi, int ks, int db) {
  const int add = (db >> 2) * 256 + ks * 16 * C_ROW;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + (voff ^ ((db & 3) << 6)) + add));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + (voff_hi ^ ((db & 3) << 6)) + add));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---- MFMA issue (inline asm) ---------------------------------------------
// The MFMAs are issued through inline asm so that the two accumulators get the
// register class each needs: S^T (read by the softmax VALU code) in VGPRs and
// the 512 x 32 output accumulator in AGPRs.  The compiler does not model the
// MFMA pipeline behind an asm statement, so the wait states it would insert
// are written out: 16 after the last S^T MFMA of a tile before VALU reads of
// S^T, 16 after the tile loop before any AGPR read or rewrite, and 4 between
// VALU writes of P and the first O^T MFMA of a tile.  Chained MFMAs on one
// accumulator need no wait states.
__device__ __forceinline__ void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\t"
      "s_nop 7"
      : "+v"(acc)
      : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile(
      "s_nop 3\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
      : "+a"(acc)
      : "v"(a), "v"(b));
}

// max / sum of a value and its twin in the other half-wave (same query row)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroups are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8).
// Give each XCD a contiguous range of work items, so the row blocks of one
// request (which stream the same KV) share an L2.
__device__ __forceinline__ int xcd_local_item(int block, int total) {
  const int x = block & 7, k = block >> 3;
  const int base = total >> 3, extra = total & 7;
  return x * base + min(x, extra) + k;
}

// ---- band schedule ----------------------------------------------------------
// Used when a request's 128-row blocks come in whole groups of 32 (one per CU
// of an XCD), or their count R divides 32.  A band is R row blocks of one
// request (R = 32, or all of the request's); they all stream the request's KV,
// Tb = ceil(L_b / 32) + ceil(N / 32) tile columns (a row block that sees fewer
// tree tiles skips the excess).  The bands are laid end to end in (request,
// band) order and their columns cut into equal windows: 256 / R of them (32 / R
// per XCD, window x on XCD x % 8), fewer when that would leave a window under
// 8 columns (the surplus workgroups idle).  Workgroup (window x, slot j) takes row block
// j of every band piece in window x, so every CU carries the same number of
// tiles however ragged the prefixes are, and the R workgroups of a window walk
// the same columns in step (one KV stream per window).  A band cut by a window
// edge leaves one partial (o, lse) per window it touches, at a slot fixed by
// (window, slot, head or tail of the window); the band combine kernel merges
// them.

__device__ __forceinline__ int64_t request_len(const int64_t* off, int b) {
  const int64_t L = off[b + 1] - off[b];
  return L > 0 ? L : 0;
}
__device__ __forceinline__ int band_tiles(const int64_t* off, int b, int ntt) {
  return (int)((request_len(off, b) + KT - 1) / KT) + ntt;
}
// Row blocks per band for n_rb row blocks per request.
__device__ __forceinline__ int band_row_blocks(int n_rb) { return n_rb % kBandRowBlocks == 0 ? kBandRowBlocks : n_rb; }

// Total band columns over all requests (same value in every lane).
__device__ int64_t band_columns_total(const int64_t* off, int B, int nb, int ntt) {
  const int lane = threadIdx.x & 63;
  long long sum = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    long long c = b < B ? (long long)nb * band_tiles(off, b, ntt) : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
    sum += c;
  }
  return sum;
}

// The first request whose columns end after column X, and in S the column its
// first band starts at; B (with S = the total) if X is past the end.
__device__ int band_find(const int64_t* off, int B, int nb, int ntt, int64_t X, int64_t& S) {
  const int lane = threadIdx.x & 63;
  long long carry = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const long long c = b < B ? (long long)nb * band_tiles(off, b, ntt) : 0;
    long long inc = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(inc, d);
      if (lane >= d) inc += y;
    }
    const unsigned long long hit = __ballot(b < B && carry + inc > X);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      S = carry + __shfl(inc - c, l);
      return b0 + l;
    }
    carry += __shfl(inc, 63);
  }
  S = carry;
  return B;
}

__device__ __forceinline__ int64_t window_edge(int64_t C, int x, int windows) { return C * x / windows; }

// Partial slot of workgroup (window, slot): the band cut at the window's start
// (head) or the one cut at its end (tail).  A window inside one band has only a head.
__device__ __forceinline__ int band_part_slot(int win, int slot, int rbb, bool head) {
  return (win * rbb + slot) * 2 + (head ? 0 : 1);
}

struct PieceCursor {
  int b, k;          // request, band within the request
  int Tb;            // columns of request b's bands
  int nb, ntt;       // bands per request, tree tiles of a band
  int rbb;           // row blocks per band
  int win, slot;     // window and row block within each band
  int64_t S;         // first column of request b
  int64_t X0, X1;    // the window's columns
  int64_t p0, L;     // request b's first cache row and prefix length
};

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The cursor read back from LDS, made wave-uniform (scalar registers).
__device__ __forceinline__ PieceCursor uniform_cursor(const PieceCursor& v) {
  PieceCursor c;
  c.b = __builtin_amdgcn_readfirstlane(v.b);
  c.k = __builtin_amdgcn_readfirstlane(v.k);
  c.Tb = __builtin_amdgcn_readfirstlane(v.Tb);
  c.nb = __builtin_amdgcn_readfirstlane(v.nb);
  c.rbb = __builtin_amdgcn_readfirstlane(v.rbb);
  c.ntt = __builtin_amdgcn_readfirstlane(v.ntt);
  c.win = __builtin_amdgcn_readfirstlane(v.win);
  c.slot = __builtin_amdgcn_readfirstlane(v.slot);
  c.S = uniform64(v.S);
  c.X0 = uniform64(v.X0);
  c.X1 = uniform64(v.X1);
  c.p0 = uniform64(v.p0);
  c.L = uniform64(v.L);
  return c;
}

// Windows this short (in tile columns) with 32 row blocks per band take the
// slot-major mapping below: a window's KV (36 KB a column) is then smaller than
// the queries of an XCD's 32 row blocks (4.7 MB), which all start at once.
constexpr int kSlotMajorMaxColumns = 4 * kBandRowBlocks;

__device__ PieceCursor band_cursor_start(const AttnArgs& a, int n_rb, int block) {
  PieceCursor c;
  c.rbb = band_row_blocks(n_rb);
  c.nb = n_rb / c.rbb;
  c.ntt = (a.N + KT - 1) / KT;
  // Up to 64 requests: lane l loads request l's bounds once, and the column
  // total, the search for the window's first request and that request's bounds
  // all come from those registers.  More requests: scans in chunks of 64.
  const bool one_chunk = a.B <= 64;
  const int lane = threadIdx.x & 63;
  int64_t o0 = 0, Lb = 0, cols = 0, inc = 0;
  int64_t C;
  if (one_chunk) {
    if (lane < a.B) {
      o0 = a.prefix_offsets[lane];
      Lb = max<int64_t>(a.prefix_offsets[lane + 1] - o0, 0);
      cols = (int64_t)c.nb * ((Lb + KT - 1) / KT + c.ntt);
    }
    inc = cols;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = __shfl_up(inc, d);
      if (lane >= d) inc += y;
    }
    C = uniform64(__shfl(inc, 63));
  } else {
    C = uniform64(band_columns_total(a.prefix_offsets, a.B, c.nb, c.ntt));
  }
  // at least kBandMinWindowColumns columns a window (bounds the pieces per band,
  // and so the partial traffic, and keeps every window non-empty)
  const int windows = (int)min<int64_t>(a.band_windows, max<int64_t>(1, C / kBandMinWindowColumns));
  // Workgroup i runs on XCD i % 8.  Window-major (the default): the R workgroups
  // of window x run on XCD x % 8, so each KV tile is fetched once per L2 and each
  // XCD loads the queries of all R row blocks.  Slot-major (R = 32, short
  // windows): XCD x runs row blocks 4x .. 4x + 3 of every window, so each row
  // block's queries are fetched once per L2 and the short windows' KV streams to
  // all 8 XCDs instead.  Both are bijections of the 256 workgroups.
  const int idx = block / kBandXcds, xcd = block % kBandXcds;
  if (c.rbb == kBandRowBlocks && C <= (int64_t)windows * kSlotMajorMaxColumns) {
    constexpr int per_xcd = kBandRowBlocks / kBandXcds;   // 4
    c.slot = xcd * per_xcd + idx % per_xcd;
    c.win = idx / per_xcd;
  } else {
    c.slot = idx % c.rbb;
    c.win = (idx / c.rbb) * kBandXcds + xcd;
  }
  c.X0 = c.win < windows ? window_edge(C, c.win, windows) : C;
  c.X1 = c.win < windows ? window_edge(C, c.win + 1, windows) : C;
  int64_t S;
  c.k = 0;
  c.Tb = 1;
  c.p0 = 0;
  c.L = 0;
  if (one_chunk) {
    const unsigned long long hit = __ballot(lane < a.B && inc > c.X0);
    c.b = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : a.B);
    S = C;
    if (c.b < a.B) {
      S = __shfl(inc - cols, c.b);
      c.p0 = uniform64(__shfl(o0, c.b));
      c.L = uniform64(__shfl(Lb, c.b));
    }
  } else {
    c.b = __builtin_amdgcn_readfirstlane(band_find(a.prefix_offsets, a.B, c.nb, c.ntt, c.X0, S));
    if (c.b < a.B) {
      c.p0 = a.prefix_offsets[c.b];
      c.L = max<int64_t>(a.prefix_offsets[c.b + 1] - c.p0, 0);
    }
  }
  c.S = uniform64(S);
  if (c.b < a.B) {
    c.Tb = (int)((c.L + KT - 1) / KT) + c.ntt;
    c.k = (int)((c.X0 - c.S) / c.Tb);
  }
  // Workgroup (window x > 0, slot 0) describes edge x for the combine kernel:
  // {cut here first, request, band, last window the band reaches}.  The band
  // holding column X_x is cut first at x when it starts inside window x - 1
  // (at or after X_{x-1}, before X_x).  Window 0's slot 0 stores {C, windows}.
  // The workspace holds records for the host's window bound only (the combine
  // kernel reads edges below the window count, which never exceeds it).
  if (c.slot == 0 && threadIdx.x == 0 && c.win < a.band_windows) {
    if (c.win == 0) {
      reinterpret_cast<int4*>(a.band_edges)[0] =
          make_int4((int)(uint32_t)(uint64_t)C, (int)(uint32_t)((uint64_t)C >> 32), windows, 0);
    } else {
      int4 d = make_int4(0, 0, 0, 0);
      if (c.win < windows && c.b < a.B) {
        const int64_t bs = c.S + (int64_t)c.k * c.Tb, be = bs + c.Tb;
        if (bs != c.X0 && window_edge(C, c.win - 1, windows) <= bs) {
          int last = c.win;
          while (last + 1 < windows && window_edge(C, last + 1, windows) < be) ++last;
          d = make_int4(1, c.b, c.k, last);
        }
      }
      reinterpret_cast<int4*>(a.band_edges)[c.win] = d;
    }
  }
  return c;
}

// The next piece's first band column bs; false when the window is done.
__device__ __forceinline__ bool band_cursor_piece(const AttnArgs& a, const PieceCursor& c, int64_t& bs) {
  if (c.X0 >= c.X1 || c.b >= a.B) return false;
  bs = c.S + (int64_t)c.k * c.Tb;
  return bs < c.X1;
}

__device__ __forceinline__ void band_cursor_next(const AttnArgs& a, PieceCursor& c) {
  if (++c.k < c.nb) return;
  c.k = 0;
  c.S += (int64_t)c.nb * c.Tb;
  if (++c.b < a.B) {
    c.p0 = a.prefix_offsets[c.b];
    c.L = max<int64_t>(a.prefix_offsets[c.b + 1] - c.p0, 0);
    c.Tb = (int)((c.L + KT - 1) / KT) + c.ntt;
  }
}

constexpr int KRING = 4;   // K-fragment reads in flight ahead of the S^T MFMAs
constexpr int QREG = DL / 16 - 4;   // latent query k-steps held in VGPRs; the last 4 are staged in LDS
constexpr int kQRowBytes = QREG * 32;                  // 896: a row's VGPR k-steps
constexpr int kQRowChunks = kQRowBytes / 16;           // 56
constexpr int kQRegionBytes = 32 * kQRowBytes;         // a wave's 32 rows: 28 KB
constexpr int kPloBytes = NWAVES * 64 * 32;
static_assert(NWAVES * kQRegionBytes <= NBUF * TILE_BYTES + kPloBytes, "the query copy fits the ring and s_plo");
static_assert(kQRegionBytes % 1024 == 0 && kQRowChunks % 8 == 0, "whole 1 KB copies; the chunk swizzle stays in a row");
static_assert(DL / 16 - QREG == DR / 16, "the staged latent queries use the rotary pair-row layout");
constexpr int VRING = 3;   // V^T-fragment reads (pairs) in flight ahead of the O^T MFMAs
// s_waitcnt operand: lgkmcnt(n), no vmcnt or expcnt wait
constexpr int lgkm_wait(int n) { return 0xC07F | (n << 8); }

constexpr int NST = 2 * (DL / 32);         // O^T MFMAs per tile: 2 key steps x 16 dim blocks
// O^T step st of a tile (st a constant after unrolling): the read of V^T fragment
// st + VRING is issued first, one LDS wait covers each pair of MFMAs (VRING - 1
// younger pairs in flight), then O^T block db += V^T fragment st . P^T of key step ks.
__device__ __forceinline__ void o_step(f32x16 (&oacc)[DL / 32], bf16x8 (&vring)[VRING], const bf16x8 (&pb)[2],
                                       const unsigned char* buf, int voff, int voff_hi, int st) {
  const int ks = st / (DL / 32), db = st % (DL / 32);
  const bf16x8 vf = vring[st % VRING];
  if (st + VRING < NST) vring[st % VRING] = load_vt(buf, voff, voff_hi, (st + VRING) / (DL / 32), (st + VRING) % (DL / 32));
  if (st % 2 == 0 && st + 1 < NST) __builtin_amdgcn_s_waitcnt(lgkm_wait(2 * (VRING - 1)));
  if (st == 0)
    mfma_o_first(oacc[db], vf, pb[ks]);
  else
    mfma_o(oacc[db], vf, pb[ks]);
}
// O^T MFMAs of tile t issued before the probabilities of tile t + 1 are prepared
// (they need neither), so that the MFMA pipe stays busy across that code.
constexpr int O_HEAD = 4;
static_assert(NST - O_HEAD >= 20, "the P pipeline needs 20 O^T steps");

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
verify_attn_bf16_kernel(AttnArgs a) {
  // the KV ring, then the second-term buffer s_plo (one array: the query copy at
  // the start of a piece uses the first NWAVES * kQRegionBytes bytes of both)
  __shared__ __attribute__((aligned(1024))) unsigned char s_kv[NBUF * TILE_BYTES + kPloBytes];
  __shared__ uint32_t s_mask[ROWS][MAXW];
  // queries of the last QREG_LDS latent k-steps (part 0) and the rotary ones (part 1), swizzled pair rows
  __shared__ __attribute__((aligned(16))) unsigned char s_qx[2 * ROWS * R_ROW];
  __shared__ PieceCursor s_cur[2];   // the current piece's cursor and the next one's
  // second bf16 term of P of one tile, per lane, in the lane's B-operand layout
  unsigned char* const s_plo = s_kv + NBUF * TILE_BYTES;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int lane = tid & 63;
  const int g = lane >> 5;          // which 8-wide k half of an MFMA operand
  const int lr = lane & 31;         // row within the wave's 32 rows

  // ---- LDS addresses (lane constants) ----
  const int kbase = lr * C_ROW + ((g ^ swz(lr)) << 4);   // K fragment, k-step 0
  // V^T fragment (A of O^T) by transpose read.  Lane = 16 G + 4 rr + cc reads key
  // 16 ks + 4 g + rr (+8 for the second read), dims 32 db + 16 (G & 1) + 4 cc .. +3,
  // i.e. logical chunk 4 db + 2 (G & 1) + (cc >> 1), byte 8 (cc & 1) in it.
  int voff;
  {
    const int G = lane >> 4;
    const int rr = (lane >> 2) & 3;
    const int cc = lane & 3;
    const int vkey = 4 * g + rr;
    voff = vkey * C_ROW + (((2 * (G & 1) + (cc >> 1)) ^ swz(vkey)) << 4) + (cc & 1) * 8;
  }
  const int voff_hi = (voff ^ 32) + 8 * C_ROW;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)s_kv;   // LDS byte address of the ring
  CopyLanes clanes;
  {
    clanes.lw = (uint32_t)((lane << 4) ^ (wave << 6));
    const int pr = wave * 4 + (lane >> 4);
    const int logical = (lane & 15) ^ (pr & 7);
    clanes.rkey = 2 * pr + (logical >> 3);
    clanes.rpiece = (uint32_t)((logical & 7) * 16);
  }

  // ---- the workgroup's pieces of work: (request, row block, tile range, destination) ----
  const int n_rows = a.N * a.H;
  const int n_rb = (n_rows + ROWS - 1) / ROWS;
  const int64_t total_rows = (int64_t)a.B * n_rows;
  // The band cursor lives in LDS between pieces, so that none of it is held in
  // registers across the tile loop.  Piece i reads s_cur[i & 1] and writes the
  // next piece's cursor to s_cur[(i + 1) & 1] as soon as it is known; the next
  // piece's first barrier orders that write before its reads.
  if (a.balanced) {
    const PieceCursor c = band_cursor_start(a, n_rb, blockIdx.x);
    if (tid == 0) s_cur[0] = c;
  }
  bool single_done = false;
  int cur_slot = 0;

  for (;;) {
  __syncthreads();   // the cursor is visible; every wave is done with the previous piece's LDS
  int b, rb, t0, t1;
  bool to_part;                   // partial result (workspace) or final (o, lse)
  int64_t dest0;                  // destination row of the piece's row 0
  int64_t p0, L;
  int n_pt;
  if (a.balanced) {
    const PieceCursor cur = uniform_cursor(s_cur[cur_slot]);
    int64_t bs;
    if (!band_cursor_piece(a, cur, bs)) break;
    b = cur.b;
    rb = cur.k * cur.rbb + cur.slot;
    const int64_t be = bs + cur.Tb;
    t0 = (int)(max(cur.X0, bs) - bs);
    t1 = (int)(min(cur.X1, be) - bs);
    to_part = !(bs >= cur.X0 && be <= cur.X1);   // a piece of a band cut by a window edge
    dest0 = to_part ? (int64_t)band_part_slot(cur.win, cur.slot, cur.rbb, bs < cur.X0) * ROWS
                    : (int64_t)b * n_rows + (int64_t)rb * ROWS;
    PieceCursor nxt = cur;
    band_cursor_next(a, nxt);
    cur_slot ^= 1;
    if (tid == 0) s_cur[cur_slot] = nxt;
    p0 = cur.p0;
    L = cur.L;
    n_pt = (int)((L + KT - 1) / KT);
    const int last_row = min(n_rows - 1, rb * ROWS + ROWS - 1);
    t1 = min(t1, n_pt + (last_row / a.H) / KT + 1);   // tree tiles this row block can see
  } else {
    // uniform KV splits: one piece, item (request, row block, split)
    if (single_done) break;
    single_done = true;
    int item = xcd_local_item(blockIdx.x, gridDim.x);
    const int split = item % a.splits;
    item /= a.splits;
    rb = item % n_rb;
    b = item / n_rb;
    p0 = a.prefix_offsets[b];
    L = max<int64_t>(a.prefix_offsets[b + 1] - p0, 0);
    n_pt = (int)((L + KT - 1) / KT);
    const int last_row = min(n_rows - 1, rb * ROWS + ROWS - 1);
    const int n_tt = (last_row / a.H) / KT + 1;     // tree tiles that any row here can see
    const int T = n_pt + n_tt;
    t0 = (int)((int64_t)split * T / a.splits);
    t1 = (int)((int64_t)(split + 1) * T / a.splits);
    const int64_t row0 = (int64_t)b * n_rows + (int64_t)rb * ROWS;
    to_part = a.splits > 1;
    dest0 = to_part ? (int64_t)split * total_rows + row0 : row0;
  }

  // ---- query fragments: B operand, lane (lr, g) holds Q[row lr][16 s + 8 g .. +8] ----
  // The 32 latent k-steps stay in VGPRs; the 4 rotary k-steps are staged in LDS
  // in the rotary pair-row layout (row rl at pair row rl >> 1) and read per tile.
  const int r_loc = rb * ROWS + wave * 32 + lr;
  const bool row_ok = r_loc < n_rows;
  const int row_local = wave * 32 + lr;
  bf16x8 qf[QREG];
  {
    // Each wave copies its own 32 rows into LDS with direct-to-LDS loads (1 KB
    // of consecutive 16-byte chunks per load): the k-steps held in VGPRs into
    // a kQRegionBytes region at the start of the ring (row rr at kQRowBytes rr,
    // its chunk q at position q ^ (rr & 7)), the staged k-steps and the rotary
    // part straight into s_qx (the wave's rows are pair rows 16 wave .. 16 wave
    // + 15 there, 4 KB a part).  Rows past the request's last row re-read its
    // last row, and their fragments are zeroed once the copies have landed.
    const int w_row0 = rb * ROWS + wave * 32;          // wave-uniform
    const int w_base = min(w_row0, n_rows - 1);
    const int w_last = n_rows - 1 - w_base;            // rows of the wave that exist, less one
    const int64_t brow = (int64_t)b * n_rows + w_base;
    const unsigned char* qlb = static_cast<const unsigned char*>(a.q_lat) + brow * (DL * 2);
    const unsigned char* qrb = static_cast<const unsigned char*>(a.q_rope) + brow * (DR * 2);
    // (lane values go through opaque() so that they are computed here, not
    // hoisted out of the piece loop and spilled)
    const uint32_t region = lds0 + (uint32_t)(wave * kQRegionBytes);
#pragma unroll
    for (int i = 0; i < kQRegionBytes / 1024; ++i) {
      const int c = 64 * i + opaque(lane);
      const int rr = c / kQRowChunks;
      const int q = (c - rr * kQRowChunks) ^ (rr & 7);
      lds_dma16_rotary(region + 1024 * i, qlb, (uint32_t)(min(rr, w_last) * (DL * 2)), (uint32_t)(q * 16));
    }
    const uint32_t sqx = (uint32_t)(uintptr_t)(lds_void_t*)s_qx + (uint32_t)(wave * 4096);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ln = opaque(lane);
      const int pr = 16 * wave + 4 * j + (ln >> 4);
      const int logical = (ln & 15) ^ (pr & 7);
      const int rr = min(2 * pr + (logical >> 3) - 32 * wave, w_last);
      const uint32_t piece = (uint32_t)((logical & 7) * 16);
      lds_dma16_rotary(sqx + 1024 * j, qlb, (uint32_t)(rr * (DL * 2)), piece + QREG * 32);
      lds_dma16_rotary(sqx + ROWS * R_ROW + 1024 * j, qrb, (uint32_t)(rr * (DR * 2)), piece);
    }
    // ---- per-row mask words (LDS), loaded while the query copies are in flight ----
    const int W = (a.N + 31) >> 5;
    for (int e = tid; e < ROWS * MAXW; e += 256) {
      const int rl = e / MAXW, w = e % MAXW;
      const int r = rb * ROWS + rl;
      uint32_t v = 0u;
      if (r < n_rows && w < W) v = a.mask[((int64_t)b * a.N + r / a.H) * W + w];
      s_mask[rl][w] = v;
    }

    wait_copies();   // this wave's copies have landed
    // chunk 2 s + g of row lr sits at 128 (s >> 2) + 16 ((2 (s & 3) + g) ^ (lr & 7)):
    // four lane bases, the rest immediate offsets
    const int lro = opaque(lr);
    const unsigned char* qrow = s_kv + wave * kQRegionBytes + lro * kQRowBytes;
#pragma unroll
    for (int s = 0; s < QREG; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + (((2 * (s & 3) + g) ^ (lro & 7)) << 4) + (s >> 2) * 128);
      qf[s] = row_ok ? v : bf16x8{};
    }
    if (!row_ok) {
#pragma unroll
      for (int c = g; c < 8; c += 2) {
        *reinterpret_cast<bf16x8*>(s_qx + (row_local >> 1) * 256 + (pair_chunk(row_local, c) << 4)) = bf16x8{};
        *reinterpret_cast<bf16x8*>(s_qx + ROWS * R_ROW + (row_local >> 1) * 256 + (pair_chunk(row_local, c) << 4)) =
            bf16x8{};
      }
    }
  }

  // ---- accumulators and softmax state (one query row per lane) ----
  // Each row's probabilities are taken relative to a fixed reference m_ref:
  // the maximum score of the first tile in which the row sees any key (the
  // output and the exp-sum are exactly zero before that, so nothing needs
  // rescaling).  Later scores may exceed the reference by up to 2^100, which
  // bf16 P and the float32 accumulators hold without overflow, so the
  // accumulators are never rescaled.  Should a score exceed that headroom,
  // the workgroup runs its tiles once more with the row's true maximum
  // (tracked in m_max) as the reference; that pass cannot overflow.
  f32x16 oacc[DL / 32];
  float m_ref = -INFINITY;   // reference max, log2 units
  float m_max = -INFINITY;   // true max of the scores seen, log2 units
  float l_run = 0.f;         // this lane's half of the row's exp-sum
  const float c_log2 = a.scale * 1.4426950408889634f;
  // The second bf16 term of P (slow-path tiles) serves rows that see only a few
  // keys.  A piece with kTwoTermMinFullTiles or more full prefix tiles gives every
  // row at least that many tiles of keys, and single terms (as on the fast path)
  // then suffice on its slow tiles too.
  const int64_t full_end = min<int64_t>((int64_t)t1, L / KT);
  const bool two_term = full_end - t0 < kTwoTermMinFullTiles;

  // Ring slot 2 starts zeroed: the first PV of a pass runs on it with a zero P
  // (once every wave has read its queries out of the ring).
  __syncthreads();
  for (int i = tid; i < TILE_BYTES / 16; i += 256)
    reinterpret_cast<uint4*>(s_kv + 2 * TILE_BYTES)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  for (int pass = 0; pass < 2; ++pass) {
  bool overflow = false;
  l_run = 0.f;
#pragma unroll
  for (int db = 0; db < DL / 32; ++db) oacc[db] = f32x16{};

  // Software pipeline: iteration t runs QK of tile t + 1, then PV of tile t, and
  // computes P of tile t + 1 in the shadow of the PV MFMAs.  Tile t + 1 lives in
  // ring slot (j + 1) % 3, tile t in j % 3; the copies of tile t + 2 go to slot
  // (j + 2) % 3, whose last reader (PV of tile t - 1) every wave has finished
  // by the barrier at the top of iteration t.

  // ---- prologue: tile t0 in flight ----
  bf16x8 pb[2] = {bf16x8{}, bf16x8{}};
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): nothing of the compiler's pending inside the loop
  if (t0 < t1) {
    const CopyPlan cp0 = copy_plan(a, b, p0, L, n_pt, t0);
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) issue_copy(cp0, clanes, lds0, wave, i);
  }
  int slot = 2;                          // ring slot of tile t (t0 - 1: none)
  bool lo_t = false;                     // tile t carries a second P term (s_plo)

  for (int t = t0 - 1; t < t1; ++t) {
    const int slot_n = slot == 2 ? 0 : slot + 1;      // tile t + 1
    const int slot_d = slot_n == 2 ? 0 : slot_n + 1;  // tile t + 2
    const int tn = t + 1;

    // ---- second term of P for tile t (slow-path tiles only): O^T += V^T . P_lo^T,
    // P_lo staged by this lane in s_plo when tile t was prepared ----
    if (lo_t) {
      const unsigned char* buf = s_kv + slot * TILE_BYTES;
      const bf16x8* pl = reinterpret_cast<const bf16x8*>(s_plo + (wave * 64 + lane) * 32);
      const bf16x8 plo0 = pl[0], plo1 = pl[1];
#pragma unroll
      for (int st = 0; st < 2 * (DL / 32); ++st) {
        const int ks = st / (DL / 32), db = st % (DL / 32);
        mfma_o(oacc[db], load_vt(buf, voff, voff_hi, ks, db), ks ? plo1 : plo0);
      }
    }

    // The first VRING V^T fragments of tile t (the A operands of its first O^T
    // MFMAs) are read during the last S^T MFMAs of tile tn, or here when there is
    // no tile tn: slot t is complete since the previous barrier, and the O^T
    // stream then starts without an LDS round trip.
    constexpr int S_STEPS = DL / 16 + DR / 16;
    constexpr int VT_EARLY = S_STEPS - KRING;     // first S^T step with no K read to issue
    static_assert(VT_EARLY + VRING <= S_STEPS, "the early V^T reads fit after the last K read");
    const unsigned char* obuf = s_kv + slot * TILE_BYTES;
    bf16x8 vring[VRING];

    f32x16 sn;                    // S^T, then exponents, of tile tn
    float c, m, m_abs;
    bool lo_n = false;            // tile tn carries a second P term
    if (tn < t1) {
      wait_copies();              // this wave's copies of tile tn have landed
      __syncthreads();            // ... and every wave's; every wave is done with tile t - 1

      // ---- S^T[key][row] = K . Q^T over 576 dims for tile tn; K-fragment reads
      // KRING steps ahead, rotary query fragments QRING ahead.  The copies of tile
      // tn + 1 are issued once the first fragment reads are in flight. ----
      {
        const unsigned char* kbuf = s_kv + slot_n * TILE_BYTES;
        constexpr int QRING = 2;
        bf16x8 kring[KRING];
        bf16x8 qrr[QRING];
#pragma unroll
        for (int s = 0; s < KRING; ++s) kring[s] = *reinterpret_cast<const bf16x8*>(kbuf + kaddr(kbase, s));
        // tile tn + 1 (past the end: tile t1 - 1 again, into the free slot, so
        // that the copies need no branch); one copy every fourth S^T MFMA
        const CopyPlan cplan = copy_plan(a, b, p0, L, n_pt, min(tn + 1, t1 - 1));
        const uint32_t lds_d = lds0 + slot_d * TILE_BYTES;
#pragma unroll
        for (int s = 0; s < S_STEPS; ++s) {
          const bf16x8 kf = kring[s % KRING];
          const int nx = s + KRING;
          if (nx < DL / 16) {
            kring[s % KRING] = *reinterpret_cast<const bf16x8*>(kbuf + kaddr(kbase, nx));
          } else if (nx < DL / 16 + DR / 16) {   // rotary key rows
            const int cc = 2 * (nx - DL / 16) + g;
            kring[s % KRING] =
                *reinterpret_cast<const bf16x8*>(kbuf + R_OFF + (lr >> 1) * 256 + (pair_chunk(lr, cc) << 4));
          }
          const bf16x8 qv = s < QREG ? qf[s] : qrr[s % QRING];
          const int nq = s + QRING;
          if (nq >= QREG && nq < DL / 16 + DR / 16) {   // queries staged in s_qx
            const int part = nq >= DL / 16;
            const int cc = 2 * (part ? nq - DL / 16 : nq - QREG) + g;
            qrr[nq % QRING] = *reinterpret_cast<const bf16x8*>(s_qx + part * ROWS * R_ROW + (row_local >> 1) * 256 +
                                                               (pair_chunk(row_local, cc) << 4));
          }
          if (s % 4 == 1 && s / 4 < LOADS_PER_WAVE) issue_copy(cplan, clanes, lds_d, wave, s / 4);
          // one LDS wait per pair of MFMAs: K fragments s and s + 1 (KRING - 1 younger reads in
          // flight); past the last K read the compiler's own waits cover the remaining steps
          if (s % 2 == 0 && s < VT_EARLY) __builtin_amdgcn_s_waitcnt(lgkm_wait(KRING - 1));
          if (s == 0)
            mfma_s_first(sn, kf, qv);
          else if (s == S_STEPS - 1)
            mfma_s_last(sn, kf, qv);
          else
            mfma_s(sn, kf, qv);
          if (s >= VT_EARLY && s < VT_EARLY + VRING) {
            const int st = s - VT_EARLY;
            vring[st] = load_vt(obuf, voff, voff_hi, st / (DL / 32), st % (DL / 32));
          }
          __builtin_amdgcn_sched_barrier(0);   // each step's reads and copy stay with its MFMA
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < VRING; ++st) vring[st] = load_vt(obuf, voff, voff_hi, st / (DL / 32), st % (DL / 32));
    }

    // ---- O^T[dim][row] += V^T[dim][key] . P^T[key][row] for tile t (the pass's first
    // iteration multiplies a zero P with the zero-filled slot 2), V^T read VRING steps
    // ahead: the first O_HEAD steps here, the rest below with P of tile tn in their shadow.
#pragma unroll
    for (int st = 0; st < O_HEAD; ++st) o_step(oacc, vring, pb, obuf, voff, voff_hi, st);

    if (tn < t1) {
      // ---- scores -> exponent form.  sn[4 jj + i] is key 8 jj + 4 g + i of row lr.
      // P element e is 2^(c * sn[e] - m).  Full prefix tiles, once every row has its
      // reference, use (c, m) = (scale * log2 e, m_ref) directly.  Other tiles (the
      // partial last prefix tile, tree tiles, a row's first visible tile) are masked
      // here: sn becomes the masked exponent itself and (c, m) = (1, 0), and a row's
      // first visible tile fixes its reference.  m_abs is the absolute value (log2
      // units) the exponents are relative to. ----
      const bool fast = tn < n_pt && (int64_t)(tn + 1) * KT <= L &&
                        __builtin_amdgcn_ballot_w64(m_ref == -INFINITY) == 0;
      if (fast) {
        c = c_log2;
        m = m_ref;
        m_abs = m_ref;
      } else {
        float sc[16];
        if (tn < n_pt) {
          const int count = (int)min<int64_t>(L - (int64_t)tn * KT, KT);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + 4 * g + (e & 3);
            sc[e] = key < count ? sn[e] * c_log2 : -INFINITY;
          }
        } else {
          // the row offset is recomputed here (opaque to the optimiser) rather
          // than carried round the loop in a register
          const int mrow = opaque(row_local * MAXW);
          const uint32_t word = (&s_mask[0][0])[mrow + (tn - n_pt)] >> (4 * g);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 8 * (e >> 2) + (e & 3);          // + 4 g, folded into the shift above
            sc[e] = ((word >> key) & 1u) ? sn[e] * c_log2 : -INFINITY;
          }
        }
        float mx = sc[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
        mx = halves_max(mx);
        if (m_ref == -INFINITY) m_ref = mx;            // first visible keys fix the row's reference
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
        for (int e = 0; e < 16; ++e) sn[e] = sc[e] - m_use;
        c = 1.f;
        m = 0.f;
        m_abs = m_use;
        // P = hi + lo with both terms bf16: hi is what the shadow below rounds
        // 2^sn to (the same exp2 of the same exponent), lo the rounded
        // remainder, applied by a second O^T pass over this tile next
        // iteration.  Tiles on this path (tree tiles, a partial last prefix
        // tile, a row's first visible tile) hold every key of the rows that see
        // only a few, where a single bf16 term would leave a 2^-9 relative
        // error uncancelled.
        if (two_term) {
          bf16x8 lo[2];
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(sn[e]), p1 = __builtin_amdgcn_exp2f(sn[e + 1]);
            bf16x2 pr;
            pr[0] = (__bf16)(p0 - (float)(__bf16)p0);
            pr[1] = (__bf16)(p1 - (float)(__bf16)p1);
            lo[e >> 3][e & 7] = pr[0];
            lo[e >> 3][(e + 1) & 7] = pr[1];
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, kBf16Ones, l_run, false);
          }
          bf16x8* pl = reinterpret_cast<bf16x8*>(s_plo + (wave * 64 + lane) * 32);
          pl[0] = lo[0];
          pl[1] = lo[1];
          lo_n = true;
        }
      }
    } else {
      // nothing after this tile: the shadow work below evaluates to p = 0
#pragma unroll
      for (int e = 0; e < 16; ++e) sn[e] = 0.f;
      c = 0.f;
      m = INFINITY;
      m_abs = 0.f;
    }

    // ---- the remaining O^T steps of tile t; P of tile tn (one element per MFMA),
    // then its row max, in their shadow. ----
    bf16x8 pn[2];
    float pe[16];
    float mx = -INFINITY;
    {
#pragma unroll
      for (int st = O_HEAD; st < NST; ++st) {
        o_step(oacc, vring, pb, obuf, voff, voff_hi, st);
        // three-stage pipeline over the 16 elements, so that the VALU work of one
        // step is independent: exponent of element q, 2^x and row max of q - 1,
        // bf16 pair and exp-sum of q - 2 (q = st - O_HEAD).  The exp-sum adds the
        // bf16-rounded values the O^T MFMAs use (one dot2 per pair), so the weights
        // applied to V sum to exactly the normaliser.
        const int q = st - O_HEAD;
        if (q < 16) sn[q] = __builtin_fmaf(sn[q], c, -m);
        if (q >= 1 && q <= 16) {
          pe[q - 1] = __builtin_amdgcn_exp2f(sn[q - 1]);
          mx = fmaxf(mx, sn[q - 1]);
        }
        if (q >= 2 && q <= 17) {
          const int e = q - 2;
          if (e & 1) {
            bf16x2 pr;
            pr[0] = (__bf16)pe[e - 1];
            pr[1] = (__bf16)pe[e];
            pn[e >> 3][(e - 1) & 7] = pr[0];
            pn[e >> 3][e & 7] = pr[1];
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, kBf16Ones, l_run, false);
          }
        }
        if (q == 18) mx = halves_max(mx);
        if (q == 19) {
          m_max = fmaxf(m_max, m_abs + mx);
          overflow |= mx > kHeadroomLog2;
        }
        // Keep each step's share of the P pipeline next to its MFMA: left free,
        // the scheduler bunches these VALU instructions between a few MFMAs, in
        // a pattern that shifts with code elsewhere in the kernel.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    pb[0] = pn[0];
    pb[1] = pn[1];
    slot = slot_n;
    lo_t = lo_n;
  }
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");   // last O^T MFMA -> AGPR reads / rewrites
  wait_copies();   // the repeated copy of the last tile (if any) has landed

  // rare: a score beyond the headroom anywhere in the workgroup -> one more pass
  if (!__syncthreads_or(overflow ? 1 : 0)) break;
  m_ref = m_max;
  }

  // ---- epilogue ----
  const float l_tot = halves_sum(l_run);
  if (row_ok && !to_part) {
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_ref + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    float* orow = a.o + (dest0 + row_local) * DL;
    // oacc[db][4 jj + i] is dim 32 db + 8 jj + 4 g + i of row lr
#pragma unroll
    for (int db = 0; db < DL / 32; ++db) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float4 v;
        v.x = oacc[db][4 * jj + 0] * inv_l;
        v.y = oacc[db][4 * jj + 1] * inv_l;
        v.z = oacc[db][4 * jj + 2] * inv_l;
        v.w = oacc[db][4 * jj + 3] * inv_l;
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * jj + 4 * g) = v;
      }
    }
    if (g == 0) a.lse[dest0 + row_local] = lse;
  } else if (row_ok) {
    // Partial record (see partial_chunk_dim): the unnormalised output in fp16,
    // scaled by 2^(14 - e) so that the row's largest magnitude lies in [2^13,
    // 2^14), and {lse2, k} in log2 units: the piece adds 2^lse2 to the merged
    // exp-sum and 2^k times the stored values to the merged numerator.
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < DL / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(oacc[db][e]));
    amax = halves_max(amax);
    int ex = 0;
    if (amax <= 3.4e38f) frexpf(amax, &ex);   // amax = f 2^ex, f in [0.5, 1); 0, inf, NaN: ex = 0
    const int sh = kPartialTopExp - ex;
    f16x8* prow = reinterpret_cast<f16x8*>(static_cast<_Float16*>(a.part_o) + (dest0 + row_local) * DL);
    // chunk 4 db + 2 jp + g of the row is oacc[db][8 jp .. 8 jp + 7] of lane (lr, g)
#pragma unroll
    for (int db = 0; db < DL / 32; ++db) {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        f16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (_Float16)ldexpf(oacc[db][8 * jp + i], sh);
        prow[4 * db + 2 * jp + g] = v;
      }
    }
    if (g == 0) {
      const bool seen = l_tot > 0.f;
      a.part_aux[dest0 + row_local] =
          make_float2(seen ? m_ref + log2f(l_tot) : -INFINITY, seen ? m_ref - (float)sh : -INFINITY);
    }
  }
  }   // pieces
}

// Partial records: dims of fp16 chunk c (8 values) of a row.  Values 0..3 are
// dims 32 db + 16 jp + 4 gg + (0..3), values 4..7 the same + 8, with db = c / 4,
// jp = (c / 2) % 2, gg = c % 2 (the order the attention kernel's lanes hold them).
__device__ __forceinline__ int partial_chunk_dim(int c) { return 32 * (c >> 2) + 16 * ((c >> 1) & 1) + 4 * (c & 1); }

// Adds w times fp16 chunk v (dims partial_chunk_dim(c) + 0..3 and + 8..11) into acc[0], acc[1].
__device__ __forceinline__ void partial_chunk_fma(float4 (&acc)[2], float w, const f16x8& v) {
  acc[0].x += w * (float)v[0];
  acc[0].y += w * (float)v[1];
  acc[0].z += w * (float)v[2];
  acc[0].w += w * (float)v[3];
  acc[1].x += w * (float)v[4];
  acc[1].y += w * (float)v[5];
  acc[1].z += w * (float)v[6];
  acc[1].w += w * (float)v[7];
}

// Merge split partials (records as written by the attention kernel's epilogue):
// with M = max_s lse2_s, o = sum_s 2^(k_s - M) v_s / sum_s 2^(lse2_s - M) and
// lse = (M + log2 sum_s 2^(lse2_s - M)) ln 2.  One thread per (row, fp16 chunk).
__global__ void __launch_bounds__(256) attn_combine_kernel(const _Float16* __restrict__ part_o,
                                                           const float2* __restrict__ part_aux, int splits,
                                                           int64_t total_rows, float* __restrict__ o,
                                                           float* __restrict__ lse) {
  constexpr int per_row = DL / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = idx / per_row;
  const int c = (int)(idx - row * per_row);
  if (row >= total_rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, part_aux[s * total_rows + row].x);
  float wsum = 0.f;
  float4 acc[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  if (mx != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float2 ax = part_aux[s * total_rows + row];
      if (ax.x == -INFINITY) continue;   // an empty split: exp-sum 0, output 0
      wsum += exp2f(ax.x - mx);
      partial_chunk_fma(acc, exp2f(ax.y - mx),
                        reinterpret_cast<const f16x8*>(part_o + (s * total_rows + row) * DL)[c]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float* orow = o + row * DL + partial_chunk_dim(c);
  *reinterpret_cast<float4*>(orow) = make_float4(acc[0].x * inv, acc[0].y * inv, acc[0].z * inv, acc[0].w * inv);
  *reinterpret_cast<float4*>(orow + 8) = make_float4(acc[1].x * inv, acc[1].y * inv, acc[1].z * inv, acc[1].w * inv);
  if (c == 0) lse[row] = wsum > 0.f ? (mx + log2f(wsum)) * 0.6931471805599453f : -INFINITY;
}

// Band schedule: merge the pieces of every band cut by a window edge.
// Workgroup (pair p, group g) takes edge e = 1 + p / R and slot j = p % R (R = 32
// row blocks per band): if the band at edge e is cut there first (the attention
// kernel's descriptor), rows 8 g .. 8 g + 7 of its row block j, from the tail
// piece of window e - 1 and the head pieces of windows e .. last (no window is
// empty).  With 32 row blocks a band there are at most 256 / 32 = 8 windows, so
// at most 8 pieces: 32 threads per row, lane i < 8 loads piece i's {lse2, k},
// and every lane loads its fp16 chunks c0 and c0 + 32 of all the pieces in the
// same round trip (the loads do not wait for the weights).
constexpr int kCombineRowsPerGroup = 8;
constexpr int kCombineGroups = ROWS / kCombineRowsPerGroup;
constexpr int kCombineMaxPieces = kBandWorkgroups / kBandRowBlocks;   // 8
constexpr int kCombinePiecesInFlight = 8;   // the split kernel: pieces per wave in flight, 2 chunk loads each

__device__ __forceinline__ void store_merged_row(const AttnArgs& a, int64_t grow, int c0, const float4 (&acc)[2][2],
                                                 float wsum, float mx) {
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float* orow = a.o + grow * DL + partial_chunk_dim(c0 + 32 * h);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<float4*>(orow + 8 * q) =
          make_float4(acc[h][q].x * inv, acc[h][q].y * inv, acc[h][q].z * inv, acc[h][q].w * inv);
  }
  if (c0 == 0) a.lse[grow] = wsum > 0.f ? (mx + log2f(wsum)) * 0.6931471805599453f : -INFINITY;
}

__global__ void __launch_bounds__(256) attn_band_combine_kernel(AttnArgs a) {
  const int n_rows = a.N * a.H;
  const int rbb = kBandRowBlocks;
  const int windows = reinterpret_cast<const int4*>(a.band_edges)[0].z;
  const int p = (int)blockIdx.x / kCombineGroups;
  const int grp = (int)blockIdx.x % kCombineGroups;
  if (p >= (windows - 1) * rbb) return;
  const int e = 1 + p / rbb;
  const int j = p % rbb;
  const int4 d = reinterpret_cast<const int4*>(a.band_edges)[e];
  if (!d.x) return;
  const int b = d.y, kb = d.z, n_pc = d.w - e + 2;   // pieces: window e - 1's tail, heads of e .. last
  const int rl = grp * kCombineRowsPerGroup + ((int)threadIdx.x >> 5);
  const int r = (kb * rbb + j) * ROWS + rl;
  if (r >= n_rows) return;
  const int c0 = threadIdx.x & 31;
  const _Float16* part = static_cast<const _Float16*>(a.part_o);
  auto piece_rec = [&](int i) { return (int64_t)band_part_slot(e - 1 + i, j, rbb, i > 0) * ROWS + rl; };
  float2 ax = make_float2(-INFINITY, -INFINITY);
  if (c0 < n_pc) ax = a.part_aux[piece_rec(c0)];
  f16x8 v[kCombineMaxPieces][2];
#pragma unroll
  for (int u = 0; u < kCombineMaxPieces; ++u) {
    if (u < n_pc) {   // uniform in the workgroup
      const f16x8* src = reinterpret_cast<const f16x8*>(part + piece_rec(u) * DL);
      v[u][0] = src[c0];
      v[u][1] = src[c0 + 32];
    }
  }
  float mx = ax.x;
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
  mx = __shfl(mx, 0, 32);
  // an empty piece (lse2 -inf) has weight 0 (its stored values are 0)
  const bool live = c0 < n_pc && mx != -INFINITY;
  const float wl = live ? exp2f(ax.x - mx) : 0.f;
  const float wk = live ? exp2f(ax.y - mx) : 0.f;
  float wsum = wl;
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off, 32);
  wsum = __shfl(wsum, 0, 32);
  float4 acc[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) acc[h][0] = acc[h][1] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kCombineMaxPieces; ++u) {
    if (u < n_pc) {
      const float w = __shfl(wk, u, 32);
      partial_chunk_fma(acc[0], w, v[u][0]);
      partial_chunk_fma(acc[1], w, v[u][1]);
    }
  }
  store_merged_row(a, (int64_t)b * n_rows + r, c0, acc, wsum, mx);
}

// Band schedule with small bands (R < 32): a cut band has few rows and may have
// hundreds of pieces (one request, one row block, 256 windows), so the four
// waves of a workgroup split the pieces of 2 rows, kCombinePiecesInFlight at a
// time, with weights against the max over all the pieces; the waves' sums are
// added through LDS.  Same (edge, slot) pairs as above, 64 groups of 2 rows per
// row block.
constexpr int kSplitRows = 2;
constexpr int kSplitGroups = ROWS / kSplitRows;

__global__ void __launch_bounds__(256) attn_band_combine_split_kernel(AttnArgs a) {
  __shared__ float4 s_acc[3][64][4];
  __shared__ float s_w[3][64];
  const int n_rows = a.N * a.H;
  const int rbb = band_row_blocks((n_rows + ROWS - 1) / ROWS);
  const int windows = reinterpret_cast<const int4*>(a.band_edges)[0].z;
  const int p = (int)blockIdx.x / kSplitGroups;
  const int grp = (int)blockIdx.x % kSplitGroups;
  if (p >= (windows - 1) * rbb) return;
  const int e = 1 + p / rbb;
  const int j = p % rbb;
  const int4 d = reinterpret_cast<const int4*>(a.band_edges)[e];
  if (!d.x) return;
  const int b = d.y, kb = d.z, n_pc = d.w - e + 2;   // pieces: window e - 1's tail, heads of e .. last
  const int wave = (int)threadIdx.x >> 6;
  const int lane = (int)threadIdx.x & 63;
  const int rl = grp * kSplitRows + (lane >> 5);
  const int r = (kb * rbb + j) * ROWS + rl;
  if ((kb * rbb + j) * ROWS + grp * kSplitRows >= n_rows) return;   // the whole group is past the end
  const bool row_ok = r < n_rows;
  const int c0 = lane & 31;
  const _Float16* part = static_cast<const _Float16*>(a.part_o);
  auto piece_rec = [&](int i) { return (int64_t)band_part_slot(e - 1 + i, j, rbb, i > 0) * ROWS + rl; };
  float mx = -INFINITY;
  for (int i = c0; i < n_pc; i += 32) mx = fmaxf(mx, a.part_aux[piece_rec(i)].x);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
  float wsum = 0.f;
  float4 acc[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) acc[h][0] = acc[h][1] = make_float4(0.f, 0.f, 0.f, 0.f);
  // wave w takes pieces P q .. P q + P - 1 for q = w, w + 4, ... (P pieces in flight); a piece
  // past the end re-reads piece P q with weight 0, an empty piece (lse2 -inf) has weight 0
  constexpr int P = kCombinePiecesInFlight;
  if (mx != -INFINITY) {
    for (int i0 = P * wave; i0 < n_pc; i0 += 4 * P) {
      float w[P];
      f16x8 v[P][2];
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const bool ok = i0 + u < n_pc;
        const int64_t rec = piece_rec(ok ? i0 + u : i0);
        const float2 ax = a.part_aux[rec];
        wsum += ok ? exp2f(ax.x - mx) : 0.f;
        w[u] = ok ? exp2f(ax.y - mx) : 0.f;
        const f16x8* src = reinterpret_cast<const f16x8*>(part + rec * DL);
        v[u][0] = src[c0];
        v[u][1] = src[c0 + 32];
      }
#pragma unroll
      for (int u = 0; u < P; ++u) {
        partial_chunk_fma(acc[0], w[u], v[u][0]);
        partial_chunk_fma(acc[1], w[u], v[u][1]);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q) s_acc[wave - 1][lane][2 * h + q] = acc[h][q];
    s_w[wave - 1][lane] = wsum;
  }
  __syncthreads();
  if (wave > 0 || !row_ok) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    wsum += s_w[w][lane];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float4 t = s_acc[w][lane][2 * h + q];
        acc[h][q].x += t.x;
        acc[h][q].y += t.y;
        acc[h][q].z += t.z;
        acc[h][q].w += t.w;
      }
  }
  store_merged_row(a, (int64_t)b * n_rows + r, c0, acc, wsum, mx);
}

}  // namespace

hipError_t launch_verify_attn_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int n_rb = (a.N * a.H + ROWS - 1) / ROWS;
  const int grid = a.balanced ? kBandWorkgroups : a.B * n_rb * a.splits;
  hipLaunchKernelGGL(verify_attn_bf16_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t stream) {
  const int64_t total_rows = (int64_t)a.B * a.N * a.H;
  const int64_t threads = total_rows * (DL / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const _Float16*>(a.part_o), a.part_aux, a.splits, total_rows, a.o, a.lse);
  return hipGetLastError();
}

hipError_t launch_attn_band_combine(const AttnArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int n_rb = (a.N * a.H + ROWS - 1) / ROWS;
  const int rbb = n_rb % kBandRowBlocks == 0 ? kBandRowBlocks : n_rb;
  const int pairs = (a.band_windows - 1) * rbb;   // (edge, slot) pairs of the most windows the kernel can use
  if (pairs <= 0) return hipSuccess;
  if (rbb == kBandRowBlocks)
    hipLaunchKernelGGL(attn_band_combine_kernel, dim3(pairs * kCombineGroups), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_band_combine_split_kernel, dim3(pairs * kSplitGroups), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ddtree
