/*
 * Host-side argument checks of every ddtree entry point, run against a build of
 * the library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
 * (the device code is built as usual).  No call here passes validation, so nothing
 * touches a GPU: the program exercises the size arithmetic, the overlap checks and
 * the status strings, including shapes at the limits of their integer types.
 *
 * Exit status: 0 when every call returns the expected status; 1 otherwise.  A
 * sanitizer report aborts the program with its own message and a nonzero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ddtree.h"

#define A ((uintptr_t)0x10000) /* fake, 16-byte aligned device addresses: never dereferenced */
#define P(x) ((void*)(uintptr_t)(x))

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d (%s), expected %d (%s)\n", line, what, got, ddtree_status_string(got),
            want, ddtree_status_string(want));
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

/* ---- ddtree_verify_attn with defaults that pass the shape checks ---- */
typedef struct {
  int32_t dtype, B, N, H, Dl, Dr;
  uintptr_t q, qr, ckv;
  int64_t ld_ckv;
  uintptr_t krope;
  int64_t ld_krope;
  uintptr_t offs;
  int64_t max_len;
  uintptr_t ckv_t;
  int64_t ld_ckv_t;
  uintptr_t krope_t;
  int64_t ld_krope_t;
  uintptr_t mask;
  float scale;
  int32_t splits;
  uintptr_t o, lse, ws;
  size_t ws_bytes;
} AttnCall;

static AttnCall attn_defaults(void) {
  AttnCall c;
  memset(&c, 0, sizeof c);
  c.dtype = DDTREE_BF16; c.B = 1; c.N = 8; c.H = 64; c.Dl = 512; c.Dr = 64;
  c.q = A; c.qr = A + (1u << 24); c.ckv = A + (2u << 24); c.ld_ckv = 576; c.krope = A + (2u << 24) + 1024;
  c.ld_krope = 576; c.offs = A + (3u << 24); c.max_len = 64; c.ckv_t = A + (4u << 24); c.ld_ckv_t = 576;
  c.krope_t = A + (4u << 24) + 1024; c.ld_krope_t = 576; c.mask = A + (5u << 24); c.scale = 0.07f; c.splits = 1;
  c.o = A + (6u << 24); c.lse = A + (7u << 24); c.ws = 0; c.ws_bytes = 0;
  return c;
}

static int attn(AttnCall c) {
  return ddtree_verify_attn(c.dtype, c.B, c.N, c.H, c.Dl, c.Dr, P(c.q), P(c.qr), P(c.ckv), c.ld_ckv, P(c.krope),
                            c.ld_krope, (const int64_t*)P(c.offs), c.max_len, P(c.ckv_t), c.ld_ckv_t, P(c.krope_t),
                            c.ld_krope_t, (const uint32_t*)P(c.mask), c.scale, c.splits, (float*)P(c.o),
                            (float*)P(c.lse), P(c.ws), c.ws_bytes, NULL);
}

static int attn_noalloc(AttnCall c) {
  return ddtree_verify_attn_noalloc(c.dtype, c.B, c.N, c.H, c.Dl, c.Dr, P(c.q), P(c.qr), P(c.ckv), c.ld_ckv,
                                    P(c.krope), c.ld_krope, (const int64_t*)P(c.offs), c.max_len, P(c.ckv_t),
                                    c.ld_ckv_t, P(c.krope_t), c.ld_krope_t, (const uint32_t*)P(c.mask), c.scale,
                                    c.splits, (float*)P(c.o), (float*)P(c.lse), NULL);
}

static void check_verify_attn(void) {
  AttnCall c;
  const int32_t dtypes[] = {DDTREE_F32, DDTREE_BF16, 7};
  const int32_t sizes[] = {INT32_MIN, -1, 0, 1, 63, 64, 256, 257, 1 << 20, INT32_MAX};
  const int64_t lens[] = {INT64_MIN, -1, 0, 1, 4096, (int64_t)1 << 40, ((int64_t)1 << 40) + 1, INT64_MAX - 31,
                          INT64_MAX};
  const int32_t splits[] = {INT32_MIN, -1, 0, 1, 8, 1024, 1025, INT32_MAX};
  size_t i, j, k, s;

  /* the sizing queries take any arguments */
  for (i = 0; i < 3; ++i)
    for (j = 0; j < sizeof sizes / sizeof *sizes; ++j)
      for (k = 0; k < sizeof lens / sizeof *lens; ++k)
        for (s = 0; s < sizeof splits / sizeof *splits; ++s) {
          (void)ddtree_verify_attn_workspace_size(dtypes[i], sizes[j], 64, sizes[j], 512, 64, lens[k], splits[s]);
          (void)ddtree_verify_attn_workspace_size(dtypes[i], 16, sizes[j], 64, sizes[j], 64, lens[k], splits[s]);
          (void)ddtree_verify_attn_auto_splits(dtypes[i], sizes[j], sizes[j], 64, 512, 64, lens[k]);
          (void)ddtree_verify_attn_auto_splits(dtypes[i], 1, 64, sizes[j], 512, sizes[j], lens[k]);
        }

  /* shapes */
  c = attn_defaults(); c.dtype = 7; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.N = 0; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.N = 257; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.H = 0; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.B = -2; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.B = 0; EXPECT(attn(c), DDTREE_OK);
  c = attn_defaults(); c.B = INT32_MAX; c.H = INT32_MAX; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.Dl = 1024; c.ld_ckv = c.ld_ckv_t = 1088; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.Dl = INT32_MAX; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.Dr = -1; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.max_len = -1; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.max_len = INT64_MAX; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.max_len = INT64_MAX; c.splits = 0; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.max_len = ((int64_t)1 << 40) + 1; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.splits = INT32_MAX; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.splits = -1; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.scale = NAN; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.scale = INFINITY; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  /* pointers and strides */
  c = attn_defaults(); c.q = 0; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.mask = 0; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.ckv = 0; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.ld_ckv = 500; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.ld_ckv = INT64_MAX; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.ld_ckv = INT64_MAX - 7; EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.ld_krope_t = INT64_MIN; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.ckv = A + (2u << 24) + 2; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.dtype = DDTREE_F32; c.Dl = 64; c.Dr = 32; c.ld_ckv = INT64_MAX; c.ld_ckv_t = INT64_MAX;
  EXPECT(attn(c), DDTREE_ERR_UNSUPPORTED);
  /* aliasing, including pointers at the top of the address space */
  c = attn_defaults(); c.o = A + 64; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.lse = c.o + 4096; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.o = A + (2u << 24) + 4096; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.o = UINTPTR_MAX - 4095; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.q = UINTPTR_MAX - 15; EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  /* workspace */
  c = attn_defaults(); c.splits = 4; EXPECT(attn(c), DDTREE_ERR_WORKSPACE);
  c = attn_defaults(); c.N = 64; c.splits = 0; EXPECT(attn(c), DDTREE_ERR_WORKSPACE);
  c = attn_defaults(); c.splits = 4; c.ws = A + (8u << 24); c.ws_bytes = (size_t)4 * 8 * 64 * 1032 - 4;
  EXPECT(attn(c), DDTREE_ERR_WORKSPACE);
  c = attn_defaults(); c.splits = 4; c.ws = A + (8u << 24) + 8; c.ws_bytes = (size_t)4 * 8 * 64 * 1032;
  EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.splits = 4; c.ws = A + (2u << 24) + 32; c.ws_bytes = (size_t)4 * 8 * 64 * 1032;
  EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.splits = 4; c.ws = UINTPTR_MAX - 4095; c.ws_bytes = SIZE_MAX;
  EXPECT(attn(c), DDTREE_ERR_INVALID_ARG);

  /* the no-allocation variant refuses what its scratch cannot hold, before any HIP call */
  c = attn_defaults(); c.N = 64; c.splits = 18; c.max_len = 4096; EXPECT(attn_noalloc(c), DDTREE_ERR_WORKSPACE);
  c = attn_defaults(); c.N = 64; c.splits = 1024; c.max_len = 4096; EXPECT(attn_noalloc(c), DDTREE_ERR_WORKSPACE);
  c = attn_defaults(); c.B = 0; EXPECT(attn_noalloc(c), DDTREE_OK);
  c = attn_defaults(); c.q = 0; EXPECT(attn_noalloc(c), DDTREE_ERR_INVALID_ARG);
  c = attn_defaults(); c.max_len = INT64_MAX; EXPECT(attn_noalloc(c), DDTREE_ERR_UNSUPPORTED);
  c = attn_defaults(); c.splits = INT32_MAX; EXPECT(attn_noalloc(c), DDTREE_ERR_UNSUPPORTED);
}

static void check_build_mask(void) {
  uint32_t* mask = (uint32_t*)P(A + 8192);
  int32_t* depth = (int32_t*)P(A + 12288);
  int64_t* pos = (int64_t*)P(A + 16384);
  int32_t* ok = (int32_t*)P(A + 20480);
  const int32_t* parents = (const int32_t*)P(A);
  const int64_t* offs = (const int64_t*)P(A + 4096);
  EXPECT(ddtree_build_mask(parents, 2, 0, offs, mask, depth, pos, ok, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_mask(parents, INT32_MIN, 8, offs, mask, depth, pos, ok, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_mask(parents, 2, INT32_MAX, offs, mask, depth, pos, ok, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_build_mask(parents, 0, 8, offs, mask, depth, pos, ok, NULL), DDTREE_OK);
  EXPECT(ddtree_build_mask(NULL, 2, 8, offs, mask, depth, pos, ok, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_mask(parents, 2, 8, offs, (uint32_t*)P(A + 16), depth, pos, ok, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_mask(parents, INT32_MAX, 256, offs, mask, depth, pos, ok, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_mask(parents, 2, 8, offs, mask, depth, (int64_t*)P(A + 4096), ok, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_mask((const int32_t*)P(UINTPTR_MAX - 15), 2, 8, offs, mask, depth, pos, ok, NULL),
         DDTREE_ERR_INVALID_ARG);
}

static void check_greedy_accept(void) {
  const float* logits = (const float*)P(A);
  const int32_t* tokens = (const int32_t*)P(A + (1u << 24));
  const int32_t* parents = (const int32_t*)P(A + (1u << 24) + 4096);
  int32_t* tstar = (int32_t*)P(A + (2u << 24));
  int32_t* alen = (int32_t*)P(A + (2u << 24) + 4096);
  int32_t* nodes = (int32_t*)P(A + (2u << 24) + 8192);
  int32_t* commit = (int32_t*)P(A + (2u << 24) + 12288);
  EXPECT(ddtree_greedy_accept(logits, 512, tokens, parents, 1, 8, 0, tstar, alen, nodes, commit, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_greedy_accept(logits, 100, tokens, parents, 1, 8, 512, tstar, alen, nodes, commit, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_greedy_accept(logits, 512, tokens, parents, 1, 300, 512, tstar, alen, nodes, commit, NULL),
         DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_greedy_accept(logits, 512, tokens, parents, 0, 8, 512, tstar, alen, nodes, commit, NULL), DDTREE_OK);
  EXPECT(ddtree_greedy_accept(NULL, 512, tokens, parents, 1, 8, 512, tstar, alen, nodes, commit, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_greedy_accept(logits, 512, tokens, parents, 1, 8, 512, (int32_t*)P(A + 100), alen, nodes, commit,
                              NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_greedy_accept(logits, INT64_MAX, tokens, parents, INT32_MAX, 256, INT32_MAX, tstar, alen, nodes,
                              commit, NULL),
         DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_greedy_accept(logits, INT64_MAX, tokens, parents, 1, 8, 512, tstar, alen, nodes, commit, NULL),
         DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_greedy_accept(logits, (int64_t)1 << 40, tokens, parents, 1 << 20, 256, 512, tstar, alen, nodes,
                              commit, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_greedy_accept((const float*)P(UINTPTR_MAX - 4095), 512, tokens, parents, 1, 8, 512, tstar, alen,
                              nodes, commit, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_greedy_accept(logits, INT64_MIN, tokens, parents, 1, 8, 512, tstar, alen, nodes, commit, NULL),
         DDTREE_ERR_INVALID_ARG);
}

static void check_compact_kv(void) {
  const void* ct = P(A + (1u << 24));
  const void* rt = P(A + (1u << 24) + 1024);
  const int32_t* alen = (const int32_t*)P(A);
  const int32_t* nodes = (const int32_t*)P(A + 4096);
  const int64_t* dest = (const int64_t*)P(A + 8192);
  void* c = P(A + (2u << 24));
  void* r = P(A + (2u << 24) + 1024);
  EXPECT(ddtree_compact_kv(5, 2, 16, 512, 64, ct, 576, rt, 576, alen, nodes, dest, c, 576, r, 576, NULL),
         DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, 2, 0, 512, 64, ct, 576, rt, 576, alen, nodes, dest, c, 576, r, 576, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, 0, 16, 512, 64, ct, 576, rt, 576, alen, nodes, dest, c, 576, r, 576, NULL),
         DDTREE_OK);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, 2, 16, 512, 64, ct, 500, rt, 576, alen, nodes, dest, c, 576, r, 576, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, 2, 16, 512, 64, ct, 576, rt, 576, alen, (const int32_t*)P(A + (1u << 24) + 64),
                           dest, c, 576, r, 576, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, INT32_MAX, 256, INT32_MAX, INT32_MAX, ct, INT64_MAX, rt, INT64_MAX, alen,
                           nodes, dest, c, INT64_MAX, r, INT64_MAX, NULL),
         DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, INT32_MAX, 256, 512, 64, ct, (int64_t)1 << 40, rt, (int64_t)1 << 40, alen,
                           nodes, dest, c, 576, r, 576, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_compact_kv(DDTREE_BF16, 2, 16, 512, 64, ct, 576, rt, 576, (const int32_t*)P(UINTPTR_MAX - 7), nodes,
                           dest, c, 576, r, 576, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_compact_kv(DDTREE_F32, 2, 16, 512, 64, ct, INT64_MIN, rt, 576, alen, nodes, dest, c, 576, r, 576,
                           NULL),
         DDTREE_ERR_INVALID_ARG);
}

static void check_build_tree(void) {
  const int32_t* root = (const int32_t*)P(A);
  const int32_t* ct = (const int32_t*)P(A + 4096);
  const float* cl = (const float*)P(A + 8192);
  int32_t* par = (int32_t*)P(A + 16384);
  int32_t* tok = (int32_t*)P(A + 20480);
  int32_t* dep = (int32_t*)P(A + 24576);
  float* sc = (float*)P(A + 28672);
  EXPECT(ddtree_build_tree(2, 0, 8, 4, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_tree(2, 257, 8, 4, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_build_tree(2, 64, INT32_MAX, 4, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_build_tree(2, 64, 8, INT32_MAX, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_build_tree(0, 7, 2, 2, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_OK);
  EXPECT(ddtree_build_tree(0, 8, 2, 2, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_build_tree(0, 256, 64, 64, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_OK);
  EXPECT(ddtree_build_tree(2, 64, 8, 4, NULL, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_tree(2, 64, 8, 4, root, ct, cl, (int32_t*)P(A + 8192 + 64), tok, dep, sc, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_build_tree(INT32_MAX, 256, 64, 64, root, ct, cl, par, tok, dep, sc, NULL), DDTREE_ERR_INVALID_ARG);
}

static void check_rope_tree(void) {
  void* q = P(A);
  void* k = P(A + (1u << 24));
  const int64_t* pos = (const int64_t*)P(A + (2u << 24));
  const double* inv = (const double*)P(A + (3u << 24));
  EXPECT(ddtree_rope_tree(9, 2, 16, 64, 64, q, k, 576, pos, inv, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_rope_tree(DDTREE_BF16, 2, 16, 64, 63, q, k, 576, pos, inv, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_rope_tree(DDTREE_BF16, 2, 16, 64, INT32_MAX - 1, q, k, 576, pos, inv, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_rope_tree(DDTREE_BF16, 0, 16, 64, 64, q, k, 576, pos, inv, NULL), DDTREE_OK);
  EXPECT(ddtree_rope_tree(DDTREE_BF16, 2, 16, 64, 64, NULL, NULL, 576, pos, inv, NULL), DDTREE_OK);
  EXPECT(ddtree_rope_tree(DDTREE_BF16, 2, 16, 64, 64, q, k, 32, pos, inv, NULL), DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_rope_tree(DDTREE_BF16, 2, 16, 64, 64, q, k, 576, (const int64_t*)P(A + 64), inv, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_rope_tree(DDTREE_F32, INT32_MAX, 256, INT32_MAX, 64, q, k, INT64_MAX, pos, inv, NULL),
         DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_rope_tree(DDTREE_F32, 2, 16, INT32_MAX, 64, q, k, 576, pos, inv, NULL), DDTREE_ERR_UNSUPPORTED);
  EXPECT(ddtree_rope_tree(DDTREE_F32, 2, 16, 64, 64, q, k, INT64_MAX, pos, inv, NULL), DDTREE_ERR_UNSUPPORTED);
  /* no key rows: their stride is not looked at (the call fails on the overlap instead) */
  EXPECT(ddtree_rope_tree(DDTREE_F32, 2, 16, 64, 64, q, NULL, INT64_MAX, (const int64_t*)P(A + 64), inv, NULL),
         DDTREE_ERR_INVALID_ARG);
  EXPECT(ddtree_rope_tree(DDTREE_F32, 1 << 20, 256, 1 << 16, 64, q, k, (int64_t)1 << 40, pos, inv, NULL),
         DDTREE_ERR_INVALID_ARG);
}

int main(void) {
  int s;
  for (s = -8; s <= 4; ++s) (void)strlen(ddtree_status_string(s));
  (void)strlen(ddtree_status_string(INT32_MIN));
  (void)strlen(ddtree_status_string(INT32_MAX));
  if (strlen(ddtree_build_digest()) == 0) {
    fprintf(stderr, "empty build digest\n");
    ++failures;
  }
  check_verify_attn();
  check_build_mask();
  check_greedy_accept();
  check_compact_kv();
  check_build_tree();
  check_rope_tree();
  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("host ABI checks: all statuses as expected\n");
  return 0;
}
