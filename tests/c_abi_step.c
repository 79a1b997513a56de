/*
 * c_abi_step.c -- one DDTree verify step driven through libddtree.so from
 * plain C: no Python, no torch.  The caller owns every buffer (hipMalloc),
 * passes a hipStream_t as void*, and reads the ddtree_status of each call.
 *
 * Usage: c_abi_step DIR
 *   DIR/meta.txt   "B N H Dl Dr V max_prefix_len cache_rows scale"
 *   DIR/*.bin      raw little-endian inputs (names below; bf16 as 16-bit words)
 * Writes the outputs as raw files into DIR and prints the library's build
 * digest and the hash of the source it was built from.  Exit status 0 on
 * success; any failed call prints its status string and exits non-zero.
 *
 * Steps: ddtree_build_mask -> ddtree_verify_attn (automatic schedule, caller
 * workspace) -> ddtree_verify_attn_noalloc (same inputs, for comparison) ->
 * ddtree_greedy_accept -> ddtree_compact_kv (the accepted rows appended to the
 * cache at dest_rows).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ddtree.h"

#ifndef C_ABI_STEP_SOURCE_HASH
#define C_ABI_STEP_SOURCE_HASH "unknown"
#endif

static const char* g_dir;

static void die(const char* what, const char* why) {
  fprintf(stderr, "c_abi_step: %s: %s\n", what, why);
  exit(1);
}

static void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

static void dd_check(int st, const char* what) {
  if (st != DDTREE_OK) die(what, ddtree_status_string(st));
}

static void* read_file(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) die(path, "cannot open");
  void* buf = malloc(bytes ? bytes : 1);
  if (!buf) die(path, "out of host memory");
  if (fread(buf, 1, bytes, f) != bytes) die(path, "short read");
  fclose(f);
  return buf;
}

static void write_file(const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) die(path, "cannot create");
  if (fwrite(data, 1, bytes, f) != bytes) die(path, "short write");
  fclose(f);
}

/* Host file -> new device buffer. */
static void* upload(const char* name, size_t bytes) {
  void* h = read_file(name, bytes);
  void* d = NULL;
  hip_check(hipMalloc(&d, bytes ? bytes : 1), "hipMalloc");
  hip_check(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
  free(h);
  return d;
}

static void* device_buffer(size_t bytes) {
  void* d = NULL;
  hip_check(hipMalloc(&d, bytes ? bytes : 1), "hipMalloc");
  return d;
}

/* Device buffer -> host file. */
static void download(const char* name, const void* d, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (!h) die(name, "out of host memory");
  hip_check(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
  write_file(name, h, bytes);
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  g_dir = argv[1];
  char meta_path[4096];
  snprintf(meta_path, sizeof meta_path, "%s/meta.txt", g_dir);
  FILE* mf = fopen(meta_path, "r");
  if (!mf) die(meta_path, "cannot open");
  int B, N, H, Dl, Dr, V;
  long long max_len, cache_rows;
  float scale;
  if (fscanf(mf, "%d %d %d %d %d %d %lld %lld %f", &B, &N, &H, &Dl, &Dr, &V, &max_len, &cache_rows, &scale) != 9)
    die(meta_path, "expected B N H Dl Dr V max_prefix_len cache_rows scale");
  fclose(mf);
  printf("source %s\n", C_ABI_STEP_SOURCE_HASH);
  printf("digest %s\n", ddtree_build_digest());
  printf("case B=%d N=%d H=%d Dl=%d Dr=%d V=%d max_prefix_len=%lld cache_rows=%lld\n", B, N, H, Dl, Dr, V, max_len,
         cache_rows);
  fflush(stdout);

  const size_t nodes = (size_t)B * N, rows = nodes * H, W = (size_t)(N + 31) / 32, bf = 2;
  void* q_lat = upload("q_lat.bin", rows * Dl * bf);
  void* q_rope = upload("q_rope.bin", rows * Dr * bf);
  void* ckv = upload("ckv.bin", (size_t)cache_rows * Dl * bf);
  void* krope = upload("krope.bin", (size_t)cache_rows * Dr * bf);
  int64_t* offsets = (int64_t*)upload("offsets.bin", (size_t)(B + 1) * 8);
  void* ckv_tree = upload("ckv_tree.bin", nodes * Dl * bf);
  void* krope_tree = upload("krope_tree.bin", nodes * Dr * bf);
  int32_t* parents = (int32_t*)upload("parents.bin", nodes * 4);
  float* logits = (float*)upload("logits.bin", nodes * V * 4);
  int32_t* tokens = (int32_t*)upload("tokens.bin", nodes * 4);
  int64_t* dest_rows = (int64_t*)upload("dest_rows.bin", (size_t)B * 8);

  uint32_t* mask = (uint32_t*)device_buffer(nodes * W * 4);
  int32_t* depth = (int32_t*)device_buffer(nodes * 4);
  int64_t* pos = (int64_t*)device_buffer(nodes * 8);
  int32_t* ok = (int32_t*)device_buffer((size_t)B * 4);
  float* o = (float*)device_buffer(rows * Dl * 4);
  float* lse = (float*)device_buffer(rows * 4);
  float* o_na = (float*)device_buffer(rows * Dl * 4);
  float* lse_na = (float*)device_buffer(rows * 4);
  int32_t* targ = (int32_t*)device_buffer(nodes * 4);
  int32_t* alen = (int32_t*)device_buffer((size_t)B * 4);
  int32_t* acc_nodes = (int32_t*)device_buffer(nodes * 4);
  int32_t* commit = (int32_t*)device_buffer(nodes * 4);

  const size_t ws_bytes =
      ddtree_verify_attn_workspace_size(DDTREE_BF16, B, N, H, Dl, Dr, (int64_t)max_len, 0);
  void* ws = device_buffer(ws_bytes);
  printf("workspace %zu bytes, auto splits %d\n", ws_bytes,
         (int)ddtree_verify_attn_auto_splits(DDTREE_BF16, B, N, H, Dl, Dr, (int64_t)max_len));
  fflush(stdout);

  hipStream_t s;
  hip_check(hipStreamCreate(&s), "hipStreamCreate");
  dd_check(ddtree_build_mask(parents, B, N, offsets, mask, depth, pos, ok, s), "ddtree_build_mask");
  dd_check(ddtree_verify_attn(DDTREE_BF16, B, N, H, Dl, Dr, q_lat, q_rope, ckv, Dl, krope, Dr, offsets,
                              (int64_t)max_len, ckv_tree, Dl, krope_tree, Dr, mask, scale, 0, o, lse, ws, ws_bytes,
                              s),
           "ddtree_verify_attn");
  dd_check(ddtree_verify_attn_noalloc(DDTREE_BF16, B, N, H, Dl, Dr, q_lat, q_rope, ckv, Dl, krope, Dr, offsets,
                                      (int64_t)max_len, ckv_tree, Dl, krope_tree, Dr, mask, scale, 0, o_na, lse_na,
                                      s),
           "ddtree_verify_attn_noalloc");
  dd_check(ddtree_greedy_accept(logits, V, tokens, parents, B, N, V, targ, alen, acc_nodes, commit, s),
           "ddtree_greedy_accept");
  dd_check(ddtree_compact_kv(DDTREE_BF16, B, N, Dl, Dr, ckv_tree, Dl, krope_tree, Dr, alen, acc_nodes, dest_rows,
                             ckv, Dl, krope, Dr, s),
           "ddtree_compact_kv");
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");

  /* a refused call enqueues nothing and says why */
  if (ddtree_verify_attn(DDTREE_BF16, B, N, H, Dl, Dr, q_lat, q_rope, ckv, Dl, krope, Dr, offsets, (int64_t)max_len,
                         ckv_tree, Dl, krope_tree, Dr, mask, scale, 0, o, lse, ws, ws_bytes ? ws_bytes - 1 : 0,
                         s) == DDTREE_OK &&
      ws_bytes > 0)
    die("ddtree_verify_attn", "accepted a workspace one byte short");

  download("out_mask.bin", mask, nodes * W * 4);
  download("out_depth.bin", depth, nodes * 4);
  download("out_pos.bin", pos, nodes * 8);
  download("out_ok.bin", ok, (size_t)B * 4);
  download("out_o.bin", o, rows * Dl * 4);
  download("out_lse.bin", lse, rows * 4);
  download("out_o_noalloc.bin", o_na, rows * Dl * 4);
  download("out_lse_noalloc.bin", lse_na, rows * 4);
  download("out_target_argmax.bin", targ, nodes * 4);
  download("out_accept_len.bin", alen, (size_t)B * 4);
  download("out_accept_nodes.bin", acc_nodes, nodes * 4);
  download("out_commit_tokens.bin", commit, nodes * 4);
  download("out_ckv.bin", ckv, (size_t)cache_rows * Dl * bf);
  download("out_krope.bin", krope, (size_t)cache_rows * Dr * bf);

  hip_check(hipStreamDestroy(s), "hipStreamDestroy");
  void* bufs[] = {q_lat, q_rope,  ckv, krope, offsets, ckv_tree,  krope_tree, parents, logits, tokens, dest_rows,
                  mask,  depth,   pos, ok,    o,       lse,       o_na,       lse_na,  targ,   alen,   acc_nodes,
                  commit, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) hip_check(hipFree(bufs[i]), "hipFree");
  printf("done\n");
  return 0;
}
