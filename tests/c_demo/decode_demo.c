/* A plain C consumer of libkvdecode: it allocates device memory with the HIP
 * runtime, builds a pool, stores K/V and runs one decode step through the C
 * ABI alone (no Python, no PyTorch), then writes the output for the caller to
 * check.
 *
 * usage: decode_demo IN OUT
 * IN  (little-endian): int32 header {dtype (0 bf16, 1 FP8 E4M3), b, n_q, n_kv,
 *     head_dim, num_blocks, max_blocks_per_seq, n_tok, chunk_tokens}, then
 *     uint16 q[b][n_q][head_dim], uint16 k[n_tok][n_kv][head_dim], uint16 v[same],
 *     int32 slot_mapping[n_tok], int32 block_table[b][max_blocks_per_seq],
 *     int32 context_lens[b]  (bf16 values as raw bits)
 * OUT: uint16 out[b][n_q][head_dim], then float lse[b][n_q]
 * Exit status 0 on success; on any error a message on stderr and status 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvdecode.h"

#define FAIL(...)                     \
  do {                                \
    fprintf(stderr, __VA_ARGS__);     \
    fputc('\n', stderr);              \
    exit(1);                          \
  } while (0)

#define CHECK_HIP(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_));              \
  } while (0)

#define CHECK_KVD(call)                                                              \
  do {                                                                               \
    kvd_status s_ = (call);                                                          \
    if (s_ != KVD_OK) FAIL("%s: %s (%s)", #call, kvd_status_string(s_), kvd_last_hip_error()); \
  } while (0)

static void* read_exact(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p) FAIL("out of host memory");
  if (bytes && fread(p, 1, bytes, f) != bytes) FAIL("input file too short");
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) FAIL("usage: %s IN OUT", argv[0]);
  FILE* f = fopen(argv[1], "rb");
  if (!f) FAIL("cannot open %s", argv[1]);
  int32_t h[9];
  if (fread(h, sizeof h, 1, f) != 1) FAIL("input header too short");
  const int32_t dtype = h[0], b = h[1], n_q = h[2], n_kv = h[3], d = h[4], num_blocks = h[5],
                max_blocks = h[6], n_tok = h[7], chunk = h[8];
  if (b < 1 || n_q < 1 || n_kv < 1 || d < 1 || num_blocks < 1 || max_blocks < 1 || n_tok < 0)
    FAIL("bad header");
  const size_t nq = (size_t)b * n_q * d, nkv = (size_t)n_tok * n_kv * d;
  uint16_t* q = read_exact(f, nq * 2);
  uint16_t* k = read_exact(f, nkv * 2);
  uint16_t* v = read_exact(f, nkv * 2);
  int32_t* slots = read_exact(f, (size_t)n_tok * 4);
  int32_t* table = read_exact(f, (size_t)b * max_blocks * 4);
  int32_t* lens = read_exact(f, (size_t)b * 4);
  fclose(f);
  int32_t max_len = 0;
  for (int32_t i = 0; i < b; ++i) max_len = lens[i] > max_len ? lens[i] : max_len;

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  kvd_pool_desc desc = {1, num_blocks, 16, n_kv, d, dtype == 1 ? KVD_FP8_E4M3 : KVD_BF16};
  size_t kv_bytes = 0, scale_bytes = 0;
  CHECK_KVD(kvd_pool_bytes(&desc, &kv_bytes, &scale_bytes));
  void* kv = NULL;
  float* scales = NULL;
  CHECK_HIP(hipMalloc(&kv, kv_bytes));
  CHECK_HIP(hipMemset(kv, 0, kv_bytes));
  if (scale_bytes) {
    CHECK_HIP(hipMalloc((void**)&scales, scale_bytes));
    CHECK_HIP(hipMemset(scales, 0, scale_bytes));
  }
  kvd_pool* pool = NULL;
  CHECK_KVD(kvd_create_pool(&desc, kv, scales, &pool));

  void* dk = to_device(k, nkv * 2);
  void* dv = to_device(v, nkv * 2);
  int32_t* dslots = to_device(slots, (size_t)n_tok * 4);
  CHECK_KVD(kvd_write_kv(pool, 0, dk, dv, dslots, n_tok, stream));

  void* dq = to_device(q, nq * 2);
  int32_t* dtable = to_device(table, (size_t)b * max_blocks * 4);
  int32_t* dlens = to_device(lens, (size_t)b * 4);
  void* dout = NULL;
  float* dlse = NULL;
  CHECK_HIP(hipMalloc(&dout, nq * 2));
  CHECK_HIP(hipMalloc((void**)&dlse, (size_t)b * n_q * 4));

  kvd_decode_args args;
  memset(&args, 0, sizeof args);
  args.b = b;
  args.n_q = n_q;
  args.max_blocks_per_seq = max_blocks;
  args.max_context_len = max_len;
  args.q = dq;
  args.block_table = dtable;
  args.context_lens = dlens;
  args.out = dout;
  args.lse_out = dlse;
  args.chunk_tokens = chunk;
  size_t ws_bytes = 0;
  CHECK_KVD(kvd_decode_workspace_bytes(pool, &args, &ws_bytes));
  void* ws = NULL;
  if (ws_bytes) CHECK_HIP(hipMalloc(&ws, ws_bytes));   /* hipMalloc returns 256-byte aligned memory */
  args.workspace = ws;
  args.workspace_bytes = ws_bytes;
  int32_t chunk_used = 0, n_chunks = 0;
  CHECK_KVD(kvd_decode_plan(pool, &args, &chunk_used, &n_chunks));
  if (dtype == 1) CHECK_KVD(kvd_decode_attn_fp8(pool, 0, &args, stream));
  else CHECK_KVD(kvd_decode_attn(pool, 0, &args, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  uint16_t* out = malloc(nq * 2);
  float* lse = malloc((size_t)b * n_q * 4);
  if (!out || !lse) FAIL("out of host memory");
  CHECK_HIP(hipMemcpy(out, dout, nq * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse, dlse, (size_t)b * n_q * 4, hipMemcpyDeviceToHost));
  FILE* g = fopen(argv[2], "wb");
  if (!g) FAIL("cannot open %s", argv[2]);
  if (fwrite(out, 2, nq, g) != nq || fwrite(lse, 4, (size_t)b * n_q, g) != (size_t)b * n_q) FAIL("write failed");
  fclose(g);
  printf("decoded b=%d n_q=%d n_kv=%d d=%d dtype=%s chunk=%d n_chunks=%d workspace=%zu\n", b, n_q, n_kv, d,
         dtype == 1 ? "fp8" : "bf16", chunk_used, n_chunks, ws_bytes);

  CHECK_KVD(kvd_destroy_pool(pool));
  CHECK_HIP(hipFree(kv));
  if (scales) CHECK_HIP(hipFree(scales));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  CHECK_HIP(hipFree(dslots));
  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dtable));
  CHECK_HIP(hipFree(dlens));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dlse));
  if (ws) CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipStreamDestroy(stream));
  free(q); free(k); free(v); free(slots); free(table); free(lens); free(out); free(lse);
  return 0;
}
