/*
 * A plain C11 caller of the library's C ABI (include/mla.h), with no C++ and
 * no PyTorch: device buffers come from hipMalloc, the inputs from integer
 * hashes, and every input and output goes to a file in the directory named on
 * the command line, so that a test can hold the results to the float64
 * oracle.  It runs
 *   1. mla_decode on a small fp8 call (four requests of 0, 5, 300 and 1,500
 *      cached entries, one query token each, 16 heads, 2,048-entry pool, q and
 *      kv scales 0.75 and 1.25, lse returned), with the workspace sized by
 *      mla_decode_workspace_bytes;
 *   2. mla_merge_partials over three fp32 shards of (4 tokens, 16 heads),
 *      one shard empty (lse = -inf) on a few rows.
 * Files (little-endian, row-major): q.u8 (4, 16, 576) e4m3 codes,
 * kv.u8 (2048, 576), kv_indptr.i32 (5), kv_indices.i32, o.u16 (4, 16, 512)
 * bf16 bits, lse.f32 (4, 16), parts.f32 (3, 4, 16, 512), lse_parts.f32
 * (3, 4, 16), merged_o.u16 (4, 16, 512), merged_lse.f32 (4, 16).
 * Exit status 0 on success; otherwise the failing call is named on stderr.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mla.h"

#define BATCH 4
#define TOKENS 4
#define HEADS 16
#define POOL 2048
#define ROW 576
#define LATENT 512
#define PARTS 3

static const int kLengths[BATCH] = {0, 5, 300, 1500};

/* xorshift32 */
static uint32_t next_u32(uint32_t* s) {
  uint32_t x = *s;
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  *s = x;
  return x;
}

/* A finite e4m3fn code with |value| < 2: exponent field 0..7, any mantissa,
 * either sign. */
static uint8_t code_of(uint32_t h) { return (uint8_t)((h & 0x3Fu) | ((h >> 6 & 1u) << 7)); }

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int mla_ok(mla_status s, const char* what) {
  if (s != MLA_OK) {
    fprintf(stderr, "%s: %s\n", what, mla_status_string((int)s));
    return 0;
  }
  return 1;
}

static int write_file(const char* dir, const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (f == NULL) {
    fprintf(stderr, "cannot write %s\n", path);
    return 0;
  }
  size_t n = fwrite(data, 1, bytes, f);
  fclose(f);
  if (n != bytes) {
    fprintf(stderr, "short write to %s\n", path);
    return 0;
  }
  return 1;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s <output directory>\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  uint32_t seed = 0x2545F491u;

  /* ---- host inputs */
  int32_t kv_indptr[BATCH + 1], qo_indptr[BATCH + 1];
  kv_indptr[0] = 0;
  qo_indptr[0] = 0;
  for (int b = 0; b < BATCH; ++b) {
    kv_indptr[b + 1] = kv_indptr[b] + kLengths[b];
    qo_indptr[b + 1] = b + 1;
  }
  const int n_idx = kv_indptr[BATCH];
  int32_t* kv_indices = malloc(sizeof(int32_t) * (size_t)n_idx);
  uint8_t* q = malloc((size_t)TOKENS * HEADS * ROW);
  uint8_t* kv = malloc((size_t)POOL * ROW);
  float* parts = malloc(sizeof(float) * (size_t)PARTS * TOKENS * HEADS * LATENT);
  float* lse_parts = malloc(sizeof(float) * (size_t)PARTS * TOKENS * HEADS);
  uint16_t* o = malloc(sizeof(uint16_t) * (size_t)TOKENS * HEADS * LATENT);
  uint16_t* merged_o = malloc(sizeof(uint16_t) * (size_t)TOKENS * HEADS * LATENT);
  float* lse = malloc(sizeof(float) * (size_t)TOKENS * HEADS);
  float* merged_lse = malloc(sizeof(float) * (size_t)TOKENS * HEADS);
  if (!kv_indices || !q || !kv || !parts || !lse_parts || !o || !merged_o || !lse || !merged_lse) {
    fprintf(stderr, "host allocation failed\n");
    return 1;
  }
  /* Distinct pool entries: 7919 is odd, so i -> (7919 i + 13) mod 2048 is a
   * bijection on the pool. */
  for (int i = 0; i < n_idx; ++i) kv_indices[i] = (int32_t)((7919L * i + 13) % POOL);
  for (size_t i = 0; i < (size_t)TOKENS * HEADS * ROW; ++i) q[i] = code_of(next_u32(&seed));
  for (size_t i = 0; i < (size_t)POOL * ROW; ++i) kv[i] = code_of(next_u32(&seed));
  for (size_t i = 0; i < (size_t)PARTS * TOKENS * HEADS * LATENT; ++i)
    parts[i] = ((float)(next_u32(&seed) % 2001u) - 1000.0f) / 500.0f; /* [-2, 2] */
  for (int i = 0; i < PARTS * TOKENS * HEADS; ++i) {
    const uint32_t h = next_u32(&seed);
    lse_parts[i] = (h % 7u == 0u) ? -INFINITY : ((float)(h % 1001u) - 500.0f) / 100.0f;
  }
  /* One row empty in every shard: o = 0, lse = -inf. */
  for (int s = 0; s < PARTS; ++s) lse_parts[(s * TOKENS + 1) * HEADS + 3] = -INFINITY;
  const float scales[2] = {0.75f, 1.25f}; /* q_scale, kv_scale */
  const float sm_scale = 1.0f / sqrtf(192.0f);

  /* ---- device buffers */
  void *d_q = NULL, *d_kv = NULL, *d_o = NULL, *d_lse = NULL, *d_qo = NULL, *d_kvp = NULL;
  void *d_idx = NULL, *d_scales = NULL, *d_ws = NULL, *d_parts = NULL, *d_lse_parts = NULL;
  void *d_mo = NULL, *d_mlse = NULL;
  const size_t ws_bytes = mla_decode_workspace_bytes(BATCH, TOKENS, HEADS, 1);
  if (ws_bytes == 0) {
    fprintf(stderr, "mla_decode_workspace_bytes: 0 for a valid shape\n");
    return 1;
  }
  if (!hip_ok(hipMalloc(&d_q, (size_t)TOKENS * HEADS * ROW), "hipMalloc q") ||
      !hip_ok(hipMalloc(&d_kv, (size_t)POOL * ROW), "hipMalloc kv") ||
      !hip_ok(hipMalloc(&d_o, sizeof(uint16_t) * TOKENS * HEADS * LATENT), "hipMalloc o") ||
      !hip_ok(hipMalloc(&d_lse, sizeof(float) * TOKENS * HEADS), "hipMalloc lse") ||
      !hip_ok(hipMalloc(&d_qo, sizeof qo_indptr), "hipMalloc qo_indptr") ||
      !hip_ok(hipMalloc(&d_kvp, sizeof kv_indptr), "hipMalloc kv_indptr") ||
      !hip_ok(hipMalloc(&d_idx, sizeof(int32_t) * (size_t)n_idx), "hipMalloc kv_indices") ||
      !hip_ok(hipMalloc(&d_scales, sizeof scales), "hipMalloc scales") ||
      !hip_ok(hipMalloc(&d_ws, ws_bytes), "hipMalloc workspace") ||
      !hip_ok(hipMalloc(&d_parts, sizeof(float) * PARTS * TOKENS * HEADS * LATENT),
              "hipMalloc parts") ||
      !hip_ok(hipMalloc(&d_lse_parts, sizeof(float) * PARTS * TOKENS * HEADS),
              "hipMalloc lse_parts") ||
      !hip_ok(hipMalloc(&d_mo, sizeof(uint16_t) * TOKENS * HEADS * LATENT), "hipMalloc merged o") ||
      !hip_ok(hipMalloc(&d_mlse, sizeof(float) * TOKENS * HEADS), "hipMalloc merged lse"))
    return 1;
  if (!hip_ok(hipMemcpy(d_q, q, (size_t)TOKENS * HEADS * ROW, hipMemcpyHostToDevice), "copy q") ||
      !hip_ok(hipMemcpy(d_kv, kv, (size_t)POOL * ROW, hipMemcpyHostToDevice), "copy kv") ||
      !hip_ok(hipMemcpy(d_qo, qo_indptr, sizeof qo_indptr, hipMemcpyHostToDevice), "copy qo") ||
      !hip_ok(hipMemcpy(d_kvp, kv_indptr, sizeof kv_indptr, hipMemcpyHostToDevice), "copy kvp") ||
      !hip_ok(hipMemcpy(d_idx, kv_indices, sizeof(int32_t) * (size_t)n_idx,
                        hipMemcpyHostToDevice), "copy kv_indices") ||
      !hip_ok(hipMemcpy(d_scales, scales, sizeof scales, hipMemcpyHostToDevice), "copy scales") ||
      !hip_ok(hipMemcpy(d_parts, parts, sizeof(float) * PARTS * TOKENS * HEADS * LATENT,
                        hipMemcpyHostToDevice), "copy parts") ||
      !hip_ok(hipMemcpy(d_lse_parts, lse_parts, sizeof(float) * PARTS * TOKENS * HEADS,
                        hipMemcpyHostToDevice), "copy lse_parts"))
    return 1;

  /* ---- the calls, on the null stream */
  const float* d_qs = (const float*)d_scales;
  const float* d_ks = (const float*)d_scales + 1;
  if (!mla_ok(mla_decode(d_q, MLA_DTYPE_FP8_E4M3FN, d_kv, MLA_DTYPE_FP8_E4M3FN, POOL, d_o,
                         (const int32_t*)d_qo, (const int32_t*)d_kvp, (const int32_t*)d_idx,
                         n_idx, NULL, BATCH, TOKENS, HEADS, 1, sm_scale, d_qs, d_ks, 1,
                         (float*)d_lse, d_ws, ws_bytes, NULL),
              "mla_decode") ||
      !mla_ok(mla_merge_partials(d_parts, MLA_DTYPE_FP32, (const float*)d_lse_parts, PARTS,
                                 TOKENS, HEADS, d_mo, (float*)d_mlse, NULL),
              "mla_merge_partials"))
    return 1;
  if (!hip_ok(hipDeviceSynchronize(), "synchronize")) return 1;
  if (!hip_ok(hipMemcpy(o, d_o, sizeof(uint16_t) * TOKENS * HEADS * LATENT,
                        hipMemcpyDeviceToHost), "copy o") ||
      !hip_ok(hipMemcpy(lse, d_lse, sizeof(float) * TOKENS * HEADS, hipMemcpyDeviceToHost),
              "copy lse") ||
      !hip_ok(hipMemcpy(merged_o, d_mo, sizeof(uint16_t) * TOKENS * HEADS * LATENT,
                        hipMemcpyDeviceToHost), "copy merged o") ||
      !hip_ok(hipMemcpy(merged_lse, d_mlse, sizeof(float) * TOKENS * HEADS,
                        hipMemcpyDeviceToHost), "copy merged lse"))
    return 1;

  /* ---- files */
  if (!write_file(dir, "q.u8", q, (size_t)TOKENS * HEADS * ROW) ||
      !write_file(dir, "kv.u8", kv, (size_t)POOL * ROW) ||
      !write_file(dir, "kv_indptr.i32", kv_indptr, sizeof kv_indptr) ||
      !write_file(dir, "kv_indices.i32", kv_indices, sizeof(int32_t) * (size_t)n_idx) ||
      !write_file(dir, "o.u16", o, sizeof(uint16_t) * TOKENS * HEADS * LATENT) ||
      !write_file(dir, "lse.f32", lse, sizeof(float) * TOKENS * HEADS) ||
      !write_file(dir, "parts.f32", parts, sizeof(float) * PARTS * TOKENS * HEADS * LATENT) ||
      !write_file(dir, "lse_parts.f32", lse_parts, sizeof(float) * PARTS * TOKENS * HEADS) ||
      !write_file(dir, "merged_o.u16", merged_o, sizeof(uint16_t) * TOKENS * HEADS * LATENT) ||
      !write_file(dir, "merged_lse.f32", merged_lse, sizeof(float) * TOKENS * HEADS))
    return 1;

  hipFree(d_q);
  hipFree(d_kv);
  hipFree(d_o);
  hipFree(d_lse);
  hipFree(d_qo);
  hipFree(d_kvp);
  hipFree(d_idx);
  hipFree(d_scales);
  hipFree(d_ws);
  hipFree(d_parts);
  hipFree(d_lse_parts);
  hipFree(d_mo);
  hipFree(d_mlse);
  free(kv_indices);
  free(q);
  free(kv);
  free(parts);
  free(lse_parts);
  free(o);
  free(merged_o);
  free(lse);
  free(merged_lse);
  printf("c_abi_decode: ok (workspace %zu bytes)\n", ws_bytes);
  return 0;
}
