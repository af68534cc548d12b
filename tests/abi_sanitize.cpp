// Host-side check of the C ABI under AddressSanitizer and UndefinedBehavior-
// Sanitizer: layouts, status strings, the launch cap and every argument check
// that rejects a call before anything is enqueued. Nothing here reaches a GPU:
// every call either fails validation or has nothing to do, so the program
// runs on a machine without one. Exit status 0 when every result is the
// expected one; the sanitizers abort on the first error they find.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "taco.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                    \
  do {                                                                                        \
    const long long got_ = (long long)(expr);                                                 \
    if (got_ != (long long)(want)) {                                                          \
      fprintf(stderr, "line %d: %s = %lld, expected %lld\n", __LINE__, #expr, got_, (long long)(want)); \
      ++failures;                                                                             \
    }                                                                                         \
  } while (0)

int main() {
  const taco_codec fp8 = {TACO_FMT_FP8_DUAL, 128, 1, 0}, e5 = {TACO_FMT_FP8E5_DUAL, 128, 1, 0};
  const taco_codec i8s = {TACO_FMT_INT8_SYM, 64, 0, 0}, i4a = {TACO_FMT_INT4_ASYM, 128, 0, 0};
  const taco_codec i8a = {TACO_FMT_INT8_ASYM, 128, 0, 0}, bad_fmt = {9, 128, 0, 0};
  const taco_codec bad_blk = {TACO_FMT_FP8_DUAL, 96, 1, 0}, bad_res = {TACO_FMT_INT8_SYM, 64, 0, 7};

  // layouts, including the largest tensor accepted and one element more
  taco_layout_t L;
  memset(&L, 0xA5, sizeof(L));
  EXPECT(taco_layout(fp8, 4096, 4096, &L), TACO_OK);
  EXPECT(L.total_bytes, 4096LL * 4096 + 4096LL * 4096 / 128 + 256);
  EXPECT(taco_layout(i4a, 3, 384, &L), TACO_OK);
  EXPECT(L.aux_off, 1024);
  EXPECT(taco_layout(i8s, (int64_t)1 << 21, (int64_t)1 << 14, &L), TACO_OK);        // 2^35 elements
  EXPECT(taco_layout(i8s, ((int64_t)1 << 21) + 1, (int64_t)1 << 14, &L), TACO_ERR_INVALID_ARG);
  EXPECT(taco_layout(i8s, INT64_MAX, INT64_MAX, &L), TACO_ERR_SHAPE);                // cols % 64 != 0
  EXPECT(taco_layout(i8s, INT64_MAX, (int64_t)1 << 62, &L), TACO_ERR_INVALID_ARG);   // no overflow
  EXPECT(taco_layout(fp8, 2, 128, nullptr), TACO_ERR_INVALID_ARG);
  EXPECT(taco_layout(bad_fmt, 2, 128, &L), TACO_ERR_FORMAT);
  EXPECT(taco_layout(bad_blk, 2, 192, &L), TACO_ERR_SHAPE);
  EXPECT(taco_layout(bad_res, 2, 128, &L), TACO_ERR_INVALID_ARG);
  EXPECT(taco_compressed_bytes(i8a, 0, 128), 0);
  EXPECT(taco_compressed_bytes(i8a, 2, 100), TACO_ERR_SHAPE);
  EXPECT(taco_workspace_bytes(e5, 8, 128), TACO_WORKSPACE_BYTES);
  EXPECT(taco_workspace_bytes(i4a, 8, 128), 0);

  // status strings, every code and an unknown one
  for (int s = -8; s <= 1; ++s) EXPECT(taco_status_string(s) != nullptr, 1);
  EXPECT(strcmp(taco_status_string(TACO_ERR_ALIGN), "TACO_ERR_ALIGN"), 0);

  // launch cap: per thread, restorable
  int32_t prev = -1;
  EXPECT(taco_set_launch_limit(17, &prev), TACO_OK);
  EXPECT(prev, 0);
  EXPECT(taco_set_launch_limit(-1, &prev), TACO_ERR_INVALID_ARG);
  EXPECT(taco_set_launch_limit(0, nullptr), TACO_OK);

  // argument checks (fake, never dereferenced 16-byte aligned addresses)
  void* A = (void*)(uintptr_t)4096;
  void* B = (void*)(uintptr_t)(1 << 20);
  void* O = (void*)(uintptr_t)(1 << 21);
  char ws[64];
  EXPECT(taco_compress(fp8, nullptr, 2, 128, 1.0f, B, nullptr, 0, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_compress(fp8, (char*)A + 2, 2, 128, 1.0f, B, nullptr, 0, 0), TACO_ERR_ALIGN);
  EXPECT(taco_compress(fp8, A, 2, 128, 0.0f, B, nullptr, 0, 0), TACO_ERR_WORKSPACE);
  EXPECT(taco_compress(fp8, A, 2, 128, 0.0f, B, ws, sizeof(ws), 0), TACO_ERR_WORKSPACE);
  EXPECT(taco_compress(fp8, A, 2, 128, 1e30f, B, nullptr, 0, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_compress(fp8, A, 2, 128, 1.0f, A, nullptr, 0, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_compress(fp8, A, 0, 128, 1.0f, B, nullptr, 0, 0), TACO_OK);
  EXPECT(taco_compress_noalloc(fp8, A, 2, 100, 0.0f, B, 0), TACO_ERR_SHAPE);
  EXPECT(taco_compress_noalloc(e5, A, 0, 128, -1.0f, B, 0), TACO_OK);
  EXPECT(taco_compress_debug(i8s, A, 2, 64, 1.0f, B, nullptr, 0, nullptr, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_requantize(i8s, (const float*)A, 2, 96, 1.0f, B, nullptr, 0, 0), TACO_ERR_SHAPE);
  EXPECT(taco_decompress(i8s, A, 2, 64, B, 3, 0), TACO_ERR_INVALID_ARG);
  const void* shards[17];
  for (int r = 0; r < 17; ++r) shards[r] = (char*)A + (r << 16);
  EXPECT(taco_decompress_reduce(i8s, shards, 17, 4, 64, (float*)B, i8s, nullptr, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_decompress_reduce(i8s, shards, 2, 4, 64, nullptr, i8a, B, 0), TACO_ERR_SHAPE);   // no 128-group
  EXPECT(taco_decompress_reduce(i8s, shards, 2, 4, 128, nullptr, i8a, B, 0), TACO_ERR_FORMAT);
  EXPECT(taco_decompress_reduce(i4a, shards, 2, 4, 128, (float*)A, i8a, nullptr, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_decompress_reduce(fp8, shards, 16, 0, 128, (float*)B, fp8, nullptr, 0), TACO_OK);
  EXPECT(taco_ring_hop(fp8, A, B, 4, 128, (float*)O, fp8, nullptr, 0), TACO_ERR_FORMAT);
  EXPECT(taco_ring_hop(i8s, A, B, 4, 64, nullptr, i8s, nullptr, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_chunk_order(A, 2, 1000, (int32_t*)O, 0), TACO_ERR_SHAPE);
  EXPECT(taco_chunk_order(A, 2, 1024, (int32_t*)A, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_compress_reordered(fp8, A, 2, 1024, 1.0f, B, nullptr, 0, nullptr, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_compress_reordered(i8s, A, 1, 262144, 1.0f, B, nullptr, 0, (int32_t*)O, 0), TACO_ERR_SHAPE);
  EXPECT(taco_decompress_reordered(i8s, A, 2, 1024, B, 0, (int32_t*)((char*)O + 4), 0), TACO_ERR_ALIGN);
  EXPECT(taco_decompress_gemm(fp8, A, 128, 128, B, 128, O, 0, 0), TACO_ERR_FORMAT);        // Hadamard codec
  EXPECT(taco_decompress_gemm(i8a, A, 100, 128, B, 128, O, 0, 0), TACO_ERR_SHAPE);
  EXPECT(taco_decompress_gemm(i8a, A, 128, 128, B, 128, O, 2, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_decompress_gemm(i8a, A, 128, 128, B, 128, (char*)O + 8, 0, 0), TACO_ERR_ALIGN);
  EXPECT(taco_decompress_gemm(i8a, A, 1 << 18, 128, B, 1 << 18, O, 0, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_decompress_gemm(i8a, A, 128, 128, B, 128, (char*)A + 64, 0, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_decompress_gemm(i8a, nullptr, 0, 128, nullptr, 128, nullptr, 0, 0), TACO_OK);
  EXPECT(taco_e4m3_encode((const float*)A, (uint8_t*)A + 16, 64, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_e5m2_encode((const float*)A, nullptr, 16, 0), TACO_ERR_INVALID_ARG);
  EXPECT(taco_e5m2_encode((const float*)A, (uint8_t*)B, 0, 0), TACO_OK);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_sanitize: all checks passed\n");
  return 0;
}
