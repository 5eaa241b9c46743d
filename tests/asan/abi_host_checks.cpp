// Host-only checks of the C ABI's argument validation, built with the
// address and undefined-behaviour sanitizers (tests/test_asan_host.py).
// Every call here is rejected (or is a documented no-op) before any HIP call,
// so no GPU is needed; the sanitizers watch the validation code itself: the
// slice bookkeeping, the size arithmetic at extreme sizes, the error buffer.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lora.h"

static int failures = 0;

static void expect(const char* what, lora_status got, lora_status want) {
  const char* msg = lora_last_error();
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d (%s), wanted %d; last error '%s'\n", what, (int)got,
            lora_status_string(got), (int)want, msg);
    ++failures;
  }
  if (want != LORA_OK && strlen(msg) == 0) {
    fprintf(stderr, "FAIL %s: no error description\n", what);
    ++failures;
  }
}

int main() {
  char* const F = reinterpret_cast<char*>(0x10000);  // aligned, never dereferenced
  const void* A8[8] = {F, F, F, F, F, F, F, F};
  const void* B8[8] = {F, F, F, F, F, F, F, F};
  int64_t sizes8[8] = {64, 64, 64, 64, 64, 64, 64, 64};
  int64_t offs8[8] = {0, 64, 128, 192, 256, 320, 384, 448};
  int64_t overlap[8] = {0, 32, 128, 192, 256, 320, 384, 448};

  // sizes and offsets at the limits
  if (lora_segments_bytes(-1, 4) != 0 || lora_segments_bytes(10, 0) != 0 || lora_segments_bytes(10, 1025) != 0)
    ++failures;
  if (lora_segments_bytes(INT32_MAX, 1024) == 0) ++failures;
  if (lora_segments_offset(INT32_MAX, 1024, LORA_SEG_TILES) <= 0) ++failures;
  if (lora_segments_offset(10, 4, (lora_seg_field)99) != -1) ++failures;
  if (lora_shrink_expand_workspace_bytes(INT32_MAX, 1024, 8, 64) == 0) ++failures;
  if (lora_shrink_expand_workspace_bytes(4, 4, 9, 8) != 0) ++failures;
  if (lora_mask_workspace_bytes(LORA_BF16, INT32_MAX, INT32_MAX, 2, 8, 64) == 0) ++failures;
  if (lora_mask_workspace_bytes(LORA_BF16, 10, 64, 3, 1, 64) != 0) ++failures;  // 192 lanes
  if (strcmp(lora_status_string((lora_status)1234), "LORA_ERR_UNKNOWN") != 0) ++failures;

  // shrink
  expect("shrink dtype", lora_shrink((lora_dtype)7, F, 64, 8, 64, 1, A8, 4, 16, nullptr, nullptr, F, 1,
                                     (float*)F, nullptr), LORA_ERR_INVALID_ARG);
  expect("shrink ldx", lora_shrink(LORA_F16, F, 32, 8, 64, 1, A8, 4, 16, nullptr, nullptr, F, 1, (float*)F,
                                   nullptr), LORA_ERR_INVALID_ARG);
  expect("shrink 9 slices", lora_shrink(LORA_F16, F, 64, 8, 64, 9, A8, 4, 16, nullptr, nullptr, F, 1,
                                        (float*)F, nullptr), LORA_ERR_UNSUPPORTED);
  expect("shrink x > 4 GiB", lora_shrink(LORA_F16, F, (int64_t)1 << 40, 8, 64, 1, A8, 4, 16, nullptr, nullptr,
                                         F, 1, (float*)F, nullptr), LORA_ERR_UNSUPPORTED);
  expect("shrink inactive", lora_shrink(LORA_F16, F, 64, 8, 64, 8, A8, 4, 16, nullptr, nullptr, F, 0,
                                        (float*)F, nullptr), LORA_OK);
  // expand: eight slices, overlapping slices, a slice past ldy, bad layouts
  expect("expand overlap", lora_expand(LORA_BF16, (float*)F, 0, 8, 8, B8, sizes8, overlap, 4, 16, nullptr, 0,
                                       F, 1, F, 512, nullptr), LORA_ERR_INVALID_ARG);
  expect("expand past ldy", lora_expand(LORA_BF16, (float*)F, 0, 8, 8, B8, sizes8, offs8, 4, 16, nullptr, 0, F,
                                        1, F, 448, nullptr), LORA_ERR_INVALID_ARG);
  expect("expand layout", lora_expand(LORA_BF16, (float*)F, 0, 8, 8, B8, sizes8, offs8, 4, 16, nullptr, 7, F,
                                      1, F, 512, nullptr), LORA_ERR_INVALID_ARG);
  expect("expand inactive", lora_expand(LORA_BF16, (float*)F, 0, 8, 8, B8, sizes8, offs8, 4, 16, nullptr, 1, F,
                                        0, F, 512, nullptr), LORA_OK);
  // one-call forms
  expect("fused short workspace",
         lora_shrink_expand(LORA_F16, F, 64, 8, 64, 1, A8, B8, sizes8, offs8, 4, 16, nullptr, 0, nullptr, F,
                            nullptr, 1, nullptr, F, 64, F, 1024, nullptr), LORA_ERR_INVALID_ARG);
  expect("fused inactive",
         lora_shrink_expand(LORA_F16, F, 64, 8, 64, 8, A8, B8, sizes8, offs8, 4, 16, nullptr, 0, nullptr, F,
                            nullptr, 0, nullptr, F, 512, F, lora_shrink_expand_workspace_bytes(8, 4, 8, 16),
                            nullptr), LORA_OK);
  expect("noalloc too large",
         lora_shrink_expand_noalloc(LORA_BF16, F, 64, 16384, 64, 8, A8, B8, sizes8, offs8, 4, 64, nullptr, 0,
                                    nullptr, F, nullptr, 1, nullptr, F, 512, nullptr, nullptr),
         LORA_ERR_UNSUPPORTED);
  expect("mask lanes", lora_shrink_expand_mask(LORA_F16, F, 64, 8, 64, 1, A8, B8, sizes8, offs8, 3, 64, nullptr,
                                               nullptr, (const int32_t*)F, 1, nullptr, F, 64, F, 1 << 20, nullptr),
         LORA_ERR_UNSUPPORTED);
  expect("mask inactive", lora_shrink_expand_mask(LORA_F16, F, 64, 8, 64, 8, A8, B8, sizes8, offs8, 2, 64,
                                                  nullptr, nullptr, (const int32_t*)F, 0, nullptr, F, 512, F,
                                                  1 << 20, nullptr), LORA_OK);
  // segment build, embedding, slot copy
  expect("build mode", lora_build_segments((const int32_t*)F, 4, 4, 9, F, nullptr, nullptr), LORA_ERR_INVALID_ARG);
  expect("embedding table size", lora_embedding_shrink(LORA_BF16, (const int32_t*)F, 8, (int64_t)1 << 40, F, 1024,
                                                       64, nullptr, nullptr, (const int32_t*)F, 1, (float*)F,
                                                       nullptr), LORA_ERR_UNSUPPORTED);
  expect("embedding inactive", lora_embedding_shrink(LORA_BF16, (const int32_t*)F, 8, 100, F, 4, 64, nullptr,
                                                     nullptr, (const int32_t*)F, 0, (float*)F, nullptr), LORA_OK);
  expect("copy too large", lora_copy_padded(LORA_F16, F, 9, 8, 8, 0, F, 8, 8, 8, nullptr), LORA_ERR_INVALID_ARG);
  expect("copy stride", lora_copy_padded(LORA_F16, F, 8, 4, 4, 1, F, 8, 4, 4, nullptr), LORA_ERR_INVALID_ARG);
  expect("copy empty", lora_copy_padded(LORA_F16, nullptr, 0, 0, 0, 0, F, 0, 8, 8, nullptr), LORA_OK);
  expect("errors null", lora_workspace_errors(nullptr, nullptr, nullptr), LORA_ERR_INVALID_ARG);

  if (failures) {
    fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
