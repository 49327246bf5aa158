/*
 * Drives the library's host-side argument checks under AddressSanitizer and
 * UndefinedBehaviorSanitizer: the library is built for the host only (no
 * device code) with the sanitizers on, and every call below must be
 * rejected (or be a no-op) before the library touches a device, with the
 * status the header documents.  Also exercises the pure host functions
 * (the split plan with its environment override, the group cap, the status
 * strings).  No GPU is used; pointers are never dereferenced.
 */
#define _POSIX_C_SOURCE 200112L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ets_topk.h"

static int failures = 0;
#define EXPECT(expr, want)                                                           \
  do {                                                                               \
    const long got_ = (long)(expr);                                                  \
    if (got_ != (long)(want)) {                                                      \
      fprintf(stderr, "%s:%d: %s = %ld, want %ld\n", __FILE__, __LINE__, #expr, got_, \
              (long)(want));                                                         \
      ++failures;                                                                    \
    }                                                                                \
  } while (0)

int main(void) {
  void* fake = (void*)(uintptr_t)0x1000;
  float* fs = (float*)fake;
  int32_t* fi = (int32_t*)fake;
  /* raw */
  EXPECT(ets_topk_raw(fs, 64, 1, 64, NULL, 0, fi, 64, NULL, 0, NULL), ETS_ERR_K_RANGE);
  EXPECT(ets_topk_raw(fs, 64, 1, 64, NULL, 2049, fi, 4096, NULL, 0, NULL), ETS_ERR_K_RANGE);
  EXPECT(ets_topk_raw(fs, 64, -1, 64, NULL, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_raw(fs, 32, 1, 64, NULL, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_raw(fs, 64, 1, 64, NULL, 8, fi, 4, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_raw(fs, 64, 1, 64, NULL, 8, NULL, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_raw(NULL, 64, 1, 64, NULL, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_raw(NULL, 0, 0, 0, NULL, 8, NULL, 8, NULL, 0, NULL), ETS_OK);
  /* paged and its allocation-free variant */
  EXPECT(ets_topk_paged(fs, 64, 1, 64, fi, fi, 1, 0, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged(fs, 64, 1, 64, NULL, fi, 1, 64, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged(fs, 64, 1, 64, fi, NULL, 1, 64, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged(fs, 64, 1, 64, fi, fi, -1, 64, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged_window(fs, 64, 1, 64, fi, fi, fi, 1, 0, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged_window(fs, 64, 1, 64, fi, NULL, fi, 1, 64, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged_window(fs, 64, 1, 64, fi, fi, fi, 1, 64, 4096, fi, 4096, NULL, 0, NULL), ETS_ERR_K_RANGE);
  EXPECT(ets_topk_paged_window(NULL, 0, 0, 0, fi, NULL, NULL, 0, 64, 8, NULL, 8, NULL, 0, NULL), ETS_OK);
  EXPECT(ets_topk_paged_noalloc(fs, 64, 1, 64, fi, fi, 1, 64, 0, fi, 8, NULL, NULL), ETS_ERR_K_RANGE);
  EXPECT(ets_topk_paged_noalloc(fs, 64, 1, 64, fi, fi, 1, 0, 8, fi, 8, NULL, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged_noalloc(fs, 64, 1, 64, NULL, fi, 1, 64, 8, fi, 8, NULL, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_paged_noalloc(NULL, 0, 0, 0, NULL, NULL, 0, 64, 8, NULL, 8, NULL, NULL), ETS_OK);
  /* ragged */
  EXPECT(ets_topk_ragged(fs, NULL, fi, 1, 10, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_ragged(fs, fi, fi, 1, -1, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_topk_ragged(fs, fi, NULL, 1, 10, 8, fi, 8, NULL, 0, NULL), ETS_ERR_INVALID_ARG);
  /* floors */
  EXPECT(ets_floor_read(fs, 64, -1, 64, NULL, NULL, 0, (uint32_t*)fake, 64, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_floor_read(fs, 32, 1, 64, NULL, NULL, 0, (uint32_t*)fake, 64, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_floor_read(fs, 0, 1, 0, NULL, fi, 10, (uint32_t*)fake, 64, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_floor_read(NULL, 0, 0, 0, NULL, NULL, 0, NULL, 0, NULL), ETS_OK);
  EXPECT(ets_floor_launch(-1, 100, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_floor_launch(0, 100, NULL), ETS_OK);
  /* workspace calls */
  size_t n = 0;
  EXPECT(ets_workspace_size(4, 1000, 0, -1, &n), ETS_ERR_K_RANGE);
  EXPECT(ets_workspace_size(-1, 1000, 8, -1, &n), ETS_ERR_INVALID_ARG);
  EXPECT(ets_workspace_size(4, 1000, 8, -1, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_workspace_init(NULL, 0, NULL), ETS_OK);
  EXPECT(ets_workspace_init(NULL, 256, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_workspace_init((void*)(uintptr_t)0x1004, 256, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_workspace_error(fake, 4096, NULL, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_workspace_error(NULL, 4096, fi, NULL), ETS_ERR_INVALID_ARG);
  EXPECT(ets_workspace_error(fake, 128, fi, NULL), ETS_ERR_INVALID_ARG);
  int32_t a = 0, b = 0, c = 0;
  EXPECT(ets_device_limits(-1, NULL, &b, &c), ETS_ERR_INVALID_ARG);
  /* pure host functions */
  EXPECT(ets_group_cap(256, 8, 1), 32);
  EXPECT(ets_group_cap(304, 8, 3), 64);
  EXPECT(ets_group_cap(0, 8, 1), 0);
  EXPECT(ets_ticket_cap(256, 8, 1), 8);
  EXPECT(ets_ticket_cap(0, 8, 1), 0);
  (void)a;
  unsetenv("ETS_ROW_SPLIT");
  EXPECT(ets_row_split(4, 262144, 256, 8, 1), 16);
  EXPECT(ets_row_split(64, 32768, 256, 8, 1), 0);
  EXPECT(ets_row_split(192, 65536, 256, 8, 1), 2);
  EXPECT(ets_row_split(1, (int64_t)1 << 40, 256, 0, 1), 64);
  EXPECT(ets_row_split(2147483647, (int64_t)1 << 40, 256, 8, 1), 32);
  EXPECT(ets_row_split(2147483647, 262144, 256, 8, 1), 8);
  setenv("ETS_ROW_SPLIT", "7", 1);
  EXPECT(ets_row_split(4, 262144, 256, 8, 1), 7);
  setenv("ETS_ROW_SPLIT", "33", 1);
  EXPECT(ets_row_split(4, 262144, 256, 8, 1), -1);
  setenv("ETS_ROW_SPLIT", "99999999999999999999", 1);
  EXPECT(ets_row_split(4, 262144, 256, 8, 1), -1);
  setenv("ETS_ROW_SPLIT", "-3", 1);  /* not an override: the heuristic applies */
  EXPECT(ets_row_split(4, 262144, 256, 8, 1), 16);
  setenv("ETS_ROW_SPLIT", "4x", 1);
  EXPECT(ets_row_split(4, 262144, 256, 8, 1), 16);
  unsetenv("ETS_ROW_SPLIT");
  for (int s = -1; s <= 7; ++s) {
    const char* t = ets_status_string(s);
    if (t == NULL || strlen(t) == 0) ++failures;
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("host checks under ASan/UBSan: every call rejected as documented\n");
  return 0;
}
