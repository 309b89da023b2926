/* Host-side paths of the C ABI, for a run of the host library under AddressSanitizer and
 * UndefinedBehaviorSanitizer: the size and offset arithmetic of every footprint, the shape
 * checks (including shapes whose products would overflow), and the argument checks of every
 * entry point.  No kernel is launched.  Prints "ok" when every status is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static int fails = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "line %d: %s (%s)\n", __LINE__, #cond, kv_last_error()); \
      ++fails;                                                              \
    }                                                                       \
  } while (0)

static int64_t row_bytes(int bits, int d) { /* K or V row: codes + scales */
  if (bits == 16) return 2 * (int64_t)d;
  if (bits == 9) return d + d / 32;          /* fp8 codes + exponent bytes */
  return (bits == 8 ? d : d / 2) + 2 * (int64_t)(d / 32);
}

int main(void) {
  static const int kb[6] = {16, 8, 8, 4, 4, 9}, vb[6] = {16, 8, 4, 8, 4, 4};
  static const int dims[5] = {32, 64, 96, 128, 65536};
  static const int64_t toks[6] = {1, 255, 256, 257, 8192, 100500};
  for (int l = 0; l < 6; ++l)
    for (int di = 0; di < 5; ++di)
      for (int ti = 0; ti < 6; ++ti) {
        const int d = dims[di];
        const int64_t cap = (toks[ti] + 255) / 256 * 256;
        const int64_t want = 3 * 5 * cap * (row_bytes(kb[l], d) + row_bytes(vb[l], d));
        EXPECT(kv_layout_footprint_bytes(l, 3, 5, d, toks[ti]) == want);
      }
  /* layered: the sum of the layers' footprints */
  const int lay[6] = {0, 1, 2, 3, 4, 5};
  int64_t sum = 0;
  for (int l = 0; l < 6; ++l) sum += kv_layout_footprint_bytes(l, 1, 4, 128, 1000);
  EXPECT(kv_layered_footprint_bytes(lay, 6, 4, 128, 1000) == sum);
  /* invalid and overflowing shapes are statuses, never wrapped-around sizes */
  EXPECT(kv_layout_footprint_bytes(6, 1, 1, 64, 1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(-1, 1, 1, 64, 1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 0, 1, 64, 1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 1, -5, 64, 1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 1, 1, 33, 1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 1, 1, 1 << 17, 1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 1, 1, 64, 0) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 1, 1, 64, INT64_MAX) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 1, 1, 64, -1) == KV_EINVAL);
  EXPECT(kv_layout_footprint_bytes(2, 0x7fffffff, 0x7fffffff, 65536, (int64_t)1 << 31) == KV_EINVAL);
  EXPECT(kv_layered_footprint_bytes(NULL, 2, 1, 64, 1) == KV_EINVAL);
  const int bad[2] = {2, 17};
  EXPECT(kv_layered_footprint_bytes(bad, 2, 1, 64, 1) == KV_EINVAL);
  /* creation: bad shapes fail before any device call; a good shape either allocates (a GPU is
   * present) or fails with a status (none is) */
  EXPECT(kv_cache_create(2, 1, 1, 48, 10) == NULL && kv_last_status() == KV_EINVAL);
  EXPECT(kv_cache_create(2, 1, 1, 96, 10) == NULL && kv_last_status() == KV_EUNSUPPORTED);
  EXPECT(kv_cache_create_layered(bad, 2, 1, 64, 10) == NULL && kv_last_status() == KV_EINVAL);
  kv_cache* c = kv_cache_create(2, 1, 1, 64, 10);
  EXPECT(c != NULL || kv_last_status() < 0);
  kv_cache_destroy(c);
  /* every entry point with null handles */
  int n = 0;
  int64_t t = 0;
  EXPECT(kv_append_quant(NULL, 0, NULL, NULL, 0, 1, NULL) == KV_EINVAL);
  EXPECT(kv_attend_decode(NULL, 1, 0, NULL, 0, 4, 0.1f, NULL, NULL, 0, NULL) == KV_EINVAL);
  EXPECT(kv_attend_decode_static(NULL, 1, 0, NULL, 0, 4, 0.1f, NULL, NULL) == KV_EINVAL);
  EXPECT(kv_attend_chunk(NULL, 0, NULL, 0, 4, 1, 0.1f, NULL, NULL, 0, NULL) == KV_EINVAL);
  EXPECT(kv_decode_plan(NULL, 1, 0, 4, &n, &t) == KV_EINVAL);
  EXPECT(kv_decode_launch_kind(NULL, 1, 0, KV_BF16, 4, 0) == KV_EINVAL);
  EXPECT(kv_chunk_plan(NULL, 0, 4, 1, &n, &t) == KV_EINVAL);
  EXPECT(kv_attend_decode_partial(NULL, 1, 0, NULL, 0, 4, 0.1f, 1, 512, NULL, 0, NULL) == KV_EINVAL);
  EXPECT(kv_attend_chunk_partial(NULL, 0, NULL, 0, 4, 1, 0.1f, 1, 64, NULL, 0, NULL) == KV_EINVAL);
  EXPECT(kv_decode_workspace_bytes(NULL, 1, 0, 4) == KV_EINVAL);
  EXPECT(kv_chunk_workspace_bytes(NULL, 0, 4, 1) == KV_EINVAL);
  EXPECT(kv_footprint_bytes(NULL) == KV_EINVAL);
  EXPECT(kv_cache_len(NULL, 0) == KV_EINVAL);
  EXPECT(kv_cache_reset(NULL) == KV_EINVAL);
  EXPECT(kv_cache_truncate(NULL, 0, 0) == KV_EINVAL);
  EXPECT(kv_cache_layout(NULL, 0) == KV_EINVAL);
  EXPECT(kv_cache_shape(NULL, NULL, NULL, NULL, NULL) == KV_EINVAL);
  EXPECT(kv_cache_check_guard(NULL) == KV_EINVAL);
  EXPECT(kv_session_bytes(NULL) == KV_EINVAL);
  EXPECT(kv_session_save(NULL, NULL, 0, NULL) == KV_EINVAL);
  EXPECT(kv_session_load(NULL, NULL, 0, NULL) == KV_EINVAL);
  const void* p = NULL;
  int64_t rb = 0;
  EXPECT(kv_cache_plane(NULL, 0, 0, 0, &p, &rb) == KV_EINVAL);
  EXPECT(kv_cache_copy_plane(NULL, 0, 0, 0, 0, 1, NULL, NULL) == KV_EINVAL);
  kv_cache* two[2] = {NULL, NULL};
  EXPECT(kv_attend_decode(two, 2, 0, NULL, 0, 4, 0.1f, NULL, NULL, 0, NULL) == KV_EINVAL);
  EXPECT(kv_attend_decode(two, 0, 0, NULL, 0, 4, 0.1f, NULL, NULL, 0, NULL) == KV_EINVAL);
  /* the merge's own checks */
  EXPECT(kv_merge_partials(NULL, 0, 1, 64, NULL, NULL) == KV_OK);
  EXPECT(kv_merge_partials(NULL, 4, 1, 64, NULL, NULL) == KV_EINVAL);
  EXPECT(kv_merge_partials(NULL, 4, 0, 64, NULL, NULL) == KV_EINVAL);
  EXPECT(kv_merge_partials(NULL, -1, 1, 64, NULL, NULL) == KV_EINVAL);
  EXPECT(kv_merge_partials(NULL, INT64_MAX, 1, 64, NULL, NULL) == KV_EUNSUPPORTED);
  EXPECT(kv_merge_partials((const float*)8, 4, 1, 64, (float*)24, NULL) == KV_EINVAL);
  /* a long message is truncated, never overflowed */
  EXPECT(strlen(kv_last_error()) > 0 && strlen(kv_last_error()) < 512);
  if (fails) return 1;
  printf("ok\n");
  return 0;
}
