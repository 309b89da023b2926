/* A C99 caller of the library: the header must compile as plain C and the calls must link.
 * It runs only the host-side entry points (no device needed). */
#include <stdio.h>
#include <string.h>

#include "kvq.h"

int main(void) {
  /* the 22-layer x 4 KV-head x 64 table shape at 8192 tokens, K8V4: 71.50 MiB */
  const int64_t b = kv_layout_footprint_bytes(KV_K8V4, 22, 4, 64, 8192);
  if (b != 74973184) {
    fprintf(stderr, "footprint %lld\n", (long long)b);
    return 1;
  }
  const int layouts[3] = {KV_K8V8, KV_K4V4, KV_KF8V4};
  if (kv_layered_footprint_bytes(layouts, 3, 2, 128, 300) <= 0) return 2;
  /* an invalid layout is a status plus a message, never a crash */
  if (kv_layout_footprint_bytes(99, 1, 1, 64, 1) != KV_EINVAL) return 3;
  if (kv_last_status() != KV_EINVAL || strlen(kv_last_error()) == 0) return 4;
  if (kv_cache_len(NULL, 0) != KV_EINVAL) return 5;
  kv_cache_destroy(NULL);
  printf("ok\n");
  return 0;
}
