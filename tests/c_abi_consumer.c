/* A plain C99 caller of the library (built and run by tests/test_abi.py on
 * the CPU): includes the public header as C, links libsink_attn.so, and
 * makes only calls that need no device -- the planning queries and
 * argument validation, which fails before anything is enqueued.  Fake,
 * aligned addresses stand in for device pointers: validation never
 * dereferences them. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sink_attn.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "failed at line %d: %s\n", __LINE__, #cond);   \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  const char* version = sink_attn_version();
  CHECK(version != NULL && strlen(version) > 0);
  for (int s = SINK_ATTN_OK; s <= SINK_ATTN_ERR_HIP; ++s) {
    const char* text = sink_attn_status_string((sink_attn_status)s);
    CHECK(text != NULL && strlen(text) > 0);
  }

  /* planning queries: host arithmetic only */
  CHECK(sink_attn_decode_workspace_size(4, 64, 8, 64, 131072, 32) > 0);
  CHECK(sink_attn_decode_num_splits(4, 64, 8, 131072, 32) == 32);

  void* const dev = (void*)(uintptr_t)0x10000;
  void* const out = (void*)(uintptr_t)0x20000;
  const int32_t* const idx = (const int32_t*)(uintptr_t)0x30000;

  /* a prefill without queries: rejected on the host, with a detail */
  sink_attn_status st = sink_attn_prefill(NULL, idx, dev, dev, idx, NULL, NULL, NULL, 1, 64, 8, 64,
                                          16, 128, 128, 128, 0.125f, 1, out, SINK_ATTN_F32, NULL,
                                          NULL);
  CHECK(st == SINK_ATTN_ERR_NULL_ARG);
  CHECK(strlen(sink_attn_last_error()) > 0);

  /* an unsupported head size */
  st = sink_attn_prefill(dev, idx, dev, dev, idx, NULL, NULL, NULL, 1, 64, 8, 128, 16, 128, 128,
                         128, 0.125f, 1, out, SINK_ATTN_F32, NULL, NULL);
  CHECK(st == SINK_ATTN_ERR_UNSUPPORTED);

  /* a group size that does not divide the query heads */
  st = sink_attn_decode(dev, dev, dev, idx, idx, idx, NULL, 4, 60, 8, 64, 16, 4096, 0, 0.125f, out,
                        SINK_ATTN_BF16, NULL, dev, 0, NULL);
  CHECK(st == SINK_ATTN_ERR_BAD_SHAPE);

  /* an empty prefill is a no-op: nothing to enqueue, no error */
  st = sink_attn_prefill(dev, idx, dev, dev, idx, NULL, NULL, NULL, 1, 64, 8, 64, 16, 0, 0, 0,
                         0.125f, 1, out, SINK_ATTN_F32, NULL, NULL);
  CHECK(st == SINK_ATTN_OK);

  printf("c consumer ok (%s)\n", version);
  return 0;
}
