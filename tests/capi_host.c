/* Plain C client of include/ra.h, host-side entry points only (no device
 * memory, no kernel): built and run by tests/test_capi_c.py to show that the
 * header is valid C99 and that the library is usable without Python. Prints
 * "ok" and returns 0 when every check holds; prints the failed check and
 * returns 1 otherwise. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ra.h"

static int failures = 0;
#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      printf("FAILED line %d: %s\n", __LINE__, #cond);         \
      ++failures;                                              \
    }                                                          \
  } while (0)

static ra_problem problem(int64_t len, int32_t n, int32_t r, int32_t layout) {
  ra_problem p;
  memset(&p, 0, sizeof p);
  p.dtype = RA_BF16;
  p.batch = 1;
  p.hq = 8;
  p.hkv = 2;
  p.head_dim = 128;
  p.q_len = len;
  p.kv_len = len;
  p.n_ring = n;
  p.rank = r;
  p.causal = 1;
  p.layout = layout;
  p.scale = 0.0f;
  return p;
}

int main(void) {
  /* contiguous, rank 2 of 4: block 1 is fully visible, block 3 fully masked,
   * block 2 (the diagonal) splits into FULL below, PARTIAL on and SKIP above
   * the diagonal of its tile grid */
  const int64_t len = 1024;
  const int32_t t = 128, nt = (int32_t)(len / t);
  ra_problem p = problem(len, 4, 2, RA_LAYOUT_CONTIGUOUS);
  CHECK(ra_tile_class_host(&p, 1, 0, len - 1, 0, len - 1) == RA_TILE_FULL);
  CHECK(ra_tile_class_host(&p, 3, 0, len - 1, 0, len - 1) == RA_TILE_SKIP);
  CHECK(ra_tile_class_host(&p, 2, 0, 127, 0, 127) == RA_TILE_PARTIAL);
  CHECK(ra_tile_class_host(&p, 2, 128, 255, 0, 127) == RA_TILE_FULL);
  CHECK(ra_tile_class_host(&p, 2, 0, 127, 128, 255) == RA_TILE_SKIP);
  CHECK(ra_tile_class_host(&p, 7, 0, 1, 0, 1) == -1); /* block out of range */

  int8_t* cls = (int8_t*)malloc((size_t)nt * nt);
  CHECK(ra_tile_classes_host(&p, 2, t, t, cls) == RA_OK);
  int full = 0, partial = 0, skip = 0;
  for (int32_t a = 0; a < nt; ++a)
    for (int32_t b = 0; b < nt; ++b) {
      const int8_t c = cls[a * nt + b];
      full += c == RA_TILE_FULL;
      partial += c == RA_TILE_PARTIAL;
      skip += c == RA_TILE_SKIP;
      CHECK(c == (b < a ? RA_TILE_FULL : b == a ? RA_TILE_PARTIAL : RA_TILE_SKIP));
    }
  CHECK(full == nt * (nt - 1) / 2 && partial == nt && skip == nt * (nt - 1) / 2);
  free(cls);

  /* workspace: positive for a valid problem, 0 for an invalid one */
  CHECK(ra_ring_workspace_bytes(&p) > 0);
  ra_problem bad = p;
  bad.rank = 4;
  CHECK(ra_ring_workspace_bytes(&bad) == 0);

  /* argument validation happens before any HIP call: a null input returns
   * RA_ERR_INVALID_ARG with a message, an unsupported head_dim
   * RA_ERR_UNSUPPORTED */
  CHECK(ra_block_attn_partial(&p, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == RA_ERR_INVALID_ARG);
  const char* msg = ra_last_error();
  CHECK(msg != NULL && strlen(msg) > 0);
  ra_problem odd = p;
  odd.head_dim = 96;
  CHECK(ra_ring_workspace_bytes(&odd) == 0);
  CHECK(ra_block_attn_partial(&odd, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != RA_OK);
  /* the running update validates exactly as the partial does */
  CHECK(ra_block_attn_accumulate(&p, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == RA_ERR_INVALID_ARG);
  CHECK(ra_block_attn_accumulate(&odd, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == RA_ERR_UNSUPPORTED);
  CHECK(ra_block_attn_accumulate(&p, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == RA_ERR_INVALID_ARG);

  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
