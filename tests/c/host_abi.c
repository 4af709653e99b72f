/* A plain C (C99) caller of libpkv's host-side entry points: it includes
 * include/pkv.h with no C++ and no HIP headers, links against libpkv.so and
 * checks the step metadata of two small steps (one-token pages and 4-token
 * pages) against values worked out by hand, plus the checked mode.  Prints
 * "ok" and exits 0 on success. */
#include <stdio.h>
#include <string.h>

#include "pkv.h"

static int expect(int cond, const char *what) {
  if (!cond) fprintf(stderr, "FAILED: %s\n", what);
  return cond ? 0 : 1;
}

int main(void) {
  int bad = 0;
  /* one-token pages: rows 2, 0, 1 with 3, 5, 2 tokens, 1, 2, 2 of them new */
  const int32_t table[3 * 6] = {10, 11, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25,
                                30, 31, 32, 33, 34, 35};
  const int32_t rows[3] = {2, 0, 1}, lens[3] = {3, 5, 2}, qlens[3] = {1, 2, 2};
  int32_t kv[4], qo[4], loc[8], order[3], max_len = 0, max_q = 0;
  int64_t n_new = 0;
  pkv_status st = pkv_build_step(3, rows, lens, qlens, table, 3, 6, 1, kv, qo, loc, 8, &n_new,
                                 &max_len, &max_q, order);
  bad |= expect(st == PKV_OK, "build_step status");
  const int32_t want_loc[5] = {32, 13, 14, 20, 21}, want_kv[4] = {0, 3, 8, 10};
  bad |= expect(n_new == 5 && memcmp(loc, want_loc, sizeof want_loc) == 0, "out_cache_loc");
  bad |= expect(memcmp(kv, want_kv, sizeof want_kv) == 0, "kv_indptr");
  bad |= expect(max_len == 5 && max_q == 2 && order[0] == 1, "host scalars and order");
  bad |= expect(pkv_validate_step(64, 3, 6, 1, table, 3, rows, lens, kv, qo, loc, n_new,
                                  order) == PKV_OK, "validate good step");
  loc[1] = loc[0];
  bad |= expect(pkv_validate_step(64, 3, 6, 1, table, 3, rows, lens, kv, qo, loc, n_new,
                                  NULL) == PKV_ERR_BAD_METADATA, "validate duplicate slot");

  /* 4-token pages: request on page-table row 1 = pages [5, 2], 6 tokens, 2 new:
   * positions 4, 5 -> page 2 offsets 0, 1 -> slots 8, 9 */
  const int32_t ptable[2 * 2] = {0, 1, 5, 2};
  const int32_t prow[1] = {1}, plen[1] = {6}, pq[1] = {2};
  st = pkv_build_step(1, prow, plen, pq, ptable, 2, 8, 4, kv, qo, loc, 8, &n_new, &max_len,
                      &max_q, NULL);
  bad |= expect(st == PKV_OK && n_new == 2 && loc[0] == 8 && loc[1] == 9, "paged write slots");
  bad |= expect(pkv_validate_step(24, 2, 8, 4, ptable, 1, prow, plen, kv, qo, loc, n_new,
                                  NULL) == PKV_OK, "paged validate");
  bad |= expect(pkv_build_step(1, prow, plen, pq, ptable, 2, 8, 3, kv, qo, loc, 8, &n_new,
                               &max_len, &max_q, NULL) == PKV_ERR_SHAPE, "page size 3 refused");

  bad |= expect(pkv_decode_workspace_bytes(1, 32, 128, 128) == (size_t)32 * 128 * 130 * 4,
                "workspace bytes");
  bad |= expect(strcmp(pkv_status_string(PKV_ERR_WORKSPACE_TOO_SMALL), "workspace too small") == 0,
                "status string");
  if (!bad) printf("ok\n");
  return bad;
}
