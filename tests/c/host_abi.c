/* A plain C (C99) caller of libpkv's host-side entry points: it includes
 * include/pkv.h with no C++ and no HIP headers, links against libpkv.so and
 * checks the step metadata of two small steps (one-token pages and 4-token
 * pages) against values worked out by hand, plus the checked mode.  Prints
 * "ok" and exits 0 on success. */
#include <stddef.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pkv.h"

static int expect(int cond, const char *what) {
  if (!cond) fprintf(stderr, "FAILED: %s\n", what);
  return cond ? 0 : 1;
}

int main(int argc, char **argv) {
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
  /* Load policy: a zeroed pool field is PKV_LOAD_AUTO, which streams a
   * one-request step whose K/V over all layers exceed 256 MiB. */
  pkv_pool pool;
  memset(&pool, 0, sizeof pool);
  pool.k_buffer = pool.v_buffer = (void *)0x1000;
  pool.req_to_token = (const int32_t *)0x2000;
  pool.n_layers = 32;
  pool.size = 65536;
  pool.num_reqs = 1;
  pool.max_ctx_len = 32768;
  pool.n_kv_heads = 8;
  pool.head_dim = 128;
  pool.dtype = PKV_BF16;
  bad |= expect(pkv_decode_load_kind(&pool, 1, 32768) == 1, "auto: one long request streams");
  bad |= expect(pkv_decode_load_kind(&pool, 1, 1024) == 0, "auto: short request cached");
  bad |= expect(pkv_decode_load_kind(&pool, 2, 32768) == 0, "auto: batches cached");
  pool.load_policy = PKV_LOAD_STREAM;
  bad |= expect(pkv_decode_load_kind(&pool, 64, 16) == 1, "stream policy");

  /* The ctypes binding's layout (sizes and the offset of the last pool
   * field, passed by the test) matches the compiler's. */
  if (argc == 4) {
    bad |= expect(sizeof(pkv_pool) == (size_t)atol(argv[1]), "sizeof pkv_pool");
    bad |= expect(offsetof(pkv_pool, load_policy) == (size_t)atol(argv[2]),
                  "offset of pkv_pool.load_policy");
    bad |= expect(sizeof(pkv_step) == (size_t)atol(argv[3]), "sizeof pkv_step");
  }
  if (!bad) printf("ok\n");
  return bad;
}
