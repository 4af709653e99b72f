/* Deterministic fuzz of the host entry points of libpkv (no device calls):
 * pkv_build_step, pkv_validate_step, pkv_build_positions, pkv_prefill_blocks,
 * pkv_decode_prefix_groups, pkv_decode_pick_splits, pkv_decode_load_kind,
 * pkv_decode_workspace_bytes, on random shapes, random (often invalid)
 * metadata and tables, and capacities that are exact or one short.  Every
 * buffer is a heap block of exactly its stated length, so a read or write
 * past it is caught when the library is built with AddressSanitizer.  The
 * program checks that each status is a defined one and that reported counts
 * stay within the capacities, and prints "ok". */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "pkv.h"

static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static uint32_t next_u32(void) {  /* xorshift64* */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545f4914f6cdd1dull) >> 32);
}

/* uniform in [lo, hi] */
static int32_t rnd(int32_t lo, int32_t hi) { return lo + (int32_t)(next_u32() % (uint32_t)(hi - lo + 1)); }

static int32_t *alloc_i32(int64_t n) {
  int32_t *p = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
  if (!p) exit(3);
  return p;
}

static int status_ok(pkv_status s) { return s >= PKV_OK && s <= PKV_ERR_SCRATCH_LIMIT; }

int main(void) {
  int bad = 0;
  for (int it = 0; it < 4000 && !bad; ++it) {
    const int32_t page_sizes[5] = {1, 1, 2, 16, 3};
    const int32_t ps = page_sizes[rnd(0, 4)];           /* 3 is refused */
    const int64_t num_reqs = rnd(1, 12);
    const int64_t max_ctx = rnd(1, 160);
    const int64_t per_row = (max_ctx + (ps > 0 ? ps : 1) - 1) / (ps > 0 ? ps : 1);
    const int64_t size = (int64_t)rnd(1, 400) * (ps == 3 ? 1 : ps);
    const int32_t batch = rnd(0, 10);
    const int prefill = rnd(0, 1);

    int32_t *table = alloc_i32(num_reqs * per_row);
    const int64_t units = ps == 3 ? size : size / ps;
    for (int64_t i = 0; i < num_reqs * per_row; ++i)
      table[i] = rnd(0, 9) == 0 ? rnd(-2, (int32_t)units + 2) : rnd(0, (int32_t)(units > 0 ? units - 1 : 0));
    int32_t *rows = alloc_i32(batch), *lens = alloc_i32(batch), *qls = alloc_i32(batch);
    for (int32_t b = 0; b < batch; ++b) {
      rows[b] = rnd(0, 19) == 0 ? rnd(-1, (int32_t)num_reqs) : rnd(0, (int32_t)num_reqs - 1);
      lens[b] = rnd(0, 19) == 0 ? rnd(-1, (int32_t)max_ctx + 2) : rnd(1, (int32_t)max_ctx);
      qls[b] = prefill ? (lens[b] > 0 ? rnd(0, lens[b]) : 0) : 1;
    }
    int64_t want_new = 0;
    for (int32_t b = 0; b < batch; ++b) want_new += qls[b] > 0 ? qls[b] : 0;
    const int64_t cap = want_new - (rnd(0, 7) == 0 ? 1 : 0);  /* sometimes one short */
    const int64_t room = cap > 0 ? cap : 0;  /* entries the library may write */

    int32_t *kv = alloc_i32(batch + 1), *qo = alloc_i32(batch + 1), *loc = alloc_i32(cap);
    int32_t *order = alloc_i32(batch);
    int64_t n_new = -1;
    int32_t max_len = -1, max_q = -1;
    pkv_status st = pkv_build_step(batch, rows, lens, prefill ? qls : NULL, table, num_reqs,
                                   max_ctx, ps, kv, qo, loc, cap, &n_new, &max_len, &max_q,
                                   order);
    if (!status_ok(st)) { fprintf(stderr, "build_step status %d\n", (int)st); bad = 1; }
    if (st == PKV_OK && (n_new < 0 || n_new > room)) { fprintf(stderr, "n_new %lld\n", (long long)n_new); bad = 1; }
    if (st == PKV_OK) {
      /* the built step validates, and random single corruptions never crash */
      pkv_status v = pkv_validate_step(size, num_reqs, max_ctx, ps, table, batch, rows, lens, kv,
                                       prefill ? qo : NULL, loc, n_new, order);
      if (!status_ok(v)) { fprintf(stderr, "validate status %d\n", (int)v); bad = 1; }
      if (n_new > 0 && rnd(0, 1)) loc[rnd(0, (int32_t)n_new - 1)] = rnd(-3, (int32_t)size + 3);
      if (batch > 0 && rnd(0, 1)) kv[rnd(0, batch)] = rnd(-3, 500);
      v = pkv_validate_step(size, num_reqs, max_ctx, ps, table, batch, rows, lens, kv,
                            prefill ? qo : NULL, loc, n_new, order);
      if (!status_ok(v)) { fprintf(stderr, "validate (corrupt) status %d\n", (int)v); bad = 1; }
    }

    /* positions: exact capacity or one short */
    int32_t *pos = alloc_i32(cap);
    int64_t n_pos = -1;
    st = pkv_build_positions(batch, lens, prefill ? qls : NULL, pos, cap, &n_pos);
    if (!status_ok(st) || (st == PKV_OK && (n_pos < 0 || n_pos > room))) { fprintf(stderr, "positions\n"); bad = 1; }

    /* prefill launch schedule */
    if (prefill) {
      const int32_t hk = rnd(1, 4), heads = hk * rnd(1, 6);
      int64_t blk_cap = 0;
      for (int32_t b = 0; b < batch; ++b)
        blk_cap += ((int64_t)(qls[b] > 0 ? qls[b] : 0) * (heads / hk) + PKV_PREFILL_BLOCK_ROWS - 1) /
                   PKV_PREFILL_BLOCK_ROWS;
      blk_cap -= rnd(0, 5) == 0 ? 1 : 0;
      if (blk_cap < 0) blk_cap = 0;
      int32_t *blocks = alloc_i32(2 * blk_cap);
      int64_t n_blocks = -1;
      st = pkv_prefill_blocks(batch, qls, rnd(0, 1) ? order : NULL, heads, hk, blocks, blk_cap,
                              &n_blocks);
      if (!status_ok(st) || (st == PKV_OK && (n_blocks < 0 || n_blocks > blk_cap))) { fprintf(stderr, "blocks\n"); bad = 1; }
      free(blocks);
    }

    /* prefix groups of a decode step */
    if (!prefill) {
      const int64_t groups_cap = rnd(0, batch);
      int32_t *groups = alloc_i32(groups_cap * PKV_PREFIX_GROUP_INTS);
      int32_t *kv_start = alloc_i32(batch);
      int64_t n_groups = -1;
      int32_t max_prefix = -1, max_members = -1, max_suffix = -1;
      st = pkv_decode_prefix_groups(batch, rows, lens, table, num_reqs, max_ctx, ps, rnd(1, 64),
                                    groups, groups_cap, &n_groups, kv_start, &max_prefix,
                                    &max_members, &max_suffix);
      if (!status_ok(st) || (st == PKV_OK && (n_groups < 0 || n_groups > groups_cap))) { fprintf(stderr, "groups\n"); bad = 1; }
      free(groups);
      free(kv_start);
    }

    /* scalar choices */
    const int32_t s = pkv_decode_pick_splits(rnd(-1, 300), rnd(-1, 16), rnd(-1, 128),
                                             rnd(-1, 200000), rnd(-1, 1 << 22), rnd(-1, 4096));
    if (s < 1) { fprintf(stderr, "pick_splits %d\n", (int)s); bad = 1; }
    pkv_pool pool = {0};
    pool.n_layers = rnd(0, 64);
    pool.n_kv_heads = rnd(0, 16);
    pool.head_dim = rnd(0, 256);
    pool.v_head_dim = rnd(-1, 256);
    pool.dtype = (pkv_dtype)rnd(0, 2);
    pool.load_policy = rnd(-1, 3);
    const int32_t kind = pkv_decode_load_kind(rnd(0, 1) ? &pool : NULL, rnd(-1, 4), rnd(-1, 1 << 20));
    if (kind < -1 || kind > 1) { fprintf(stderr, "load_kind %d\n", (int)kind); bad = 1; }
    (void)pkv_decode_workspace_bytes(rnd(0, 64), rnd(0, 64), rnd(0, 256), rnd(0, 128));

    free(table); free(rows); free(lens); free(qls); free(kv); free(qo); free(loc); free(order);
    free(pos);
  }
  if (!bad) printf("ok\n");
  return bad;
}
