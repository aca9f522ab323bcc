/* The host half of the C ABI driven from plain C99 (no Python, no torch):
 * reserve budgets, size and build the block tables and the split plan for a
 * hand-worked batch, release a request, and check every value against the
 * numbers worked out by hand from the rules in include/tg.h.
 *
 * Batch: H = 2 KV-heads, head_rank {1, 0} (head 1 most important), ratio
 * band 0.5 .. 0.25, C = 2 clusters, everything bf16 (recent_ppm 1e6),
 * n_comp {100, 40}, pages of 16 rows, d = 128, items of up to 32 rows.
 *   ratio(rank 0) = 500000, ratio(rank 1) = 250000 ppm
 *   budgets: r0 (h0, h1) = (ceil(.25*100), ceil(.5*100)) = (25, 50);
 *            r1 = (ceil(.25*40), ceil(.5*40)) = (10, 20)
 *   clusters in rank order: cluster 0 = {h1}, cluster 1 = {h0}
 *   pages: cluster 0: r0 ceil(50/16) = 4, r1 ceil(20/16) = 2 -> ids 0..3, 4..5
 *          cluster 1: r0 ceil(25/16) = 2, r1 1            -> ids 0..1, 2
 *   plan (r, h, tier, t0, t1, slot), natural order: (0,0,bf16,0,25,0),
 *        (0,1,bf16,0,32,1), (0,1,bf16,32,50,2) [4 pages, 2 a chunk],
 *        (1,0,bf16,0,10,3), (1,1,bf16,0,20,4); part_off {0,1,3,4,5}
 * Exit status 0 when everything matches. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tg.h"

static int failures = 0;
#define CHECK(cond)                                                 \
  do {                                                              \
    if (!(cond)) {                                                  \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                   \
    }                                                               \
  } while (0)

static int same(const int32_t* a, const int32_t* b, int n) { return memcmp(a, b, (size_t)n * sizeof(int32_t)) == 0; }

int main(void) {
  enum { B = 2, H = 2, C = 2 };
  const int32_t rank[H] = {1, 0};
  const tg_budget_table bt = {H, rank, 500000, 250000, C, 1000000, 64};
  const int32_t n_comp[B] = {100, 40};
  int32_t budget[B * H], length[B * H], n_i8[B * H], n_bf[B * H], coh[H], sic[H], csize[C];
  tg_reservation res;
  memset(&res, 0, sizeof res);
  res.budget = budget;
  res.length = length;
  res.n_i8 = n_i8;
  res.n_bf = n_bf;
  res.cluster_of_head = coh;
  res.slot_in_cluster = sic;
  res.cluster_size = csize;
  CHECK(tg_reserve(&bt, B, n_comp, NULL, NULL, &res) == TG_OK);
  const int32_t want_budget[B * H] = {25, 50, 10, 20}, want_zero[B * H] = {0, 0, 0, 0};
  const int32_t want_coh[H] = {1, 0}, want_sic[H] = {0, 0}, want_csize[C] = {1, 1};
  CHECK(same(budget, want_budget, B * H) && same(length, want_budget, B * H));
  CHECK(same(n_bf, want_budget, B * H) && same(n_i8, want_zero, B * H));
  CHECK(same(coh, want_coh, H) && same(sic, want_sic, H) && same(csize, want_csize, C));

  const tg_plan_opts opts = {32, 64, 0, 0, 0, 0};
  tg_table_sizes sz;
  CHECK(tg_size_tables(&res, 16, 64, NULL, &opts, &sz) == TG_OK);
  CHECK(sz.n_items == 5 && sz.n_gitems == 0 && sz.n_slots == 5);
  CHECK(sz.stride[0][TG_TIER_BF16] == 4 && sz.stride[1][TG_TIER_BF16] == 2);
  CHECK(sz.pages_needed[0][TG_TIER_BF16] == 6 && sz.pages_needed[1][TG_TIER_BF16] == 3);
  CHECK(sz.pages_needed[0][TG_TIER_I8] == 0 && sz.pages_needed[1][TG_TIER_I8] == 0);

  const int64_t pages_bf[C] = {sz.pages_needed[0][TG_TIER_BF16], sz.pages_needed[1][TG_TIER_BF16]};
  const int64_t pages_i8[C] = {0, 0};
  tg_pool* pool = NULL;
  CHECK(tg_pool_create(C, csize, 128, 16, 64, 8, pages_bf, pages_i8, &pool) == TG_OK && pool != NULL);
  if (!pool) return 1;
  CHECK(tg_pool_page_bytes(pool, 0, TG_TIER_BF16) == 8192 && tg_pool_capacity(pool, 1, TG_TIER_BF16) == 3);

  int32_t bt0[B * 4], bt1[B * 2], len[B * H * 2], work[5 * 6], part_off[B * H + 1], released[B];
  tg_tables t;
  memset(&t, 0, sizeof t);
  t.bt[0][TG_TIER_BF16] = bt0;
  t.bt[1][TG_TIER_BF16] = bt1;
  t.stride[0][TG_TIER_BF16] = sz.stride[0][TG_TIER_BF16];
  t.stride[1][TG_TIER_BF16] = sz.stride[1][TG_TIER_BF16];
  t.len = len;
  t.work = work;
  t.n_items = sz.n_items;
  t.part_off = part_off;
  t.released = released;
  CHECK(tg_build_tables(pool, &res, NULL, &opts, &t) == TG_OK);
  const int32_t want_bt0[B * 4] = {0, 1, 2, 3, 4, 5, -1, -1}, want_bt1[B * 2] = {0, 1, 2, -1};
  const int32_t want_len[B * H * 2] = {0, 25, 0, 50, 0, 10, 0, 20};
  const int32_t want_work[5 * 6] = {0, 0, TG_TIER_BF16, 0, 25, 0,  0, 1, TG_TIER_BF16, 0, 32, 1,
                                    0, 1, TG_TIER_BF16, 32, 50, 2, 1, 0, TG_TIER_BF16, 0, 10, 3,
                                    1, 1, TG_TIER_BF16, 0, 20, 4};
  const int32_t want_off[B * H + 1] = {0, 1, 3, 4, 5};
  CHECK(same(bt0, want_bt0, B * 4) && same(bt1, want_bt1, B * 2));
  CHECK(same(len, want_len, B * H * 2));
  CHECK(same(work, want_work, 5 * 6));
  CHECK(same(part_off, want_off, B * H + 1));
  CHECK(tg_pool_free_pages(pool, 0, TG_TIER_BF16) == 0 && tg_pool_free_pages(pool, 1, TG_TIER_BF16) == 0);

  /* the pool is full: one more batch (into tables of its own, as a failed
     call leaves its outputs unspecified) changes nothing */
  int32_t xbt0[B * 4], xbt1[B * 2], xlen[B * H * 2], xwork[5 * 6], xoff[B * H + 1], xrel[B];
  tg_tables t2 = t;
  t2.bt[0][TG_TIER_BF16] = xbt0;
  t2.bt[1][TG_TIER_BF16] = xbt1;
  t2.len = xlen;
  t2.work = xwork;
  t2.part_off = xoff;
  t2.released = xrel;
  CHECK(tg_build_tables(pool, &res, NULL, &opts, &t2) == TG_ENOMEM);
  CHECK(tg_pool_free_pages(pool, 0, TG_TIER_BF16) == 0 && tg_pool_free_pages(pool, 1, TG_TIER_BF16) == 0);
  CHECK(tg_pool_refcount(pool, 0, TG_TIER_BF16, 5) == 1);

  /* releasing request 0 frees its 4 + 2 pages; twice is an error */
  CHECK(tg_release(pool, &t, 0) == TG_OK);
  CHECK(tg_pool_free_pages(pool, 0, TG_TIER_BF16) == 4 && tg_pool_free_pages(pool, 1, TG_TIER_BF16) == 2);
  CHECK(tg_release(pool, &t, 0) == TG_EINVAL);
  /* requests outside [0, B) are refused, and change nothing */
  CHECK(t.B == B);
  CHECK(tg_release(pool, &t, B) == TG_EINVAL && tg_release(pool, &t, -1) == TG_EINVAL);
  CHECK(tg_release(pool, &t, 1 << 30) == TG_EINVAL);
  CHECK(tg_pool_free_pages(pool, 0, TG_TIER_BF16) == 4 && tg_pool_free_pages(pool, 1, TG_TIER_BF16) == 2);
  CHECK(tg_pool_refcount(pool, 0, TG_TIER_BF16, 4) == 1 && tg_pool_refcount(pool, 0, TG_TIER_BF16, 0) == 0);
  tg_pool_destroy(pool);

  CHECK(strlen(tg_strerror(TG_ENOMEM)) > 0);
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("host ABI from C: all checks passed\n");
  return failures ? 1 : 0;
}
