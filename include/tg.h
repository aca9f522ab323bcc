/*
 * tg.h -- C ABI of the ragged-paged decode-attention library (gfx950).
 *
 * One decode step of one layer attends, for every request r and q-head hq,
 * over the rows that KV-head h = hq / G of r retains:
 *
 *     o[r][hq] = sum_t softmax_t(q[r][hq] . K_rh[t] * scale) V_rh[t]
 *
 * (TTKV page, "What real problem": each new token attends over all cached KV
 * states.)  The cache is shaped by three ideas from the pages:
 *
 *   - Budget Reservation (Tangram page, "Three mechanisms", item 1): every
 *     (request, KV-head) gets a fixed retained-token footprint at admission,
 *     from an input-invariant head ranking and a narrow per-head ratio band
 *     (Tangram page, "Key finding: two-level structural law").
 *   - Ragged Paging (same section, item 2): heads with similar budgets form a
 *     cluster with its own page pool and block table; a page holds the same
 *     token slots for every head of its cluster, so page size varies by
 *     cluster.
 *   - Recency tiers (TTKV page, "Tier Layout", "Tier Content", "Tier
 *     Interaction"): the newest share of each sequence stays bf16; older rows
 *     sit in 64-token blocks quantised to INT8 with per-channel scales.
 *   Shared-prefix pages (RadixAttention lesson, "The concept") are
 *   reference-counted and appear in many block tables.
 *
 * Conventions
 *   - Every call returns an int status (TG_OK or a negative TG_E* code) and
 *     never throws.  On error, outputs are unspecified and pool state is
 *     unchanged.
 *   - The caller owns every buffer.  Host outputs go to caller-allocated
 *     arrays whose sizes come from a sizing call.  Device memory (pools,
 *     tables, q, out, workspace) is allocated by the caller; the library never
 *     allocates device memory.
 *   - "device" pointers are HIP device pointers on the current device;
 *     "host" pointers are ordinary host memory.  `stream` is a hipStream_t
 *     (NULL = the default stream); device work is enqueued asynchronously and
 *     faults surface at the caller's next synchronisation.
 *   - Host functions are deterministic and not thread-safe per pool.
 *
 * Index conventions: B requests, H KV-heads, Hq = G*H q-heads with q-head hq
 * reading KV-head hq / G; tier 0 = INT8 (TG_TIER_I8), tier 1 = bf16
 * (TG_TIER_BF16); logical rows of (r, h) run oldest first, rows
 * [0, n_i8) in the INT8 tier and [n_i8, L) in the bf16 tier.
 */
#ifndef TG_H_
#define TG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_OK 0
#define TG_EINVAL (-1)       /* malformed argument or inconsistent sizes */
#define TG_ENOMEM (-2)       /* a page pool is exhausted (nothing changed) */
#define TG_EOVERFLOW (-3)    /* a size does not fit its integer type */
#define TG_EDEVICE (-4)      /* a HIP launch or runtime call failed */
#define TG_EUNSUPPORTED (-5) /* shape the device kernels do not implement */

#define TG_TIER_I8 0
#define TG_TIER_BF16 1
#define TG_MAX_CLUSTERS 16
#define TG_GROUP_WIDTH 32  /* member entries per group item of the plan */

#define TG_Q_F32 0
#define TG_Q_BF16 1

/* Human-readable text for a status code (static storage). */
const char* tg_strerror(int status);

/* ------------------------------------------------------------------------
 * Admission: budget reservation, clustering, tier split  (host only)
 *
 * Tangram page, "Key finding" and "Three mechanisms" items 1-2; TTKV page,
 * "Tier Content".  Rules (exact integers, 64-bit intermediates):
 *   ratio(k) = hi - floor((hi - lo) * k / (H - 1))   (k = rank, 0 = most
 *              important; hi when H == 1)
 *   budget   = clamp(ceil(ratio(rank[h]) * n_comp[r] / 1e6), 1, n_comp[r]),
 *              or budget_override[r*H + h] when given
 *   L        = n_fixed[r] + budget
 *   clusters = heads sorted by rank, cut into n_clusters contiguous groups,
 *              group c holding ceil(H/C) heads if c < H mod C else floor(H/C);
 *              slot_in_cluster = position inside the group in rank order
 *   n_bf0    = ceil(L * recent_ppm / 1e6);  n_i8 = floor((L - n_bf0) / Qb) * Qb;
 *   n_bf     = L - n_i8
 * ---------------------------------------------------------------------- */
typedef struct tg_budget_table {
  int32_t n_kv_heads;        /* H >= 1 */
  const int32_t* head_rank;  /* host [H]: a permutation of 0..H-1 */
  int32_t ratio_hi_ppm;      /* ratio of rank 0, in parts per million */
  int32_t ratio_lo_ppm;      /* ratio of rank H-1; 0 < lo <= hi <= 1e6 */
  int32_t n_clusters;        /* 1 <= C <= min(H, TG_MAX_CLUSTERS) */
  int32_t recent_ppm;        /* share kept bf16, 0..1e6 (1e6 = no INT8 tier) */
  int32_t quant_block;       /* INT8 block length Qb >= 1 (tokens) */
} tg_budget_table;

typedef struct tg_reservation {
  int32_t B, n_kv_heads, n_clusters; /* written by tg_reserve */
  int32_t* budget;           /* host [B*H] retained compressible tokens */
  int32_t* length;           /* host [B*H] L = n_fixed + budget */
  int32_t* n_i8;             /* host [B*H] rows in the INT8 tier */
  int32_t* n_bf;             /* host [B*H] rows in the bf16 tier */
  int32_t* cluster_of_head;  /* host [H] */
  int32_t* slot_in_cluster;  /* host [H] */
  int32_t* cluster_size;     /* host [C] */
  int32_t recent_ppm, quant_block; /* written by tg_reserve: the tier rule */
} tg_reservation;

/* Fill `out` (all arrays caller-allocated, sizes as listed).  n_comp [B]
 * (>= 1) are the compressible tokens of each request, n_fixed [B] (>= 0,
 * nullable = all 0) the always-kept shared-path tokens, budget_override
 * [B*H] (nullable) explicit budgets in [1, n_comp[r]].  TG_EINVAL on a
 * malformed table or length, TG_EOVERFLOW if L exceeds int32. */
int tg_reserve(const tg_budget_table* table, int32_t B, const int32_t* n_comp,
               const int32_t* n_fixed, const int32_t* budget_override,
               tg_reservation* out);

/* ------------------------------------------------------------------------
 * Page pools  (host bookkeeping; the bytes live in caller device memory)
 *
 * Ragged Paging (Tangram page, "Three mechanisms", item 2): one pool per
 * (cluster, tier).  A page of cluster c holds S token slots for each of its
 * n_c heads, S = page_size (bf16) or quant_block (INT8).  Each head slot of
 * a page (s = slot_in_cluster) is head_bytes laid out as below; where the
 * slots sit in the pool (page-major: s * head_bytes into the page;
 * head-major: one run of pages per slot) is tg_cache.head_major:
 *   bf16 : K block then V block, 2*S*d bytes each      head_bytes = 4*S*d
 *          (S = 16; element (row t, channel c) at byte
 *           K: ((c>>5)*64 + ((c>>3)&3)*16 + t)*16 + (c&7)*2
 *           V: ((c>>5)*64 + (t>>2)*16 + (c&15))*16 + ((c>>4)&1)*8 + (t&3)*2,
 *           so that each contiguous 1 KiB is one matrix-core operand)
 *   INT8 : K codes, V codes (S*d int8 each), then     head_bytes = 2*S*d + 4*d
 *          K scales [d] fp16, V scales [d] fp16
 *          (S = 64; code of (row t, channel c) at byte
 *           K: ((t>>4)*(d/64) + (c>>6))*1024 + (((c>>3)&3)*16 + (t&15))*16
 *              + ((c>>5)&1)*8 + (c&7)
 *           V: S*d + ((t>>4)*(d/64) + (c>>6))*1024 + (((t>>2)&3)*16 + (c&15))*16
 *              + ((c>>4)&3)*4 + (t&3))
 *   INT4 : (old_bits 4, d = 128) K codes, V codes     head_bytes = S*d + 4*d
 *          (S*d/2 bytes each; a code is u = q4 + 8 in 4 bits), then K
 *          scales [d] fp16, V scales [d] fp16.  In 32-bit words of a block,
 *          nibble p of a word being bits 4p..4p+3:
 *           K (t, c): word (((t>>4)*64 + (t&15) + 16*((c>>3)&3))*4 + (c>>5)),
 *                     nibble ((c&1)<<2) | ((c&7)>>1)
 *           V (t, c): at +S*d/2, word (((t>>4)*64 + (c&15) + 16*((t>>2)&3))*4
 *                     + (c>>5)), nibble ((t&1)<<2) | (((c>>4)&1)<<1) | ((t&3)>>1)
 * Pages are handed out lowest free id first; shared pages are
 * reference-counted; a failing allocation changes nothing.
 * ---------------------------------------------------------------------- */
typedef struct tg_pool tg_pool;

/* cluster_size [C] from tg_reserve; pages_bf / pages_i8 [C] capacities (>= 0);
 * old_bits 8 (INT8 pages) or 4 (INT4 pages) sizes the slow tier's pages.
 * TG_EINVAL on bad geometry, TG_EOVERFLOW if a pool's byte size overflows. */
int tg_pool_create(int32_t n_clusters, const int32_t* cluster_size, int32_t head_dim,
                   int32_t page_size, int32_t quant_block, int32_t old_bits, const int64_t* pages_bf,
                   const int64_t* pages_i8, tg_pool** out);
void tg_pool_destroy(tg_pool* pool);
/* Bytes of one page of (cluster c, tier), or -1 on a bad index. */
int64_t tg_pool_page_bytes(const tg_pool* pool, int32_t c, int32_t tier);
/* Capacity in pages, and pages currently free, of (c, tier); -1 on a bad index. */
int64_t tg_pool_capacity(const tg_pool* pool, int32_t c, int32_t tier);
int64_t tg_pool_free_pages(const tg_pool* pool, int32_t c, int32_t tier);
/* Reference count of page `page` of (c, tier); -1 on a bad index. */
int32_t tg_pool_refcount(const tg_pool* pool, int32_t c, int32_t tier, int64_t page);

/* ------------------------------------------------------------------------
 * Block tables and the ahead-of-time split plan  (host only)
 *
 * Tangram page, "Three mechanisms", items 2-3 (per-cluster tables; work
 * partitioned ahead of time, no per-step re-planning); RadixAttention lesson,
 * "The concept" (nodes own token ranges and their KV blocks; requests on a
 * branch reuse them).
 *
 *   pages   row r of (c, t) needs ceil(max_{h in c} n_bf / page_size) bf16 or
 *           max_{h in c} n_i8 / Qb INT8 pages, allocated in order r, c,
 *           t (INT8 then bf16), page j.
 *   sharing page j is shared when every head of c starts it at the same
 *           logical row s and s + S <= n_fixed[r]; its key is (c, t, node
 *           holding row s + S - 1, s).  A known key adds a reference; a new
 *           one takes a fresh page.  Other pages are always fresh.
 *   tables  bt[c][t] is [B][stride[c][t]] int32 page ids in logical order,
 *           padded with -1; stride = max_r pages; len [B*H*2] = (n_i8, n_bf).
 *   plan    items {r, h, tier, t0, t1, slot} for r, h, tier (INT8 first);
 *           t0, t1 are row indices inside the tier.  A range of u units
 *           (pages, or INT8 blocks; the last may be partial) becomes
 *           k = ceil(u / (chunk / unit)) near-equal items, item i starting at
 *           unit floor(i * u / k).  slot = index of the item's partial;
 *           part_off [B*H + 1] = first slot of each (r, h).  With lpt != 0 the
 *           items are stably sorted by descending (t1 - t0) * w, w in
 *           proportion to a row's HBM bytes: 16 qb for bf16, old_bits * qb + 16
 *           for the quantised tier (old_bits of the pool); group items stay
 *           ahead of the others.  The split kernel runs each of the leading
 *           n_gitems entries on a whole workgroup (four wavefronts sharing the
 *           page loads); a plan in another order still decodes correctly,
 *           more slowly.
 *   groups  with group_size > 1 and `share`, the leading shared bf16 pages of
 *           each (r, h) are cut into runs of one radix node; requests whose
 *           run has the same (node, first row, pages, n_i8) are taken in
 *           ascending r, group_size at a time, and each group's rows are
 *           split as above (chunk_group, or chunk_bf when it is 0) from the
 *           run's first row into group items
 *           {-1 - k, h, bf16, t0, t1, -1}: one pass over those pages for up
 *           to group_size requests.  gitems[k] lists its members as
 *           TG_GROUP_WIDTH (r, slot) pairs, padded with (-1, -1).  Group items
 *           come first (per h, runs in order of first appearance, groups,
 *           chunks); a request's own bf16 items start after its shared rows.
 *           Slots of each (r, h): its group memberships in group-item order,
 *           then its own items in the order above.
 *   growth  with gen_tokens = T > 0 (TTKV page, "Tier Content" / "Tier
 *           Interaction": recent rows stay bf16, older ones are quantised in
 *           blocks), each (r, h) may gain T rows by tg_append_kv.  An
 *           appended row becomes the newest bf16 row and the tier split above
 *           is applied to the new length; when the INT8 boundary moves (one
 *           block) the oldest Qb bf16 rows become the next INT8 block.  Pages
 *           are reserved now for the largest sizes on the way (INT8 rows of
 *           L + T, the most bf16 rows at any length from L to L + T), and the
 *           plan covers those capacities with as many items per range as the
 *           live rows give (k = ceil(u_live / c) for u_live units of chunk c
 *           units), more only where items would pass 2 c units (k =
 *           ceil(u / 2c)); the decode kernels clip every item to the live
 *           lengths.  The bf16 tier turns over its ring[r][c]
 *           pages (logical bf16 row j of (r, h) lives at ring row
 *           (bf_base[r][h] + j) mod (16 ring[r][c])).
 * ---------------------------------------------------------------------- */
typedef struct tg_share_desc {
  const int32_t* n_nodes;   /* host [B] radix-path length of each request */
  const int32_t* node_ids;  /* host [sum n_nodes] paths, root first */
  int32_t n_node_table;     /* number of distinct node ids */
  const int32_t* node_len;  /* host [n_node_table] tokens owned by each node */
} tg_share_desc;            /* sum of node_len over r's path must be n_fixed[r] */

typedef struct tg_plan_opts {
  int32_t chunk_bf;  /* bf16 item length, a positive multiple of page_size */
  int32_t chunk_i8;  /* INT8 item length, a positive multiple of quant_block */
  int32_t lpt;       /* nonzero: longest items first */
  int32_t group_size; /* 0 or 1: no group items; at most TG_GROUP_WIDTH (a
                         workgroup scores 128 / G members a pass over the
                         pages, so 128 / G or less is one pass) */
  int32_t gen_tokens; /* >= 0: rows each (r, h) may still gain by tg_append_kv
                         (see growth below); 0 with `share` only */
  int32_t chunk_group; /* group item length in rows, a multiple of page_size;
                          0: chunk_bf */
} tg_plan_opts;

typedef struct tg_table_sizes {
  int32_t stride[TG_MAX_CLUSTERS][2];        /* entries per table row */
  int32_t n_items;                           /* plan length */
  int32_t n_gitems;                          /* group items */
  int32_t n_slots;                           /* partials = part_off[B*H] */
  int64_t pages_needed[TG_MAX_CLUSTERS][2];  /* from an empty pool */
} tg_table_sizes;

/* Sizes of the arrays tg_build_tables fills; touches no pool.  `share` is
 * nullable.  TG_EINVAL on malformed input, TG_EOVERFLOW on int32 overflow. */
int tg_size_tables(const tg_reservation* res, int32_t page_size, int32_t quant_block,
                   const tg_share_desc* share, const tg_plan_opts* opts,
                   tg_table_sizes* out);

typedef struct tg_tables {
  int32_t* bt[TG_MAX_CLUSTERS][2];     /* host [B][stride[c][t]] (may be NULL if stride 0) */
  int32_t stride[TG_MAX_CLUSTERS][2];  /* in: must equal tg_size_tables' values */
  int32_t* len;                        /* host [B*H*2] */
  int32_t* work;                       /* host [n_items*6] */
  int32_t n_items;                     /* in: must equal tg_size_tables' value */
  int32_t* part_off;                   /* host [B*H + 1] */
  int32_t* released;                   /* host [B] zeroed here; set by tg_release */
  int32_t* gitems;                     /* host [n_gitems][TG_GROUP_WIDTH][2] (may be NULL if 0) */
  int32_t n_gitems;                    /* in: must equal tg_size_tables' value */
  int32_t* ring;                       /* host [B][C]: bf16 pages of (r, c) (nullable) */
  int32_t B;                           /* out: requests the tables hold (written by
                                          tg_build_tables; tg_release refuses r outside
                                          [0, B)) */
} tg_tables;

/* Allocate every page of the batch from `pool` (all or nothing) and fill the
 * tables.  TG_ENOMEM leaves the pool unchanged. */
int tg_build_tables(tg_pool* pool, const tg_reservation* res, const tg_share_desc* share,
                    const tg_plan_opts* opts, tg_tables* out);

/* Consistency check of tables against the reservation and the pool they
 * were built from (host; a debugging aid for tables that were edited, copied
 * or made elsewhere before they go to the device).  Released requests are
 * skipped.  Checks, in this order:
 *   - block tables: each row lists page ids in [0, capacity) of its
 *     (cluster, tier) pool, then -1 only; no page appears in more rows than
 *     its reference count;
 *   - lengths: n_i8 a multiple of Qb, n_i8 <= (INT8 pages of the row) * Qb,
 *     n_bf <= (bf16 pages, or ring pages when `ring` is set) * page_size;
 *   - slots: part_off starts at 0 and never decreases; every item's slot (and
 *     every group member's) lies in its (r, h)'s range and each slot is used
 *     exactly once;
 *   - plan items: a valid head and tier, 0 <= t0 < t1 within the rows the
 *     pages hold; group items bf16, listed once, members in ascending request
 *     order then (-1, -1) padding, every member's pages over the item's rows
 *     the very pages of its first member;
 *   - cover: the items of each (r, h, tier) tile rows 0, 1, ... once each, up
 *     to at least the live length.
 * Returns TG_OK, or TG_EINVAL with a description of the first failed check
 * written to msg (nullable; msg_bytes including the terminating zero);
 * TG_ENOMEM if the check's own bookkeeping cannot be allocated. */
int tg_check_tables(const tg_pool* pool, const tg_reservation* res, const tg_tables* tables, char* msg,
                    size_t msg_bytes);

/* Drop request r's page references; pages reaching zero become free and their
 * share keys are forgotten.  TG_EINVAL if r is outside [0, tables->B), if r
 * was already released, or if a page of r's rows is not live in `pool`
 * (nothing changes then). */
int tg_release(tg_pool* pool, tg_tables* tables, int32_t r);

/* ------------------------------------------------------------------------
 * Device view of a populated cache  (all pointers device, except the struct)
 * ---------------------------------------------------------------------- */
typedef struct tg_cache {
  int32_t B, n_kv_heads, head_dim, page_size, quant_block, n_clusters;
  void* pool[TG_MAX_CLUSTERS][2];            /* pool base of (c, t), 16-byte aligned */
  int64_t page_bytes[TG_MAX_CLUSTERS][2];    /* from tg_pool_page_bytes */
  int64_t n_pages[TG_MAX_CLUSTERS][2];       /* pool capacities */
  const int32_t* bt[TG_MAX_CLUSTERS][2];     /* device [B][stride[c][t]] */
  int32_t stride[TG_MAX_CLUSTERS][2];
  const int32_t* cluster_of_head;            /* device [H] */
  const int32_t* slot_in_cluster;            /* device [H] */
  int32_t* len;                              /* device [B*H*2] live (n_i8, n_bf); updated by
                                                tg_append_kv */
  const int32_t* n_fixed;                    /* device [B] shared-path rows of each request, or
                                                NULL when nothing is shared; rows on the
                                                shared path are read through the caches, all
                                                other rows with streaming (non-temporal) loads */
  const int32_t* ring;                       /* device [B*C] bf16 ring pages (tg_tables.ring),
                                                or NULL: no ring (bf_base unused) */
  int32_t* bf_base;                          /* device [B*H] ring row of logical bf16 row 0
                                                (zero at admission; updated by tg_append_kv) */
  int32_t recent_ppm;                        /* tier rule of the reservation (tg_append_kv) */
  int32_t old_bits;                          /* slow-tier codes: 8 (0 = 8) or 4 (d = 128 only) */
  int32_t head_major[TG_MAX_CLUSTERS][2];   /* layout of pool (c, t), see below: 0 page-major,
                                                1 head-major (0 for an INT8 pool in host memory) */
} tg_cache;

/* Pool layouts.  A page of cluster c holds one slot of head_bytes (the page
 * layouts above) for each of the n_c heads of the cluster, so page_bytes =
 * n_c * head_bytes and a pool of n_pages pages has n_pages * page_bytes bytes
 * either way; the layout only decides where the slots sit:
 *   page-major (0): page p, slot s at p * page_bytes + s * head_bytes (a
 *                   page is contiguous);
 *   head-major (1): slot s, page p at (s * n_pages + p) * head_bytes (the
 *                   pages of one head slot are contiguous: a sequence's
 *                   pages, allocated in order, read as one run per head).
 * Page ids, tables and plans are the same for both, and so is every output
 * bit.  (Head-major slots a large power of two apart, n_pages * head_bytes
 * = 2^k, read measurably slower on MI355X: pad n_pages.)  tg_write_kv, tg_append_kv and tg_decode_* follow the flag of each
 * pool; tg_decode_streamed requires page-major INT8 pools (it copies whole
 * pages) and returns TG_EUNSUPPORTED otherwise. */

/* ------------------------------------------------------------------------
 * Cache fill  (device)
 *
 * Writes logical rows into their pages: row i of (r, h) is
 * rows[index[offsets[r*H + h] + i]] ([2][d] bf16 bits: K then V).  Rows
 * [0, n_i8) are quantised per 64-token block and channel (TTKV page, "Tier
 * Layout" / "Tier Interaction"; symmetric absmax reading):
 *   s  = fp16_rne(fp32(absmax) / 127), +inf saturating to 65504
 *   q8 = s > 0 ? clamp(rint_even(x / s), -127, 127) : 0       (fp32 math)
 * Shared pages may be written by several sequences with identical data.
 * rows: device uint16 [n_rows][2][d]; index: device int32 [offsets[B*H]];
 * offsets: device int64 [B*H + 1].  TG_EINVAL on a bad shape; TG_EOVERFLOW
 * if B*H exceeds int32 (any B*H below that is one launch per tier: the grid
 * strides over pairs past the 65535 workgroups of one grid dimension).
 * ---------------------------------------------------------------------- */
int tg_write_kv(const tg_cache* cache, const uint16_t* rows, const int32_t* index,
                const int64_t* offsets, void* stream);

/* ------------------------------------------------------------------------
 * Decode-step append and tier ageing  (device)
 *
 * For every (r, h): the new row rows[r*H + h] ([2][d] bf16 bits: K then V;
 * device uint16 [B*H][2][d]) is written in place as the newest bf16 row, in
 * the page reserved for it (ring row (bf_base + n_bf) mod 16 ring[r][c]).
 * Then the tier split is applied to the new length (TTKV page, "Tier
 * Content": the newest share stays bf16; "Tier Interaction": older rows are
 * quantised block by block): when it moves the INT8 boundary, the oldest Qb
 * bf16 rows are quantised as in tg_write_kv into INT8 block n_i8 / Qb, and
 * the ring advances by Qb rows.  cache->len and cache->bf_base are updated
 * on the device.  The cache must come from tables built with gen_tokens > 0
 * (cache->ring, cache->bf_base set).  A (r, h) whose step would pass the
 * capacity reserved at admission is left unchanged and sets bit 0 of
 * *status (device int32, nullable).  TG_EINVAL on a malformed cache.
 * ---------------------------------------------------------------------- */
int tg_append_kv(const tg_cache* cache, const uint16_t* rows, int32_t* status, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention  (device)
 *
 * Split-K over the plan: each item (r, h, tier, t0, t1) computes, for the G
 * q-heads of h, the partial (m, l, acc) of the online normaliser (CAP survey
 * page, section 2.4.3, online normaliser [88]): m = max score, l = sum
 * exp(s - m), acc = sum exp(s - m) v, with INT8 rows dequantised in
 * registers.  A second kernel merges the partials of each (r, h):
 *   o = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s,  M = max_s m_s.
 *
 *   q         device [B][Hq][d], fp32 (TG_Q_F32) or bf16 bits (TG_Q_BF16)
 *   work, part_off, gitems, n_items, n_gitems  device copies of
 *             tg_build_tables' plan; n_slots = part_off[B*H]
 *   workspace device fp32, >= tg_decode_workspace_bytes(n_slots, G, d) bytes:
 *             acc [n_slots][G][d] then (m, l) [n_slots][G][2] (m in natural
 *             log units of the scaled score)
 *   out       device fp32 [B][Hq][d]
 *   sm_scale  score scale, finite and >= 0; 0 means 1/sqrt(d)
 * TG_EUNSUPPORTED unless d in {64, 128}, G in {1, 2, 4, 8}, page_size 16 and
 * quant_block 64; TG_EINVAL on inconsistent arguments; TG_EDEVICE on a
 * failed launch.  A group item computes the partials of all its members (G
 * score columns each); a leading group item runs on a whole workgroup, 128 /
 * G members (64 / G for G = 8 with fp32 q) per pass over its pages.
 * ---------------------------------------------------------------------- */
size_t tg_decode_workspace_bytes(int32_t n_slots, int32_t G, int32_t d);

typedef struct tg_decode_args {
  int32_t n_q_heads;
  int32_t q_dtype;
  const void* q;
  const int32_t* work;
  int32_t n_items;
  const int32_t* part_off;
  float* workspace;
  size_t workspace_bytes;
  float* out;
  float sm_scale;
  const int32_t* gitems;  /* device [n_gitems][TG_GROUP_WIDTH][2], or NULL if n_gitems 0 */
  int32_t n_gitems;
  int32_t n_slots;
} tg_decode_args;

int tg_decode_attn(const tg_cache* cache, const tg_decode_args* args, void* stream);

/* tg_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the partials go to a fixed device array of the library instead of
 * args->workspace (ignored, as is args->workspace_bytes).  The array holds
 * TG_NOALLOC_SCRATCH_BYTES on each device the library runs on, from the
 * device's first call until the process ends; the call itself allocates
 * nothing.  Every call on one device shares that device's array, so calls
 * that overlap in time on one device (on different streams) race; calls on
 * one stream are ordered.  Nothing in the array needs to start at zero.
 * TG_EOVERFLOW when tg_decode_workspace_bytes(n_slots, G, d) exceeds
 * TG_NOALLOC_SCRATCH_BYTES (nothing is launched); otherwise the errors of
 * tg_decode_attn, and TG_EDEVICE if the array's address cannot be taken. */
#define TG_NOALLOC_SCRATCH_BYTES (32u << 20)
int tg_decode_attn_noalloc(const tg_cache* cache, const tg_decode_args* args, void* stream);

/* Split stage alone: writes the partials of every plan item into
 * `workspace` (layout above) without merging them; `out` is not used.
 * tg_decode_attn == tg_decode_split followed by tg_merge_partials over the
 * B*H pairs of `part_off`.  Same errors as tg_decode_attn. */
int tg_decode_split(const tg_cache* cache, const tg_decode_args* args, void* stream);

/* Measurement aid: tg_decode_split with the split kernel's own start and end
 * recorded into start_event and stop_event (hipEvent_t, created by the
 * caller with timing enabled), so that their elapsed time is the kernel's
 * execution without the dispatch latency that a separately recorded event
 * adds.  A plan with no items launches nothing and records neither event.
 * TG_EINVAL on a null event; otherwise the errors of tg_decode_split. */
int tg_decode_split_timed(const tg_cache* cache, const tg_decode_args* args, void* start_event, void* stop_event,
                          void* stream);

/* Merge stage alone (also the merge of partials computed on different
 * shards).  For each pair p in [0, n_pairs) and g < G, merges slots
 * [part_off[p], part_off[p+1]) of `workspace` (layout as above, n_slots
 * slots) into out[p*G + g][d].  Pairs with no slot are written as 0. */
int tg_merge_partials(const float* workspace, int32_t n_slots, int32_t n_pairs, int32_t G,
                      int32_t d, const int32_t* part_off, float* out, void* stream);

/* ------------------------------------------------------------------------
 * INT8 tier in host DRAM, streamed per step  (host orchestration + device)
 *
 * TTKV page, "Tier Layout" (the slow tier sits in DRAM) and its block-wise
 * streaming of the slow tier: cache->pool[c][TG_TIER_I8] are host pointers
 * to pinned memory (e.g. hipHostMalloc) holding the INT8 pages; everything
 * else is as for tg_decode_attn.  Per call, the bf16 items run first on
 * `stream`; then, request by request, the INT8 pages of request r are copied
 * (hipMemcpyAsync on the library's own copy stream, one copy per run of
 * consecutive page ids) into staging slot r mod 2 while the kernels of
 * request r - 1 run, and the INT8 items of r run on `stream` once their copy
 * is done; the merge follows.  The results are those of tg_decode_attn bit
 * for bit.
 *
 *   tables     host tables of the cache (the INT8 block table rows name the
 *              pages to copy)
 *   args.work  the plan reordered by tg_stream_order (device copy);
 *   chunk_off  host [B + 1] from tg_stream_order
 *   staging    device, 256-byte aligned, >= tg_stream_staging_bytes bytes
 * The library creates one copy stream and its events per device, on the
 * device's first call, and keeps them until the process ends: calls on one
 * device must not overlap in time; calls on different devices may.  Errors
 * as tg_decode_attn; TG_EINVAL on a bad chunk_off or staging size. */
size_t tg_stream_staging_bytes(const tg_cache* cache, const tg_tables* tables);
int tg_decode_streamed(const tg_cache* cache, const tg_tables* tables, const tg_decode_args* args,
                       const int32_t* chunk_off, void* staging, size_t staging_bytes, void* stream);
/* Plan order for tg_decode_streamed (host): bf16 and group items first, in
 * plan order, then the INT8 items of request 0, 1, ... (plan order within a
 * request).  work_out [n_items*6]; chunk_off [B + 1]: chunk_off[0] = number
 * of bf16 items, request r's INT8 items are [chunk_off[r], chunk_off[r+1]).
 * TG_EINVAL on a malformed plan. */
int tg_stream_order(const tg_tables* tables, int32_t B, int32_t* work_out, int32_t* chunk_off);

/* ------------------------------------------------------------------------
 * Lossless bf16 exponent codec  (device)
 *
 * SplitZip page ("Die SplitZip-Strategie"): the 16 most frequent exponents
 * of the input get 4-bit codes, two per byte; sign and mantissa take one
 * byte per value; values with another exponent are listed in an escape
 * stream that decoding writes over its first result.  Codebook: exponents by
 * count descending, ties to the smaller exponent.  Compressed buffer (n a
 * multiple of 8, little endian):
 *   [0, 8) n (int64), [8, 16) n_esc (int64), [16, 32) codebook (uint8, rank
 *   order), [32, 256) zero, [256, 256 + n) sign << 7 | mantissa per value,
 *   [256 + n, 256 + 3n/2) codes (value i in bits 4(i%2).. of byte i/2, an
 *   escaped value's code is 0), then n_esc uint32 escape positions
 *   (ascending) and n_esc uint8 escape exponents.
 *   Size 256 + 3n/2 + 5 n_esc (read n_esc from the header).
 * src, dst, workspace: device, 16-byte aligned; dst of tg_zip_bound(n) bytes,
 * workspace of tg_zip_workspace_bytes(n).  TG_EINVAL on a bad size or
 * pointer; n <= 2^32.
 * ---------------------------------------------------------------------- */
size_t tg_zip_bound(int64_t n);
size_t tg_zip_workspace_bytes(int64_t n);
int tg_zip_encode(const uint16_t* src, int64_t n, void* dst, size_t dst_bytes, void* workspace,
                  size_t workspace_bytes, void* stream);
int tg_zip_decode(const void* src, int64_t n, uint16_t* dst, void* stream);

/* ------------------------------------------------------------------------
 * Measurement aid  (device)
 *
 * Streaming read of `bytes` (a multiple of 16) at `src` (16-byte aligned
 * device memory) with non-temporal loads over TG_BENCH_READ_BLOCKS
 * workgroups sweeping the buffer together (pass k of workgroup b reads the
 * 16 KiB tile k * TG_BENCH_READ_BLOCKS + b); each writes one fold of what it
 * read to sink[block] (device
 * uint32 [TG_BENCH_READ_BLOCKS]) so that no load is elided.  Timing it gives
 * the device's achievable read rate.  start_event, stop_event: null, or
 * hipEvent_t that receive the kernel's own start and end.  TG_EINVAL on a
 * bad size or pointer.
 * ---------------------------------------------------------------------- */
#define TG_BENCH_READ_BLOCKS 4096
int tg_bench_read(const void* src, size_t bytes, uint32_t* sink, void* start_event, void* stop_event, void* stream);

/* Streaming read in the decode split kernels' own access pattern: n_streams
 * independent streams, one wavefront each (four to a workgroup), stream w
 * reading the 8 KiB chunks chunk[off[w]] .. chunk[off[w + 1] - 1] of `src`
 * (chunk c = bytes [8192 c, 8192 c + 8192)) in list order, in 1 KiB wave
 * loads with two chunks in flight, non-temporal -- as a decode item reads its
 * pages.  Chunk ids are taken modulo bytes / 8192, so any list stays inside
 * `src`.  sink[w] (device uint32 [n_streams]) receives the XOR of every
 * 32-bit word stream w read (a chunk listed twice cancels).  Timing it over
 * the chunk counts of a plan gives the rate that pattern allows, with no
 * arithmetic.  src: 16-byte aligned device memory, `bytes` a positive
 * multiple of 8192; chunk, off (n_streams + 1 entries, non-decreasing):
 * device int32.  start_event, stop_event: as for tg_bench_read.  TG_EINVAL
 * on a bad size or pointer; TG_EDEVICE on a failed launch. */
int tg_bench_streams(const void* src, size_t bytes, const int32_t* chunk, const int32_t* off, int32_t n_streams,
                     uint32_t* sink, void* start_event, void* stop_event, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TG_H_ */
