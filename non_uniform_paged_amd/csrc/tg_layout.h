#ifndef TG_LAYOUT_H_
#define TG_LAYOUT_H_
// Byte strides of a cache's page pools (host code).  A page of cluster c
// holds one slot of head_bytes for each head of the cluster (include/tg.h).
// Page-major pools (tg_cache.head_major[c][t] 0) keep a page's slots side by side:
// page p, slot s at p * page_bytes + s * head_bytes.  Head-major pools give
// each slot its own run of pages: slot s, page p at (s * n_pages + p) *
// head_bytes, so that consecutive pages of one head are adjacent in memory.

#include <cstdint>

#include "tg.h"

namespace tg_dev {

// Bytes of one head's slot in a page of tier t.
inline int64_t head_slot_bytes(const tg_cache* c, int t) {
  const int64_t d = c->head_dim;
  if (t == TG_TIER_BF16) return 4 * static_cast<int64_t>(c->page_size) * d;
  const int64_t bits = c->old_bits == 4 ? 4 : 8;
  return 2 * static_cast<int64_t>(c->quant_block) * d * bits / 8 + 4 * d;
}

// Strides of pool (cl, t): between page ids and between the head slots of
// one page.
inline void pool_strides(const tg_cache* c, int cl, int t, int64_t* page_stride, int64_t* head_stride) {
  const int64_t hb = head_slot_bytes(c, t);
  const bool hm = c->head_major[cl][t] != 0;
  *page_stride = hm ? hb : c->page_bytes[cl][t];
  *head_stride = hm ? hb * c->n_pages[cl][t] : hb;
}

// Every layout flag of the cache's clusters is 0 or 1.
inline bool layout_flags_valid(const tg_cache* c) {
  for (int32_t cl = 0; cl < c->n_clusters && cl < TG_MAX_CLUSTERS; ++cl)
    for (int t = 0; t < 2; ++t)
      if (c->head_major[cl][t] != 0 && c->head_major[cl][t] != 1) return false;
  return true;
}

}  // namespace tg_dev

#endif  // TG_LAYOUT_H_
