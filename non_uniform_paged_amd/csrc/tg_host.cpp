// Host side of the C ABI: budget reservation, clustering, tier split, the
// ref-counted ragged page pools, block tables and the ahead-of-time split
// plan.  Pure C++17, no device calls.
//
// Sources: Tangram page (arXiv 2606.06302 explainer), "Key finding: two-level
// structural law" and "Three mechanisms" items 1-3 (Budget Reservation,
// Ragged Paging, AOT load balancing); TTKV page (arXiv 2604.19769 explainer),
// "Tier Content" (newest share stays high precision, the rest is quantised in
// blocks); RadixAttention lesson, "The concept" (radix nodes own token ranges
// and their KV blocks, reused by every request on the branch).  The exact
// integer rules are the ones documented in include/tg.h.

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <new>
#include <unordered_map>
#include <vector>

#include "tg.h"

namespace {

constexpr int64_t kPpm = 1000000;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct ShareKey {
  int32_t c, t, node;
  int64_t start;
  bool operator==(const ShareKey& o) const {
    return c == o.c && t == o.t && node == o.node && start == o.start;
  }
};
struct ShareKeyHash {
  size_t operator()(const ShareKey& k) const {
    uint64_t h = static_cast<uint64_t>(k.start) * 0x9E3779B97F4A7C15ull;
    h ^= (static_cast<uint64_t>(k.node) + 0x7F4A7C15ull) * 0xBF58476D1CE4E5B9ull;
    h ^= static_cast<uint64_t>(k.c * 2 + k.t) * 0x94D049BB133111EBull;
    return static_cast<size_t>(h ^ (h >> 31));
  }
};

// One (cluster, tier) pool: refcounts, plus a bitmap of free pages searched
// lowest-first.  `hint` is the lowest word that may hold a free bit.
struct SubPool {
  int64_t cap = 0;
  int64_t page_bytes = 0;
  std::vector<int32_t> ref;
  std::vector<uint64_t> free_bits;  // bit set = page free
  int64_t hint = 0;
  int64_t n_free = 0;
  std::vector<ShareKey> key_of;     // valid where has_key
  std::vector<uint8_t> has_key;

  void init(int64_t capacity, int64_t bytes) {
    cap = capacity;
    page_bytes = bytes;
    ref.assign(static_cast<size_t>(cap), 0);
    free_bits.assign(static_cast<size_t>((cap + 63) / 64), ~0ull);
    if (cap % 64) free_bits.back() = (1ull << (cap % 64)) - 1;
    hint = 0;
    n_free = cap;
    key_of.assign(static_cast<size_t>(cap), ShareKey{0, 0, 0, 0});
    has_key.assign(static_cast<size_t>(cap), 0);
  }
  int64_t take_lowest() {
    const int64_t nw = static_cast<int64_t>(free_bits.size());
    for (int64_t w = hint; w < nw; ++w) {
      if (free_bits[w]) {
        hint = w;
        const int b = __builtin_ctzll(free_bits[w]);
        free_bits[w] &= ~(1ull << b);
        --n_free;
        const int64_t pid = w * 64 + b;
        ref[pid] = 1;
        return pid;
      }
    }
    hint = nw;
    return -1;
  }
  void give_back(int64_t pid) {
    free_bits[pid / 64] |= 1ull << (pid % 64);
    ++n_free;
    if (pid / 64 < hint) hint = pid / 64;
  }
};

}  // namespace

struct tg_pool {
  int32_t C = 0, d = 0, page_size = 0, quant_block = 0, old_bits = 8;
  std::vector<int32_t> cluster_size;
  SubPool sub[TG_MAX_CLUSTERS][2];
  std::unordered_map<ShareKey, int64_t, ShareKeyHash> registry;
};

extern "C" const char* tg_strerror(int status) {
  switch (status) {
    case TG_OK: return "ok";
    case TG_EINVAL: return "invalid argument";
    case TG_ENOMEM: return "page pool exhausted";
    case TG_EOVERFLOW: return "integer overflow";
    case TG_EDEVICE: return "device error";
    case TG_EUNSUPPORTED: return "unsupported shape";
    default: return "unknown status";
  }
}

// --------------------------------------------------------------------------
// reservation
// --------------------------------------------------------------------------
extern "C" int tg_reserve(const tg_budget_table* tb, int32_t B, const int32_t* n_comp,
                          const int32_t* n_fixed, const int32_t* override_b,
                          tg_reservation* out) {
  if (!tb || !out || !n_comp || !tb->head_rank || B < 1) return TG_EINVAL;
  const int32_t H = tb->n_kv_heads, C = tb->n_clusters;
  if (H < 1) return TG_EINVAL;
  if (!(0 < tb->ratio_lo_ppm && tb->ratio_lo_ppm <= tb->ratio_hi_ppm && tb->ratio_hi_ppm <= kPpm))
    return TG_EINVAL;
  if (C < 1 || C > H || C > TG_MAX_CLUSTERS) return TG_EINVAL;
  if (tb->recent_ppm < 0 || tb->recent_ppm > kPpm || tb->quant_block < 1) return TG_EINVAL;
  if (!out->budget || !out->length || !out->n_i8 || !out->n_bf || !out->cluster_of_head ||
      !out->slot_in_cluster || !out->cluster_size)
    return TG_EINVAL;
  std::vector<int32_t> head_at_rank(H, -1);
  for (int32_t h = 0; h < H; ++h) {
    const int32_t k = tb->head_rank[h];
    if (k < 0 || k >= H || head_at_rank[k] != -1) return TG_EINVAL;
    head_at_rank[k] = h;
  }
  for (int32_t r = 0; r < B; ++r) {
    if (n_comp[r] < 1) return TG_EINVAL;
    if (n_fixed && n_fixed[r] < 0) return TG_EINVAL;
    if (override_b)
      for (int32_t h = 0; h < H; ++h) {
        const int32_t b = override_b[int64_t(r) * H + h];
        if (b < 1 || b > n_comp[r]) return TG_EINVAL;
      }
  }
  // validate everything (including overflow) before writing any output
  for (int32_t r = 0; r < B; ++r) {
    const int64_t nf = n_fixed ? n_fixed[r] : 0;
    if (nf + n_comp[r] > std::numeric_limits<int32_t>::max()) return TG_EOVERFLOW;
  }
  const int64_t hi = tb->ratio_hi_ppm, lo = tb->ratio_lo_ppm;
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = n_comp[r];
    const int64_t nf = n_fixed ? n_fixed[r] : 0;
    for (int32_t h = 0; h < H; ++h) {
      const int64_t i = int64_t(r) * H + h;
      int64_t b;
      if (override_b) {
        b = override_b[i];
      } else {
        const int64_t k = tb->head_rank[h];
        const int64_t ratio = (H == 1) ? hi : hi - ((hi - lo) * k) / (H - 1);
        b = ceil_div(ratio * n, kPpm);
        b = std::min<int64_t>(std::max<int64_t>(b, 1), n);
      }
      const int64_t L = nf + b;
      const int64_t old = L - ceil_div(L * tb->recent_ppm, kPpm);
      const int64_t i8 = (old / tb->quant_block) * tb->quant_block;
      out->budget[i] = static_cast<int32_t>(b);
      out->length[i] = static_cast<int32_t>(L);
      out->n_i8[i] = static_cast<int32_t>(i8);
      out->n_bf[i] = static_cast<int32_t>(L - i8);
    }
  }
  int32_t k = 0;
  for (int32_t c = 0; c < C; ++c) {
    const int32_t sz = (c < H % C) ? (H + C - 1) / C : H / C;
    out->cluster_size[c] = sz;
    for (int32_t s = 0; s < sz; ++s, ++k) {
      out->cluster_of_head[head_at_rank[k]] = c;
      out->slot_in_cluster[head_at_rank[k]] = s;
    }
  }
  out->B = B;
  out->n_kv_heads = H;
  out->n_clusters = C;
  out->recent_ppm = tb->recent_ppm;
  out->quant_block = tb->quant_block;
  return TG_OK;
}

// --------------------------------------------------------------------------
// pools
// --------------------------------------------------------------------------
static int64_t head_bytes(int32_t tier, int32_t d, int32_t ps, int32_t qb, int32_t bits) {
  return tier == TG_TIER_BF16 ? int64_t(4) * ps * d : int64_t(2) * qb * d * bits / 8 + int64_t(4) * d;
}

extern "C" int tg_pool_create(int32_t C, const int32_t* cluster_size, int32_t d, int32_t ps,
                              int32_t qb, int32_t old_bits, const int64_t* pages_bf, const int64_t* pages_i8,
                              tg_pool** out) {
  if (!out || !cluster_size || !pages_bf || !pages_i8) return TG_EINVAL;
  if (C < 1 || C > TG_MAX_CLUSTERS || d < 1 || ps < 1 || qb < 1) return TG_EINVAL;
  if (old_bits != 8 && old_bits != 4) return TG_EINVAL;
  if (old_bits == 4 && qb % 2 && d % 2) return TG_EINVAL;  // two codes a byte: qb * d must be even
  for (int32_t c = 0; c < C; ++c)
    if (cluster_size[c] < 1 || pages_bf[c] < 0 || pages_i8[c] < 0) return TG_EINVAL;
  for (int32_t c = 0; c < C; ++c)
    for (int32_t t = 0; t < 2; ++t) {
      const int64_t pb = head_bytes(t, d, ps, qb, old_bits) * cluster_size[c];
      const int64_t cap = t == TG_TIER_BF16 ? pages_bf[c] : pages_i8[c];
      if (cap > 0 && pb > std::numeric_limits<int64_t>::max() / cap) return TG_EOVERFLOW;
    }
  tg_pool* p = new (std::nothrow) tg_pool;
  if (!p) return TG_ENOMEM;
  try {
    p->C = C;
    p->d = d;
    p->page_size = ps;
    p->quant_block = qb;
    p->old_bits = old_bits;
    p->cluster_size.assign(cluster_size, cluster_size + C);
    for (int32_t c = 0; c < C; ++c) {
      p->sub[c][TG_TIER_BF16].init(pages_bf[c], head_bytes(TG_TIER_BF16, d, ps, qb, old_bits) * cluster_size[c]);
      p->sub[c][TG_TIER_I8].init(pages_i8[c], head_bytes(TG_TIER_I8, d, ps, qb, old_bits) * cluster_size[c]);
    }
  } catch (...) {
    delete p;
    return TG_ENOMEM;
  }
  *out = p;
  return TG_OK;
}

extern "C" void tg_pool_destroy(tg_pool* p) { delete p; }

static bool bad_index(const tg_pool* p, int32_t c, int32_t t) {
  return !p || c < 0 || c >= p->C || (t != TG_TIER_I8 && t != TG_TIER_BF16);
}
extern "C" int64_t tg_pool_page_bytes(const tg_pool* p, int32_t c, int32_t t) {
  return bad_index(p, c, t) ? -1 : p->sub[c][t].page_bytes;
}
extern "C" int64_t tg_pool_capacity(const tg_pool* p, int32_t c, int32_t t) {
  return bad_index(p, c, t) ? -1 : p->sub[c][t].cap;
}
extern "C" int64_t tg_pool_free_pages(const tg_pool* p, int32_t c, int32_t t) {
  return bad_index(p, c, t) ? -1 : p->sub[c][t].n_free;
}
extern "C" int32_t tg_pool_refcount(const tg_pool* p, int32_t c, int32_t t, int64_t page) {
  if (bad_index(p, c, t) || page < 0 || page >= p->sub[c][t].cap) return -1;
  return p->sub[c][t].ref[page];
}

// --------------------------------------------------------------------------
// tables and plan
// --------------------------------------------------------------------------
namespace {

struct Geometry {
  int32_t B, H, C, ps, qb;
  std::vector<std::vector<int32_t>> heads;  // heads[c] in slot order
};

int check_reservation(const tg_reservation* res, int32_t ps, int32_t qb, Geometry* g) {
  if (!res || ps < 1 || qb < 1) return TG_EINVAL;
  if (res->B < 1 || res->n_kv_heads < 1 || res->n_clusters < 1 || res->n_clusters > TG_MAX_CLUSTERS)
    return TG_EINVAL;
  if (!res->length || !res->n_i8 || !res->n_bf || !res->cluster_of_head || !res->slot_in_cluster ||
      !res->cluster_size || !res->budget)
    return TG_EINVAL;
  g->B = res->B;
  g->H = res->n_kv_heads;
  g->C = res->n_clusters;
  g->ps = ps;
  g->qb = qb;
  g->heads.assign(g->C, {});
  for (int32_t c = 0; c < g->C; ++c) {
    if (res->cluster_size[c] < 1) return TG_EINVAL;
    g->heads[c].assign(res->cluster_size[c], -1);
  }
  for (int32_t h = 0; h < g->H; ++h) {
    const int32_t c = res->cluster_of_head[h], s = res->slot_in_cluster[h];
    if (c < 0 || c >= g->C || s < 0 || s >= res->cluster_size[c] || g->heads[c][s] != -1)
      return TG_EINVAL;
    g->heads[c][s] = h;
  }
  for (int32_t c = 0; c < g->C; ++c)
    for (int32_t h : g->heads[c])
      if (h < 0) return TG_EINVAL;
  for (int64_t i = 0; i < int64_t(g->B) * g->H; ++i) {
    if (res->n_i8[i] < 0 || res->n_bf[i] < 0 || res->n_i8[i] % qb) return TG_EINVAL;
    if (int64_t(res->n_i8[i]) + res->n_bf[i] != res->length[i] || res->length[i] < 1)
      return TG_EINVAL;
    if (res->budget[i] < 1 || res->budget[i] > res->length[i]) return TG_EINVAL;
  }
  return TG_OK;
}

// Flattened radix paths per request; validated against n_fixed = L - budget.
struct Paths {
  bool on = false;
  std::vector<std::vector<int32_t>> ids;
  std::vector<int64_t> node_len;
};

int check_share(const tg_share_desc* sh, const tg_reservation* res, const Geometry& g, Paths* p) {
  p->on = false;
  if (!sh) return TG_OK;
  if (!sh->n_nodes || !sh->node_len || sh->n_node_table < 0) return TG_EINVAL;
  p->on = true;
  p->node_len.resize(sh->n_node_table);
  for (int32_t n = 0; n < sh->n_node_table; ++n) {
    if (sh->node_len[n] < 0) return TG_EINVAL;
    p->node_len[n] = sh->node_len[n];
  }
  p->ids.assign(g.B, {});
  int64_t off = 0;
  for (int32_t r = 0; r < g.B; ++r) {
    if (sh->n_nodes[r] < 0) return TG_EINVAL;
    if (sh->n_nodes[r] > 0 && !sh->node_ids) return TG_EINVAL;
    int64_t tot = 0;
    for (int32_t k = 0; k < sh->n_nodes[r]; ++k) {
      const int32_t nid = sh->node_ids[off + k];
      if (nid < 0 || nid >= sh->n_node_table) return TG_EINVAL;
      p->ids[r].push_back(nid);
      tot += p->node_len[nid];
    }
    off += sh->n_nodes[r];
    for (int32_t h = 0; h < g.H; ++h) {
      const int64_t i = int64_t(r) * g.H + h;
      if (res->length[i] - res->budget[i] != tot) return TG_EINVAL;
    }
  }
  return TG_OK;
}

// Tier split of a sequence of L rows: INT8 rows (whole blocks of the rows
// older than the recent share).
int64_t i8_rows(int64_t L, int64_t recent_ppm, int64_t qb) {
  return ((L - ceil_div(L * recent_ppm, kPpm)) / qb) * qb;
}

// Sizes when every (r, h) may grow by T rows: INT8 rows of L + T and the most
// bf16 rows held at any length from L to L + T (the tables are built for
// these; lengths stay the live ones).
struct Capacity {
  std::vector<int32_t> length, n_i8, n_bf;
  tg_reservation view;
};

int make_capacity(const tg_reservation* res, int32_t T, Capacity* cap) {
  const int64_t n = int64_t(res->B) * res->n_kv_heads;
  if (res->quant_block < 1 || res->recent_ppm < 0 || res->recent_ppm > kPpm) return TG_EINVAL;
  cap->length.resize(n);
  cap->n_i8.resize(n);
  cap->n_bf.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    int64_t i8 = res->n_i8[i], bf = res->n_bf[i], top = bf;
    for (int32_t k = 0; k < T; ++k) {
      ++bf;
      if (i8_rows(i8 + bf, res->recent_ppm, res->quant_block) > i8) {
        i8 += res->quant_block;
        bf -= res->quant_block;
      }
      top = std::max(top, bf);
    }
    if (i8 + top > std::numeric_limits<int32_t>::max()) return TG_EOVERFLOW;
    cap->n_i8[i] = static_cast<int32_t>(i8);
    cap->n_bf[i] = static_cast<int32_t>(top);
    cap->length[i] = static_cast<int32_t>(i8 + top);
  }
  cap->view = *res;
  cap->view.length = cap->length.data();
  cap->view.n_i8 = cap->n_i8.data();
  cap->view.n_bf = cap->n_bf.data();
  return TG_OK;
}

int check_opts(const tg_plan_opts* o, int32_t ps, int32_t qb) {
  if (!o) return TG_EINVAL;
  if (o->chunk_bf < ps || o->chunk_bf % ps || o->chunk_i8 < qb || o->chunk_i8 % qb) return TG_EINVAL;
  if (o->group_size < 0 || o->group_size > TG_GROUP_WIDTH) return TG_EINVAL;
  if (o->gen_tokens < 0) return TG_EINVAL;
  if (o->chunk_group < 0 || o->chunk_group % ps) return TG_EINVAL;
  return TG_OK;
}

inline int64_t pages_of(const tg_reservation* res, const Geometry& g, int32_t r, int32_t c, int32_t t) {
  int64_t m = 0;
  for (int32_t h : g.heads[c]) {
    const int64_t i = int64_t(r) * g.H + h;
    m = std::max<int64_t>(m, t == TG_TIER_BF16 ? res->n_bf[i] : res->n_i8[i]);
  }
  return t == TG_TIER_BF16 ? ceil_div(m, g.ps) : m / g.qb;
}

// Share key of page j of row (r, c, t); false when the page is private.
bool share_key(const tg_reservation* res, const Geometry& g, const Paths& paths, int32_t r,
               int32_t c, int32_t t, int64_t j, ShareKey* key) {
  if (!paths.on) return false;
  const int64_t S = t == TG_TIER_BF16 ? g.ps : g.qb;
  int64_t start = -1;
  for (int32_t h : g.heads[c]) {
    const int64_t i = int64_t(r) * g.H + h;
    const int64_t s = (t == TG_TIER_I8 ? 0 : res->n_i8[i]) + j * S;
    if (start >= 0 && s != start) return false;
    start = s;
  }
  const int64_t n_fixed = res->length[int64_t(r) * g.H] - res->budget[int64_t(r) * g.H];
  if (start + S > n_fixed) return false;
  const int64_t last = start + S - 1;
  int64_t acc = 0;
  for (int32_t nid : paths.ids[r]) {
    acc += paths.node_len[nid];
    if (last < acc) {
      *key = ShareKey{c, t, nid, start};
      return true;
    }
  }
  return false;  // unreachable: last < n_fixed = total path length
}

int count_plan(const tg_reservation* res, const Geometry& g, const tg_plan_opts* o, int64_t* n) {
  int64_t items = 0;
  for (int64_t i = 0; i < int64_t(g.B) * g.H; ++i)
    items += ceil_div(res->n_i8[i], o->chunk_i8) + ceil_div(res->n_bf[i], o->chunk_bf);
  if (items > std::numeric_limits<int32_t>::max()) return TG_EOVERFLOW;
  *n = items;
  return TG_OK;
}

// Rows [lo, hi) as near-equal items of whole units (pages or INT8 blocks),
// at most `chunk` rows each: k = ceil(u / c) items over u units (c = chunk /
// unit), item i starting at unit floor(i * u / k).  In a plan with room for
// appended rows, rows up to hi_live are live and the rest reserved: the item
// count then follows the live rows, k = max(1, ceil(u_live / c), ceil(u /
// 2c)), so that the room adds no items (items stay under 2 chunk rows).
template <typename F>
void split_range(int64_t lo, int64_t hi, int64_t hi_live, int64_t unit, int64_t chunk, F&& emit) {
  const int64_t u = ceil_div(hi - lo, unit);
  if (u <= 0) return;
  const int64_t c = chunk / unit;
  int64_t k = ceil_div(u, c);
  if (hi_live < hi) {
    const int64_t u_live = ceil_div(std::max<int64_t>(hi_live - lo, 0), unit);
    k = std::max<int64_t>({1, ceil_div(u_live, c), ceil_div(u, 2 * c)});
  }
  for (int64_t i = 0; i < k; ++i)
    emit(lo + (i * u / k) * unit, std::min(lo + ((i + 1) * u / k) * unit, hi));
}

// The split plan: work items {r, h, tier, t0, t1, slot}, the slot CSR per
// (r, h) and the member table of group items.
struct Plan {
  std::vector<int32_t> work;      // [n_items * 6]
  std::vector<int32_t> part_off;  // [B*H + 1]
  std::vector<int32_t> gitems;    // [n_gitems * TG_GROUP_WIDTH * 2]
  int64_t n_items() const { return int64_t(work.size()) / 6; }
  int64_t n_gitems() const { return int64_t(gitems.size()) / (2 * TG_GROUP_WIDTH); }
};

// A run of leading shared bf16 pages of (r, c) that belong to one radix node.
struct Run {
  int32_t node;
  int64_t ja, jb, start;
};

std::vector<Run> shared_runs(const tg_reservation* res, const Geometry& g, const Paths& paths, int32_t r,
                             int32_t c) {
  std::vector<Run> runs;
  const int64_t np = pages_of(res, g, r, c, TG_TIER_BF16);
  ShareKey k;
  for (int64_t j = 0; j < np && share_key(res, g, paths, r, c, TG_TIER_BF16, j, &k); ++j) {
    if (!runs.empty() && runs.back().node == k.node && runs.back().jb == j)
      runs.back().jb = j + 1;
    else
      runs.push_back(Run{k.node, j, j + 1, k.start});
  }
  return runs;
}

struct RunIdent {
  int64_t node, start, npages, n_i8;
  bool operator==(const RunIdent& o) const {
    return node == o.node && start == o.start && npages == o.npages && n_i8 == o.n_i8;
  }
};
struct RunIdentHash {
  size_t operator()(const RunIdent& x) const {
    uint64_t h = 1469598103934665603ull;
    for (int64_t v : {x.node, x.start, x.npages, x.n_i8}) h = (h ^ uint64_t(v)) * 1099511628211ull;
    return size_t(h);
  }
};

// Longest-first cost of one row of tier t: its HBM bytes (4d for bf16; codes
// 2d * bits / 8 plus 4d / qb of scales for the quantised tier) times 4 qb / d.
int64_t lpt_weight(int32_t t, int32_t qb, int32_t bits) {
  return t == TG_TIER_BF16 ? 16 * int64_t(qb) : int64_t(bits) * qb + 16;
}

// `res` holds the rows the plan tiles (the reserved capacity for growth),
// `live` the live rows (the same reservation without growth).
int make_plan(const tg_reservation* res, const tg_reservation* live, const Geometry& g, const Paths& paths,
              const tg_plan_opts* o, int32_t old_bits, Plan* p) {
  int64_t bound = 0;
  int st = count_plan(res, g, o, &bound);
  if (st) return st;
  const int64_t BH = int64_t(g.B) * g.H;
  std::vector<int64_t> shared_rows(BH, 0);
  // group items: head, row range, members (ascending r)
  struct GItem {
    int32_t h;
    int64_t t0, t1;
    std::vector<int32_t> members;
  };
  std::vector<GItem> gi;
  if (o->group_size > 1 && paths.on) {
    std::vector<std::vector<Run>> runs(int64_t(g.B) * g.C);
    for (int32_t r = 0; r < g.B; ++r)
      for (int32_t c = 0; c < g.C; ++c) runs[int64_t(r) * g.C + c] = shared_runs(res, g, paths, r, c);
    for (int32_t h = 0; h < g.H; ++h) {
      const int32_t c = res->cluster_of_head[h];
      std::unordered_map<RunIdent, size_t, RunIdentHash> index;
      struct Group {
        RunIdent id;
        int64_t ja;
        std::vector<int32_t> members;
      };
      std::vector<Group> order;
      for (int32_t r = 0; r < g.B; ++r) {
        const std::vector<Run>& rr = runs[int64_t(r) * g.C + c];
        if (!rr.empty()) shared_rows[int64_t(r) * g.H + h] = rr.back().jb * g.ps;
        for (const Run& u : rr) {
          const RunIdent id{u.node, u.start, u.jb - u.ja, res->n_i8[int64_t(r) * g.H + h]};
          auto it = index.find(id);
          if (it == index.end()) {
            it = index.emplace(id, order.size()).first;
            order.push_back(Group{id, u.ja, {}});
          }
          order[it->second].members.push_back(r);
        }
      }
      for (const Group& grp : order) {
        const int64_t lo = grp.ja * g.ps, hi = (grp.ja + grp.id.npages) * g.ps;
        for (size_t k = 0; k < grp.members.size(); k += o->group_size) {
          const size_t e = std::min(grp.members.size(), k + size_t(o->group_size));
          split_range(lo, hi, hi, g.ps, o->chunk_group > 0 ? o->chunk_group : o->chunk_bf,
                      [&](int64_t t0, int64_t t1) {
            gi.push_back(GItem{h, t0, t1, std::vector<int32_t>(grp.members.begin() + k, grp.members.begin() + e)});
          });
        }
      }
    }
  }
  // memberships of each (r, h), in group-item order
  std::vector<std::vector<std::pair<int32_t, int32_t>>> member_of(BH);  // (group item, member index)
  for (size_t k = 0; k < gi.size(); ++k)
    for (size_t m = 0; m < gi[k].members.size(); ++m)
      member_of[int64_t(gi[k].members[m]) * g.H + gi[k].h].push_back({int32_t(k), int32_t(m)});
  if (int64_t(gi.size()) + bound > std::numeric_limits<int32_t>::max()) return TG_EOVERFLOW;
  p->gitems.assign(gi.size() * 2 * TG_GROUP_WIDTH, -1);
  p->part_off.assign(BH + 1, 0);
  p->work.clear();
  p->work.reserve((gi.size() + size_t(bound)) * 6);
  for (size_t k = 0; k < gi.size(); ++k) {
    const int32_t w[6] = {-1 - int32_t(k), gi[k].h, TG_TIER_BF16, int32_t(gi[k].t0), int32_t(gi[k].t1), -1};
    p->work.insert(p->work.end(), w, w + 6);
  }
  int64_t slot = 0;
  for (int32_t r = 0; r < g.B; ++r)
    for (int32_t h = 0; h < g.H; ++h) {
      const int64_t i = int64_t(r) * g.H + h;
      p->part_off[i] = int32_t(slot);
      for (const auto& km : member_of[i]) {
        int32_t* e = p->gitems.data() + (int64_t(km.first) * TG_GROUP_WIDTH + km.second) * 2;
        e[0] = r;
        e[1] = int32_t(slot++);
      }
      for (int32_t t : {TG_TIER_I8, TG_TIER_BF16}) {
        const int64_t len = t == TG_TIER_BF16 ? res->n_bf[i] : res->n_i8[i];
        const int64_t len_live = t == TG_TIER_BF16 ? live->n_bf[i] : live->n_i8[i];
        const int64_t lo = t == TG_TIER_BF16 ? shared_rows[i] : 0;
        const int32_t ch = t == TG_TIER_BF16 ? o->chunk_bf : o->chunk_i8;
        const int32_t unit = t == TG_TIER_BF16 ? g.ps : g.qb;
        split_range(lo, len, len_live, unit, ch, [&](int64_t t0, int64_t t1) {
          const int32_t w[6] = {r, h, t, int32_t(t0), int32_t(t1), int32_t(slot++)};
          p->work.insert(p->work.end(), w, w + 6);
        });
      }
    }
  if (slot > std::numeric_limits<int32_t>::max()) return TG_EOVERFLOW;
  p->part_off[BH] = int32_t(slot);
  const int64_t n = p->n_items();
  if (o->lpt && n > 1) {
    std::vector<int32_t> order(n);
    for (int32_t k = 0; k < n; ++k) order[k] = k;
    auto cost = [&](int32_t k) {
      const int32_t* w = p->work.data() + int64_t(k) * 6;
      return int64_t(w[4] - w[3]) * lpt_weight(w[2], g.qb, old_bits);
    };
    // group items (r < 0) stay ahead of the rest; each part longest first
    auto group = [&](int32_t k) { return p->work[int64_t(k) * 6] < 0; };
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      if (group(a) != group(b)) return group(a);
      return cost(a) > cost(b);
    });
    std::vector<int32_t> tmp(p->work);
    for (int64_t k = 0; k < n; ++k)
      std::memcpy(p->work.data() + k * 6, tmp.data() + int64_t(order[k]) * 6, 6 * sizeof(int32_t));
  }
  return TG_OK;
}

}  // namespace

extern "C" int tg_size_tables(const tg_reservation* live, int32_t ps, int32_t qb,
                              const tg_share_desc* share, const tg_plan_opts* opts,
                              tg_table_sizes* out) {
  if (!out) return TG_EINVAL;
  Geometry g;
  int st = check_reservation(live, ps, qb, &g);
  if (st) return st;
  Paths paths;
  if ((st = check_share(share, live, g, &paths))) return st;
  if ((st = check_opts(opts, ps, qb))) return st;
  if (opts->gen_tokens > 0 && paths.on) return TG_EINVAL;
  Capacity cap;
  const tg_reservation* res = live;
  if (opts->gen_tokens > 0) {
    try {
      if ((st = make_capacity(live, opts->gen_tokens, &cap))) return st;
    } catch (...) {
      return TG_ENOMEM;
    }
    res = &cap.view;
  }
  Plan plan;
  try {
    // (the longest-first order, the only use of the code width, changes no size)
    if ((st = make_plan(res, live, g, paths, opts, 8, &plan))) return st;
  } catch (...) {
    return TG_ENOMEM;
  }
  std::memset(out, 0, sizeof(*out));
  out->n_items = static_cast<int32_t>(plan.n_items());
  out->n_gitems = static_cast<int32_t>(plan.n_gitems());
  out->n_slots = plan.part_off.back();
  for (int32_t c = 0; c < g.C; ++c)
    for (int32_t t = 0; t < 2; ++t) {
      int64_t stride = 0, need = 0;
      std::unordered_map<ShareKey, int64_t, ShareKeyHash> seen;
      for (int32_t r = 0; r < g.B; ++r) {
        const int64_t np = pages_of(res, g, r, c, t);
        stride = std::max(stride, np);
        for (int64_t j = 0; j < np; ++j) {
          ShareKey k;
          if (share_key(res, g, paths, r, c, t, j, &k)) {
            if (seen.emplace(k, 0).second) ++need;
          } else {
            ++need;
          }
        }
      }
      if (stride > std::numeric_limits<int32_t>::max()) return TG_EOVERFLOW;
      out->stride[c][t] = static_cast<int32_t>(stride);
      out->pages_needed[c][t] = need;
    }
  return TG_OK;
}

extern "C" int tg_build_tables(tg_pool* pool, const tg_reservation* live, const tg_share_desc* share,
                               const tg_plan_opts* opts, tg_tables* out) {
  if (!pool || !out) return TG_EINVAL;
  tg_table_sizes sz;
  int st = tg_size_tables(live, pool->page_size, pool->quant_block, share, opts, &sz);
  if (st) return st;
  Geometry g;
  check_reservation(live, pool->page_size, pool->quant_block, &g);
  Paths paths;
  check_share(share, live, g, &paths);
  Capacity cap;
  const tg_reservation* res = live;
  if (opts->gen_tokens > 0) {
    try {
      if ((st = make_capacity(live, opts->gen_tokens, &cap))) return st;
    } catch (...) {
      return TG_ENOMEM;
    }
    res = &cap.view;
  }
  if (g.C != pool->C || out->n_items != sz.n_items || out->n_gitems != sz.n_gitems || !out->len ||
      !out->part_off || !out->released || (sz.n_items > 0 && !out->work) ||
      (sz.n_gitems > 0 && !out->gitems))
    return TG_EINVAL;
  Plan plan;
  try {
    if ((st = make_plan(res, live, g, paths, opts, pool->old_bits, &plan))) return st;
  } catch (...) {
    return TG_ENOMEM;
  }
  for (int32_t c = 0; c < g.C; ++c) {
    if (pool->cluster_size[c] != res->cluster_size[c]) return TG_EINVAL;
    for (int32_t t = 0; t < 2; ++t) {
      if (out->stride[c][t] != sz.stride[c][t]) return TG_EINVAL;
      if (sz.stride[c][t] > 0 && !out->bt[c][t]) return TG_EINVAL;
    }
  }

  // Allocate with an undo journal so that a failure leaves the pool intact.
  enum Kind : uint8_t { kAlloc, kRef, kReg };
  struct Entry {
    Kind kind;
    int8_t c, t;
    int64_t pid;
  };
  std::vector<Entry> journal;
  std::vector<ShareKey> reg_keys;
  auto undo = [&]() {
    for (size_t k = journal.size(); k-- > 0;) {
      const Entry& e = journal[k];
      SubPool& sp = pool->sub[e.c][e.t];
      if (e.kind == kAlloc) {
        sp.ref[e.pid] = 0;
        sp.give_back(e.pid);
      } else if (e.kind == kRef) {
        --sp.ref[e.pid];
      } else {
        pool->registry.erase(sp.key_of[e.pid]);
        sp.has_key[e.pid] = 0;
      }
    }
  };
  try {
    for (int32_t r = 0; r < g.B; ++r)
      for (int32_t c = 0; c < g.C; ++c)
        for (int32_t t : {TG_TIER_I8, TG_TIER_BF16}) {
          SubPool& sp = pool->sub[c][t];
          const int64_t np = pages_of(res, g, r, c, t);
          int32_t* row = sz.stride[c][t] ? out->bt[c][t] + int64_t(r) * sz.stride[c][t] : nullptr;
          for (int64_t j = 0; j < np; ++j) {
            ShareKey key;
            const bool shared = share_key(res, g, paths, r, c, t, j, &key);
            int64_t pid = -1;
            if (shared) {
              auto it = pool->registry.find(key);
              if (it != pool->registry.end()) {
                pid = it->second;
                ++sp.ref[pid];
                journal.push_back({kRef, int8_t(c), int8_t(t), pid});
              }
            }
            if (pid < 0) {
              pid = sp.take_lowest();
              if (pid < 0) {
                undo();
                return TG_ENOMEM;
              }
              journal.push_back({kAlloc, int8_t(c), int8_t(t), pid});
              if (shared) {
                pool->registry.emplace(key, pid);
                sp.key_of[pid] = key;
                sp.has_key[pid] = 1;
                journal.push_back({kReg, int8_t(c), int8_t(t), pid});
              }
            }
            if (pid > std::numeric_limits<int32_t>::max()) {
              undo();
              return TG_EOVERFLOW;
            }
            row[j] = static_cast<int32_t>(pid);
          }
          for (int64_t j = np; j < sz.stride[c][t]; ++j) row[j] = -1;
        }
  } catch (...) {
    undo();
    return TG_ENOMEM;
  }

  // lengths
  for (int64_t i = 0; i < int64_t(g.B) * g.H; ++i) {
    out->len[2 * i] = live->n_i8[i];
    out->len[2 * i + 1] = live->n_bf[i];
  }
  std::copy(plan.work.begin(), plan.work.end(), out->work);
  std::copy(plan.part_off.begin(), plan.part_off.end(), out->part_off);
  std::copy(plan.gitems.begin(), plan.gitems.end(), out->gitems);
  if (out->ring)
    for (int32_t r = 0; r < g.B; ++r)
      for (int32_t c = 0; c < g.C; ++c)
        out->ring[int64_t(r) * g.C + c] = static_cast<int32_t>(pages_of(res, g, r, c, TG_TIER_BF16));
  for (int32_t r = 0; r < g.B; ++r) out->released[r] = 0;
  out->B = g.B;
  return TG_OK;
}

extern "C" int tg_stream_order(const tg_tables* t, int32_t B, int32_t* work_out, int32_t* chunk_off) {
  if (!t || B < 1 || !chunk_off || (t->n_items > 0 && (!t->work || !work_out))) return TG_EINVAL;
  std::vector<int32_t> count(B, 0);
  int32_t n_bf = 0;
  for (int32_t k = 0; k < t->n_items; ++k) {
    const int32_t* w = t->work + int64_t(k) * 6;
    if (w[2] == TG_TIER_I8) {
      if (w[0] < 0 || w[0] >= B) return TG_EINVAL;
      ++count[w[0]];
    } else {
      ++n_bf;
    }
  }
  chunk_off[0] = n_bf;
  for (int32_t r = 0; r < B; ++r) chunk_off[r + 1] = chunk_off[r] + count[r];
  std::vector<int32_t> at(chunk_off, chunk_off + B);
  int32_t nb = 0;
  for (int32_t k = 0; k < t->n_items; ++k) {
    const int32_t* w = t->work + int64_t(k) * 6;
    const int32_t dst = w[2] == TG_TIER_I8 ? at[w[0]]++ : nb++;
    std::memcpy(work_out + int64_t(dst) * 6, w, 6 * sizeof(int32_t));
  }
  return TG_OK;
}

extern "C" int tg_release(tg_pool* pool, tg_tables* t, int32_t r) {
  if (!pool || !t || !t->released || r < 0 || r >= t->B) return TG_EINVAL;
  if (t->released[r]) return TG_EINVAL;
  for (int32_t c = 0; c < pool->C; ++c)
    for (int32_t tier = 0; tier < 2; ++tier) {
      const int32_t stride = t->stride[c][tier];
      if (!stride) continue;
      const int32_t* row = t->bt[c][tier] + int64_t(r) * stride;
      SubPool& sp = pool->sub[c][tier];
      for (int32_t j = 0; j < stride && row[j] >= 0; ++j) {
        const int64_t pid = row[j];
        if (pid >= sp.cap || sp.ref[pid] <= 0) return TG_EINVAL;
      }
    }
  for (int32_t c = 0; c < pool->C; ++c)
    for (int32_t tier = 0; tier < 2; ++tier) {
      const int32_t stride = t->stride[c][tier];
      if (!stride) continue;
      const int32_t* row = t->bt[c][tier] + int64_t(r) * stride;
      SubPool& sp = pool->sub[c][tier];
      for (int32_t j = 0; j < stride && row[j] >= 0; ++j) {
        const int64_t pid = row[j];
        if (--sp.ref[pid] == 0) {
          sp.give_back(pid);
          if (sp.has_key[pid]) {
            pool->registry.erase(sp.key_of[pid]);
            sp.has_key[pid] = 0;
          }
        }
      }
    }
  t->released[r] = 1;
  return TG_OK;
}

// --------------------------------------------------------------------------
// table check (debugging aid)
// --------------------------------------------------------------------------
namespace {

int check_fail(char* msg, size_t msg_bytes, const char* fmt, ...) {
  if (msg && msg_bytes > 0) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(msg, msg_bytes, fmt, ap);
    va_end(ap);
  }
  return TG_EINVAL;
}

}  // namespace

extern "C" int tg_check_tables(const tg_pool* pool, const tg_reservation* res, const tg_tables* t, char* msg,
                               size_t msg_bytes) {
  if (msg && msg_bytes > 0) msg[0] = '\0';
  if (!pool || !res || !t) return check_fail(msg, msg_bytes, "null argument");
  Geometry g;
  if (check_reservation(res, pool->page_size, pool->quant_block, &g))
    return check_fail(msg, msg_bytes, "malformed reservation");
  if (g.C != pool->C) return check_fail(msg, msg_bytes, "reservation has %d clusters, the pool %d", g.C, pool->C);
  for (int32_t c = 0; c < g.C; ++c)
    if (pool->cluster_size[c] != res->cluster_size[c])
      return check_fail(msg, msg_bytes, "cluster %d: %d heads in the reservation, %d in the pool", c,
                        res->cluster_size[c], pool->cluster_size[c]);
  if (t->B != g.B) return check_fail(msg, msg_bytes, "tables hold %d requests, the reservation %d", t->B, g.B);
  if (!t->len || !t->part_off || t->n_items < 0 || t->n_gitems < 0 || (t->n_items > 0 && !t->work) ||
      (t->n_gitems > 0 && !t->gitems))
    return check_fail(msg, msg_bytes, "missing table array or negative count");
  const int64_t BH = int64_t(g.B) * g.H;
  try {
    // block tables: page ids first, then -1; ids inside the pool, referenced
    // no more often than their reference counts allow
    std::vector<int64_t> pages(size_t(g.B) * g.C * 2, 0);  // pages in row (r, c, tier)
    auto npages = [&](int32_t r, int32_t c, int32_t tier) -> int64_t& {
      return pages[(size_t(r) * g.C + c) * 2 + tier];
    };
    for (int32_t c = 0; c < g.C; ++c)
      for (int32_t tier = 0; tier < 2; ++tier) {
        const int32_t stride = t->stride[c][tier];
        if (stride < 0) return check_fail(msg, msg_bytes, "negative stride of (%d, %d)", c, tier);
        if (stride == 0) continue;
        if (!t->bt[c][tier]) return check_fail(msg, msg_bytes, "no block table for (%d, %d)", c, tier);
        const SubPool& sp = pool->sub[c][tier];
        std::vector<int32_t> uses(size_t(sp.cap), 0);
        for (int32_t r = 0; r < g.B; ++r) {
          if (t->released && t->released[r]) continue;
          const int32_t* row = t->bt[c][tier] + int64_t(r) * stride;
          int32_t j = 0;
          for (; j < stride && row[j] >= 0; ++j) {
            if (row[j] >= sp.cap)
              return check_fail(msg, msg_bytes, "bt[%d][%d] row %d entry %d: page %d past the capacity %lld", c,
                                tier, r, j, row[j], static_cast<long long>(sp.cap));
            ++uses[row[j]];
          }
          npages(r, c, tier) = j;
          for (; j < stride; ++j)
            if (row[j] != -1)
              return check_fail(msg, msg_bytes, "bt[%d][%d] row %d entry %d: %d after the row's last page", c,
                                tier, r, j, row[j]);
        }
        for (int64_t pid = 0; pid < sp.cap; ++pid)
          if (uses[pid] > sp.ref[pid])
            return check_fail(msg, msg_bytes, "(%d, %d) page %lld: %d table entries, reference count %d", c, tier,
                              static_cast<long long>(pid), uses[pid], sp.ref[pid]);
      }
    // lengths within the rows the pages (or the bf16 ring) hold
    auto cap_rows = [&](int32_t r, int32_t c, int32_t tier) -> int64_t {
      if (tier == TG_TIER_I8) return npages(r, c, tier) * g.qb;
      if (t->ring) return int64_t(t->ring[int64_t(r) * g.C + c]) * g.ps;
      return npages(r, c, tier) * g.ps;
    };
    for (int32_t r = 0; r < g.B; ++r) {
      if (t->released && t->released[r]) continue;
      if (t->ring)
        for (int32_t c = 0; c < g.C; ++c) {
          const int32_t ring = t->ring[int64_t(r) * g.C + c];
          if (ring < 0 || ring > npages(r, c, TG_TIER_BF16))
            return check_fail(msg, msg_bytes, "ring of (%d, %d) is %d pages, the row has %lld", r, c, ring,
                              static_cast<long long>(npages(r, c, TG_TIER_BF16)));
        }
      for (int32_t h = 0; h < g.H; ++h) {
        const int64_t i = int64_t(r) * g.H + h;
        const int32_t c = res->cluster_of_head[h];
        const int32_t n8 = t->len[2 * i], nb = t->len[2 * i + 1];
        if (n8 < 0 || nb < 0 || n8 % g.qb)
          return check_fail(msg, msg_bytes, "len of (%d, %d) is (%d, %d)", r, h, n8, nb);
        if (n8 > cap_rows(r, c, TG_TIER_I8) || nb > cap_rows(r, c, TG_TIER_BF16))
          return check_fail(msg, msg_bytes, "len of (%d, %d) = (%d, %d) passes its pages (%lld, %lld rows)", r, h,
                            n8, nb, static_cast<long long>(cap_rows(r, c, TG_TIER_I8)),
                            static_cast<long long>(cap_rows(r, c, TG_TIER_BF16)));
      }
    }
    // slots
    if (t->part_off[0] != 0) return check_fail(msg, msg_bytes, "part_off[0] is %d", t->part_off[0]);
    for (int64_t i = 0; i < BH; ++i)
      if (t->part_off[i + 1] < t->part_off[i])
        return check_fail(msg, msg_bytes, "part_off decreases at %lld", static_cast<long long>(i));
    const int64_t n_slots = t->part_off[BH];
    std::vector<uint8_t> slot_used(size_t(n_slots), 0);
    auto take_slot = [&](int64_t rh, int32_t slot, int64_t item) -> int {
      if (slot < t->part_off[rh] || slot >= t->part_off[rh + 1])
        return check_fail(msg, msg_bytes, "item %lld: slot %d outside [%d, %d) of pair %lld",
                          static_cast<long long>(item), slot, t->part_off[rh], t->part_off[rh + 1],
                          static_cast<long long>(rh));
      if (slot_used[slot]++)
        return check_fail(msg, msg_bytes, "item %lld: slot %d used twice", static_cast<long long>(item), slot);
      return TG_OK;
    };
    // plan: ranges of every (r, h, tier), group items once each
    std::vector<std::vector<std::pair<int32_t, int32_t>>> ranges(size_t(BH) * 2);
    std::vector<uint8_t> gseen(size_t(t->n_gitems), 0);
    for (int64_t k = 0; k < t->n_items; ++k) {
      const int32_t* w = t->work + k * 6;
      const int32_t h = w[1], tier = w[2], t0 = w[3], t1 = w[4];
      if (h < 0 || h >= g.H || (tier != TG_TIER_I8 && tier != TG_TIER_BF16) || t0 < 0 || t1 <= t0)
        return check_fail(msg, msg_bytes, "item %lld: (h %d, tier %d, rows %d..%d)", static_cast<long long>(k), h,
                          tier, t0, t1);
      const int32_t c = res->cluster_of_head[h];
      if (w[0] >= 0) {
        const int32_t r = w[0];
        if (r >= g.B) return check_fail(msg, msg_bytes, "item %lld: request %d", static_cast<long long>(k), r);
        if (t->released && t->released[r]) continue;
        const int64_t rh = int64_t(r) * g.H + h;
        if (int st = take_slot(rh, w[5], k)) return st;
        if (t1 > cap_rows(r, c, tier))
          return check_fail(msg, msg_bytes, "item %lld: rows %d..%d pass the %lld rows of its pages",
                            static_cast<long long>(k), t0, t1, static_cast<long long>(cap_rows(r, c, tier)));
        ranges[size_t(rh) * 2 + tier].push_back({t0, t1});
        continue;
      }
      const int64_t gk = -1 - int64_t(w[0]);
      if (gk >= t->n_gitems || tier != TG_TIER_BF16 || w[5] != -1)
        return check_fail(msg, msg_bytes, "item %lld: group item %lld (tier %d, slot %d)", static_cast<long long>(k),
                          static_cast<long long>(gk), tier, w[5]);
      if (gseen[gk]++)
        return check_fail(msg, msg_bytes, "group item %lld listed twice", static_cast<long long>(gk));
      const int32_t* gm = t->gitems + gk * 2 * TG_GROUP_WIDTH;
      if (gm[0] < 0) return check_fail(msg, msg_bytes, "group item %lld has no member", static_cast<long long>(gk));
      const int32_t r0 = gm[0];
      for (int32_t m = 0; m < TG_GROUP_WIDTH; ++m) {
        const int32_t r = gm[2 * m], slot = gm[2 * m + 1];
        if (r < 0) {
          for (int32_t e = m; e < TG_GROUP_WIDTH; ++e)
            if (gm[2 * e] != -1 || gm[2 * e + 1] != -1)
              return check_fail(msg, msg_bytes, "group item %lld: member entry %d after the padding",
                                static_cast<long long>(gk), e);
          break;
        }
        if (r >= g.B || (m > 0 && r <= gm[2 * m - 2]))
          return check_fail(msg, msg_bytes, "group item %lld: member %d is request %d (not ascending or out of range)",
                            static_cast<long long>(gk), m, r);
        if (t->released && t->released[r]) continue;
        const int64_t rh = int64_t(r) * g.H + h;
        if (int st = take_slot(rh, slot, k)) return st;
        if (t1 > cap_rows(r, c, TG_TIER_BF16))
          return check_fail(msg, msg_bytes, "group item %lld: rows %d..%d pass request %d's pages",
                            static_cast<long long>(gk), t0, t1, r);
        // the members read the very same pages
        const int32_t stride = t->stride[c][TG_TIER_BF16];
        for (int64_t pg = t0 / g.ps; pg < ceil_div(t1, g.ps); ++pg)
          if (t->bt[c][TG_TIER_BF16][int64_t(r) * stride + pg] != t->bt[c][TG_TIER_BF16][int64_t(r0) * stride + pg])
            return check_fail(msg, msg_bytes, "group item %lld: request %d's page %lld differs from request %d's",
                              static_cast<long long>(gk), r, static_cast<long long>(pg), r0);
        ranges[size_t(rh) * 2 + TG_TIER_BF16].push_back({t0, t1});
      }
    }
    for (int64_t gk = 0; gk < t->n_gitems; ++gk)
      if (!gseen[gk]) return check_fail(msg, msg_bytes, "group item %lld is in no plan entry", static_cast<long long>(gk));
    for (int64_t sl = 0; sl < n_slots; ++sl)
      if (!slot_used[sl]) {
        // a released request's slots are not checked
        int64_t rh = std::upper_bound(t->part_off, t->part_off + BH + 1, int32_t(sl)) - t->part_off - 1;
        if (t->released && t->released[rh / g.H]) continue;
        return check_fail(msg, msg_bytes, "slot %lld is written by no item", static_cast<long long>(sl));
      }
    // every tier range is tiled once from row 0 past its live rows
    for (int64_t rh = 0; rh < BH; ++rh) {
      if (t->released && t->released[rh / g.H]) continue;
      for (int32_t tier = 0; tier < 2; ++tier) {
        auto& v = ranges[size_t(rh) * 2 + tier];
        std::sort(v.begin(), v.end());
        const int32_t live = t->len[2 * rh + tier];
        int64_t at = 0;
        for (const auto& x : v) {
          if (x.first != at)
            return check_fail(msg, msg_bytes, "pair %lld tier %d: items leave rows %lld..%d %s",
                              static_cast<long long>(rh), tier, static_cast<long long>(at), x.first,
                              x.first > at ? "uncovered" : "covered twice");
          at = x.second;
        }
        if (at < live)
          return check_fail(msg, msg_bytes, "pair %lld tier %d: items end at row %lld, %d rows are live",
                            static_cast<long long>(rh), tier, static_cast<long long>(at), live);
      }
    }
  } catch (...) {
    return TG_ENOMEM;
  }
  return TG_OK;
}
