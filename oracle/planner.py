"""Integer oracle for admission: budgets, clusters, tiers, pages, tables, plan.

TEST INFRASTRUCTURE (see ``oracle/__init__``).  Everything here is exact
integer arithmetic in Python ints; it is written from the pages and from the
readings stated below, never from the C++ planner.

Sources (page, section):

* Tangram page (arXiv 2606.06302 explainer), "Key finding: two-level structural
  law" -- head importance ranking is input-invariant and each head's retention
  ratio lies in a narrow band; "Three mechanisms", item 1 (Budget Reservation)
  -- each head's post-compression footprint is fixed when the request starts;
  item 2 (Ragged Paging) -- heads with similar budgets share their own page
  table, and pages need not all be the same size; item 3 (AOT load balancing)
  -- work is partitioned ahead of time by KV occupancy, with no runtime
  re-planning.
* TTKV page (arXiv 2604.19769 explainer), "Tier Content" -- the most recent N%
  of tokens stay in the high-precision fast tier, the rest go to the
  block-quantised slow tier; "Tier Interaction" -- the slow tier is quantised
  in blocks.
* RadixAttention lesson, "The concept" -- each radix-tree node owns a token
  range and its KV blocks, and requests on the same branch reuse them.

Readings where the pages are silent (each also listed in the design notes):

R-rank   ratio_ppm(k) = hi - floor((hi - lo) * k / (H - 1)) for rank k
         (k = 0 most important), hi when H == 1.
R-round  budget = clamp(ceil(ratio_ppm * n_comp / 1e6), 1, n_comp); a given
         per-(request, KV-head) override replaces it.  L = n_fixed + budget.
R-clust  heads sorted by rank are cut into C contiguous groups; group c has
         ceil(H/C) heads if c < H mod C, else floor(H/C).
R-tier   n_bf0 = ceil(L * recent_ppm / 1e6); n_i8 = floor((L - n_bf0) / Qb) * Qb;
         n_bf = L - n_i8.  INT8 rows are the oldest: logical rows [0, n_i8).
R-page   a page of tier t holds S_t token slots (P for bf16, Qb for INT8) for
         every head of its cluster.  Row r of cluster c needs
         ceil(max_h n_bf / P) bf16 pages and max_h n_i8 / Qb INT8 pages.
R-alloc  each (cluster, tier) pool hands out the lowest free page id.  Order:
         request, cluster, tier (INT8 then bf16), page.  A page is shared when
         every head of the cluster starts it at the same logical position s
         and s + S_t <= n_fixed[r]; its key is (c, t, node holding position
         s + S_t - 1, s).  A key seen before adds a reference, otherwise a
         fresh page is taken and the key registered.  A failed call leaves the
         pool exactly as it was.
R-plan   items (r, h, tier, t0, t1, slot) in order r, h, tier (INT8 first).
         A row range of u units (pages, or INT8 blocks; the last may be
         partial) is cut into k = ceil(u / (chunk / unit)) items as equal as
         whole units allow: item i starts at unit floor(i * u / k).  slot is
         the natural index; part_off is the CSR of slots per (r, h).  With lpt,
         items are stably sorted by descending cost (t1 - t0) * w_tier, w_tier
         proportional to the HBM bytes one row of the tier costs: a bf16 row is
         4d bytes, a quantised row 2d * bits / 8 bytes of codes plus 4d / Qb of
         scales, so w = 16 Qb (bf16) and bits * Qb + 16 (INT8 or INT4), the
         common factor d / (4 Qb) dropped; group items (R-group) stay ahead of
         all other items, each part sorted on its own.
R-step   (decode-step growth) an appended row becomes the newest bf16 row
         and R-tier is applied to the new length; when the INT8 boundary moves
         (by one block) the oldest Qb bf16 rows are quantised (R-q) into the
         next INT8 block.  Pages for gen_tokens appended rows are reserved at
         admission: INT8 rows of the final length, and the most bf16 rows held
         at any length on the way; the bf16 tier turns over its pages as a
         ring.  Not combined with shared radix pages.  The plan tiles the
         reserved rows; its item count per range follows the live rows
         (k = ceil(u_live / c), raised only to keep items at most 2 chunk
         rows), so that room for appended rows adds no items.
R-group  (only with a group size > 1 and radix paths) the leading shared bf16
         pages of each (r, h) are cut into runs with the same radix node;
         requests whose run has the same (node, first row, page count, INT8
         rows) are taken in ascending r, group_size at a time, and each group's
         rows are chunked as in R-plan, with chunk_group rows (chunk_bf when
         chunk_group is 0), from the run's first row into group items (listed
         first: per h, runs in order of first appearance, groups, chunks).  A
         request's own bf16 items then start after its shared rows.  Slots: per
         (r, h) in natural order, its group memberships (in group-item order)
         then its own items.

Pinned by: tests/test_oracle_planner.py (hand-worked golden tables, the
worked radix example's consistent block counts, a second allocator written
over a sorted free list, and the invariants the rules imply).
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

TIER_I8 = 0
TIER_BF = 1
PPM = 1_000_000


class OracleError(Exception):
    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _ceil_div(a: int, b: int) -> int:
    return -((-a) // b)


# ---------------------------------------------------------------- budgets
def ratio_ppm(k: int, H: int, hi: int, lo: int) -> int:
    """Retention ratio (ppm) of the head at importance rank ``k`` (R-rank)."""
    if H == 1:
        return hi
    return hi - ((hi - lo) * k) // (H - 1)


@dataclass
class Reservation:
    budget: List[List[int]]          # [B][H]
    L: List[List[int]]               # [B][H]
    n_i8: List[List[int]]            # [B][H]
    n_bf: List[List[int]]            # [B][H]
    cluster_of_head: List[int]       # [H]
    slot_in_cluster: List[int]       # [H]
    cluster_size: List[int]          # [C]
    recent_ppm: int = PPM
    quant_block: int = 64


def tier_split(L: int, recent_ppm: int, quant_block: int) -> Tuple[int, int]:
    """(n_i8, n_bf) of a sequence of L rows (R-tier)."""
    old = L - _ceil_div(L * recent_ppm, PPM)
    i8 = (old // quant_block) * quant_block
    return i8, L - i8


def reserve(head_rank: Sequence[int], ratio_hi_ppm: int, ratio_lo_ppm: int,
            n_clusters: int, recent_ppm: int, quant_block: int,
            n_comp: Sequence[int], n_fixed: Optional[Sequence[int]] = None,
            budget_override: Optional[Sequence[int]] = None) -> Reservation:
    """Budget reservation, clustering and tier split for a batch (R-rank,
    R-round, R-clust, R-tier)."""
    H = len(head_rank)
    B = len(n_comp)
    rank = [int(x) for x in head_rank]
    if sorted(rank) != list(range(H)):
        raise OracleError("EINVAL", "head_rank is not a permutation")
    if not (0 < ratio_lo_ppm <= ratio_hi_ppm <= PPM):
        raise OracleError("EINVAL", "ratio bounds")
    if not (1 <= n_clusters <= H):
        raise OracleError("EINVAL", "n_clusters")
    if not (0 <= recent_ppm <= PPM) or quant_block < 1:
        raise OracleError("EINVAL", "tier parameters")
    nf = [0] * B if n_fixed is None else [int(x) for x in n_fixed]
    budget, L = [], []
    for r in range(B):
        n = int(n_comp[r])
        if n < 1 or nf[r] < 0:
            raise OracleError("EINVAL", "lengths")
        row = []
        for h in range(H):
            if budget_override is not None:
                b = int(budget_override[r * H + h])
                if not (1 <= b <= n):
                    raise OracleError("EINVAL", "override out of range")
            else:
                b = _ceil_div(ratio_ppm(rank[h], H, ratio_hi_ppm, ratio_lo_ppm) * n, PPM)
                b = min(max(b, 1), n)
            row.append(b)
        budget.append(row)
        L.append([nf[r] + b for b in row])

    order = sorted(range(H), key=lambda h: rank[h])
    sizes = [(H + n_clusters - 1) // n_clusters if c < H % n_clusters else H // n_clusters
             for c in range(n_clusters)]
    coh, sic = [0] * H, [0] * H
    pos = 0
    for c, sz in enumerate(sizes):
        for s in range(sz):
            coh[order[pos]] = c
            sic[order[pos]] = s
            pos += 1

    n_i8, n_bf = [], []
    for r in range(B):
        ri, rb = [], []
        for h in range(H):
            i8, bf = tier_split(L[r][h], recent_ppm, quant_block)
            ri.append(i8)
            rb.append(bf)
        n_i8.append(ri)
        n_bf.append(rb)
    return Reservation(budget, L, n_i8, n_bf, coh, sic, sizes, recent_ppm, quant_block)


# ---------------------------------------------------------------- decode-step growth
def append_step(n_i8: int, n_bf: int, recent_ppm: int, quant_block: int) -> Tuple[int, int, bool]:
    """One appended row (R-step): the row becomes the newest bf16 row, then
    the tier split of the new length decides whether the oldest quant_block
    bf16 rows become the next INT8 block.  Returns (n_i8, n_bf, aged)."""
    n_bf += 1
    i8, _ = tier_split(n_i8 + n_bf, recent_ppm, quant_block)
    if i8 > n_i8:
        return n_i8 + quant_block, n_bf - quant_block, True
    return n_i8, n_bf, False


def capacity(res: Reservation, gen_tokens: int) -> Reservation:
    """The reservation's sizes when every (r, h) may grow by gen_tokens rows
    (R-step): INT8 rows of the final length, and the most bf16 rows held at
    any length on the way.  Only the sizes are meaningful."""
    B, H = len(res.L), len(res.cluster_of_head)
    n_i8 = [[0] * H for _ in range(B)]
    n_bf = [[0] * H for _ in range(B)]
    for r in range(B):
        for h in range(H):
            i8, bf = res.n_i8[r][h], res.n_bf[r][h]
            top = bf
            for _ in range(gen_tokens):
                i8, bf, _aged = append_step(i8, bf, res.recent_ppm, res.quant_block)
                top = max(top, bf)
            n_i8[r][h], n_bf[r][h] = i8, top
    L = [[n_i8[r][h] + n_bf[r][h] for h in range(H)] for r in range(B)]
    return Reservation(res.budget, L, n_i8, n_bf, res.cluster_of_head, res.slot_in_cluster,
                       res.cluster_size, res.recent_ppm, res.quant_block)


# ---------------------------------------------------------------- pages
def heads_of_cluster(res: Reservation, c: int) -> List[int]:
    hs = [h for h in range(len(res.cluster_of_head)) if res.cluster_of_head[h] == c]
    return sorted(hs, key=lambda h: res.slot_in_cluster[h])


def page_counts(res: Reservation, page_size: int, quant_block: int) -> List[List[List[int]]]:
    """np[r][c][t] -- pages of row r in the (cluster c, tier t) table (R-page)."""
    B = len(res.L)
    C = len(res.cluster_size)
    out = []
    for r in range(B):
        rc = []
        for c in range(C):
            hs = heads_of_cluster(res, c)
            i8 = max(res.n_i8[r][h] for h in hs)
            bf = max(res.n_bf[r][h] for h in hs)
            assert i8 % quant_block == 0
            rc.append([i8 // quant_block, _ceil_div(bf, page_size)])
        out.append(rc)
    return out


def _node_at(path: Sequence[int], node_len: Sequence[int], pos: int) -> int:
    acc = 0
    for nid in path:
        acc += int(node_len[nid])
        if pos < acc:
            return nid
    raise AssertionError("position beyond shared path")


def share_key(res: Reservation, r: int, c: int, t: int, j: int, page_size: int,
              quant_block: int, n_fixed: Sequence[int],
              paths: Optional[Sequence[Sequence[int]]],
              node_len: Optional[Sequence[int]]):
    """Registry key of page j of row (r, c, t), or None if the page is private
    (R-alloc)."""
    if paths is None:
        return None
    S = quant_block if t == TIER_I8 else page_size
    starts = set()
    for h in heads_of_cluster(res, c):
        starts.add(j * S if t == TIER_I8 else res.n_i8[r][h] + j * S)
    if len(starts) != 1:
        return None
    s = starts.pop()
    if s + S > int(n_fixed[r]):
        return None
    return (c, t, _node_at(paths[r], node_len, s + S - 1), s)


class Pool:
    """Refcounted page pools, one per (cluster, tier), lowest free id first.

    Free ids are the freed ids (a min-heap) plus every id at or above the
    high-water mark ``top``; the lowest free id is the smaller of the two.
    """

    def __init__(self, pages_bf: Sequence[int], pages_i8: Sequence[int]):
        C = len(pages_bf)
        self.cap = [[int(pages_i8[c]), int(pages_bf[c])] for c in range(C)]
        self.ref = [[{} for _ in range(2)] for _ in range(C)]
        self.heap = [[[] for _ in range(2)] for _ in range(C)]
        self.top = [[0, 0] for _ in range(C)]
        self.registry: Dict[tuple, int] = {}
        self.key_of: Dict[Tuple[int, int, int], tuple] = {}

    def _snapshot(self):
        return ([[dict(x) for x in rc] for rc in self.ref],
                [[list(x) for x in rc] for rc in self.heap],
                [list(x) for x in self.top],
                dict(self.registry), dict(self.key_of))

    def _restore(self, snap):
        self.ref, self.heap, self.top, self.registry, self.key_of = snap

    def alloc(self, c: int, t: int) -> int:
        h = self.heap[c][t]
        if h:
            pid = heapq.heappop(h)
        elif self.top[c][t] < self.cap[c][t]:
            pid = self.top[c][t]
            self.top[c][t] += 1
        else:
            raise OracleError("ENOMEM", f"pool (c={c}, t={t}) exhausted")
        assert self.ref[c][t].get(pid, 0) == 0
        self.ref[c][t][pid] = 1
        return pid

    def unref(self, c: int, t: int, pid: int):
        self.ref[c][t][pid] -= 1
        if self.ref[c][t][pid] == 0:
            del self.ref[c][t][pid]
            heapq.heappush(self.heap[c][t], pid)
            key = self.key_of.pop((c, t, pid), None)
            if key is not None:
                del self.registry[key]

    def refcount(self, c: int, t: int, pid: int) -> int:
        return self.ref[c][t].get(pid, 0)

    def free_pages(self, c: int, t: int) -> int:
        return self.cap[c][t] - len(self.ref[c][t])


@dataclass
class Tables:
    bt: List[List[List[List[int]]]]   # bt[c][t][r][j], padded with -1
    stride: List[List[int]]           # stride[c][t]
    lens: List[List[Tuple[int, int]]]  # [r][h] -> (n_i8, n_bf)
    work: List[Tuple[int, int, int, int, int, int]]
    part_off: List[int]
    pages: List[List[List[List[int]]]] = field(default_factory=list)  # [r][c][t] -> ids


def allocate(pool: Pool, res: Reservation, page_size: int, quant_block: int,
             n_fixed: Optional[Sequence[int]] = None,
             paths: Optional[Sequence[Sequence[int]]] = None,
             node_len: Optional[Sequence[int]] = None) -> List[List[List[List[int]]]]:
    """Allocate every page of every row, all or nothing (R-alloc)."""
    B = len(res.L)
    C = len(res.cluster_size)
    nf = [0] * B if n_fixed is None else list(n_fixed)
    counts = page_counts(res, page_size, quant_block)
    snap = pool._snapshot()
    try:
        out = []
        for r in range(B):
            rc = []
            for c in range(C):
                rt = [None, None]
                for t in (TIER_I8, TIER_BF):
                    ids = []
                    for j in range(counts[r][c][t]):
                        key = share_key(res, r, c, t, j, page_size, quant_block, nf, paths, node_len)
                        if key is not None and key in pool.registry:
                            pid = pool.registry[key]
                            pool.ref[c][t][pid] += 1
                        else:
                            pid = pool.alloc(c, t)
                            if key is not None:
                                pool.registry[key] = pid
                                pool.key_of[(c, t, pid)] = key
                        ids.append(pid)
                    rt[t] = ids
                rc.append(rt)
            out.append(rc)
        return out
    except OracleError:
        pool._restore(snap)
        raise


def pages_needed(res: Reservation, page_size: int, quant_block: int,
                 n_fixed=None, paths=None, node_len=None) -> Tuple[List[int], List[int]]:
    """Pages an empty pool must hold for this batch: (bf16[C], INT8[C])."""
    C = len(res.cluster_size)
    big = [10 ** 9] * C
    p = Pool(big, big)
    allocate(p, res, page_size, quant_block, n_fixed, paths, node_len)
    bf = [p.cap[c][TIER_BF] - p.free_pages(c, TIER_BF) for c in range(C)]
    i8 = [p.cap[c][TIER_I8] - p.free_pages(c, TIER_I8) for c in range(C)]
    return bf, i8


def release(pool: Pool, pages_of_request: List[List[List[int]]]):
    """Drop request r's references (R-alloc): pages reaching zero are freed
    and their registry keys removed."""
    for c, rt in enumerate(pages_of_request):
        for t in (TIER_I8, TIER_BF):
            for pid in rt[t]:
                pool.unref(c, t, pid)


# ---------------------------------------------------------------- tables & plan
GROUP_WIDTH = 32  # member slots per group item in the member table


def shared_segments(res: Reservation, r: int, c: int, page_size: int, quant_block: int,
                    n_fixed, paths, node_len):
    """Leading shared bf16 pages of row (r, c), cut into runs with the same
    radix node: [(node, first page, end page, first row)] (R-group)."""
    np_bf = page_counts_row(res, r, c, page_size)
    segs = []
    j = 0
    while j < np_bf:
        key = share_key(res, r, c, TIER_BF, j, page_size, quant_block, n_fixed, paths, node_len)
        if key is None:
            break
        node, start = key[2], key[3]
        if segs and segs[-1][0] == node and segs[-1][2] == j:
            segs[-1][2] = j + 1
        else:
            segs.append([node, j, j + 1, start])
        j += 1
    return segs


def page_counts_row(res: Reservation, r: int, c: int, page_size: int) -> int:
    hs = heads_of_cluster(res, c)
    return _ceil_div(max(res.n_bf[r][h] for h in hs), page_size)


def split_range(lo: int, hi: int, unit: int, chunk: int, hi_live=None):
    """Rows [lo, hi) as near-equal items of whole units, at most chunk rows
    each (R-plan).  With hi_live (a plan with room for appended rows, R-step:
    rows up to hi_live are live, the rest reserved) the item count follows the
    live rows, k = ceil(u_live / c), raised only as far as keeps the items at
    most 2 chunk rows, while the items tile the whole reserved range."""
    u = _ceil_div(hi - lo, unit)
    if u <= 0:
        return []
    c = chunk // unit
    if hi_live is None:
        k = _ceil_div(u, c)
    else:
        u_live = _ceil_div(max(hi_live - lo, 0), unit)
        k = max(1, _ceil_div(u_live, c), _ceil_div(u, 2 * c))
    return [(lo + (i * u // k) * unit, min(lo + ((i + 1) * u // k) * unit, hi)) for i in range(k)]


def lpt_weight(tier: int, quant_block: int, old_bits: int) -> int:
    """Cost of one row of ``tier`` in the longest-first order (R-plan): its
    HBM bytes times 4 Qb / d."""
    return 16 * quant_block if tier == TIER_BF else old_bits * quant_block + 16


def plan(res: Reservation, chunk_bf: int, chunk_i8: int, lpt: bool, group_size: int = 0,
         page_size: int = 16, quant_block: int = 64, n_fixed=None, paths=None, node_len=None,
         old_bits: int = 8, live=None, chunk_group: int = 0):
    """Split plan, partial CSR and group-item member table (R-plan, R-group).

    Returns (work, part_off, gitems).  A work item is (r, h, tier, t0, t1,
    slot); a group item has r = -1 - g (g its index in gitems), slot -1, and
    gitems[g] lists its (request, slot) members, padded with (-1, -1) to
    GROUP_WIDTH."""
    B = len(res.L)
    H = len(res.cluster_of_head)
    grouping = group_size > 1 and paths is not None
    gitems_members = []   # per group item: member requests
    gitem_rows = []       # per group item: (h, t0, t1)
    shared_rows = [[0] * H for _ in range(B)]
    if grouping:
        for h in range(H):
            c = res.cluster_of_head[h]
            members = {}
            order = []
            for r in range(B):
                segs = shared_segments(res, r, c, page_size, quant_block, n_fixed, paths, node_len)
                if segs:
                    shared_rows[r][h] = segs[-1][2] * page_size
                for node, ja, jb, start in segs:
                    ident = (node, start, jb - ja, res.n_i8[r][h])
                    if ident not in members:
                        members[ident] = []
                        order.append((ident, ja))
                    members[ident].append(r)
            for ident, ja in order:
                mem = members[ident]
                lo, hi = ja * page_size, (ja + ident[2]) * page_size
                for k in range(0, len(mem), group_size):
                    grp = mem[k:k + group_size]
                    for t0, t1 in split_range(lo, hi, page_size, chunk_group or chunk_bf):
                        gitems_members.append(grp)
                        gitem_rows.append((h, t0, t1))
    # slots in natural (r, h) order: group memberships first, then own items
    member_of = {}
    for gi, grp in enumerate(gitems_members):
        h = gitem_rows[gi][0]
        for m in grp:
            member_of.setdefault((m, h), []).append(gi)
    gslot = [[-1] * len(grp) for grp in gitems_members]
    own = []
    part_off = []
    slot = 0
    for r in range(B):
        for h in range(H):
            part_off.append(slot)
            for gi in member_of.get((r, h), []):
                gslot[gi][gitems_members[gi].index(r)] = slot
                slot += 1
            for t, lo, n, unit, ch in ((TIER_I8, 0, res.n_i8[r][h], quant_block, chunk_i8),
                                       (TIER_BF, shared_rows[r][h], res.n_bf[r][h], page_size, chunk_bf)):
                n_live = None if live is None else (live.n_i8 if t == TIER_I8 else live.n_bf)[r][h]
                for t0, t1 in split_range(lo, n, unit, ch, n_live):
                    own.append((r, h, t, t0, t1, slot))
                    slot += 1
    part_off.append(slot)
    work = [(-1 - gi, h, TIER_BF, t0, t1, -1) for gi, (h, t0, t1) in enumerate(gitem_rows)] + own
    gitems = [[(m, gslot[gi][k]) for k, m in enumerate(grp)] + [(-1, -1)] * (GROUP_WIDTH - len(grp))
              for gi, grp in enumerate(gitems_members)]
    if lpt:  # group items stay ahead of the rest (R-plan)
        key = lambda it: (it[0] >= 0, -(it[4] - it[3]) * lpt_weight(it[2], quant_block, old_bits))
        work = sorted(work, key=key)
    return work, part_off, gitems


def build_tables(pool: Pool, res: Reservation, page_size: int, quant_block: int,
                 chunk_bf: int, chunk_i8: int, lpt: bool,
                 n_fixed=None, paths=None, node_len=None, group_size: int = 0,
                 gen_tokens: int = 0, old_bits: int = 8, chunk_group: int = 0) -> Tables:
    """Allocate pages and emit block tables, lengths and the plan (R-alloc,
    R-page, R-plan, R-group).  With gen_tokens > 0 pages and plan cover the
    capacity for that many appended rows (R-step); lengths stay the live ones
    and ring[r][c] is the bf16 page count of (r, c), the ring the bf16 tier
    turns over."""
    if chunk_bf < page_size or chunk_bf % page_size or chunk_i8 < quant_block or chunk_i8 % quant_block:
        raise OracleError("EINVAL", "chunk sizes")
    if not 0 <= group_size <= GROUP_WIDTH:
        raise OracleError("EINVAL", "group size")
    if chunk_group < 0 or chunk_group % page_size:
        raise OracleError("EINVAL", "group chunk")
    if gen_tokens < 0 or (gen_tokens > 0 and paths is not None):
        raise OracleError("EINVAL", "growth")
    B = len(res.L)
    C = len(res.cluster_size)
    H = len(res.cluster_of_head)
    live = res
    if gen_tokens > 0:
        res = capacity(res, gen_tokens)
    pages = allocate(pool, res, page_size, quant_block, n_fixed, paths, node_len)
    stride = [[max(len(pages[r][c][t]) for r in range(B)) for t in range(2)] for c in range(C)]
    bt = [[[pages[r][c][t] + [-1] * (stride[c][t] - len(pages[r][c][t])) for r in range(B)]
           for t in range(2)] for c in range(C)]
    lens = [[(live.n_i8[r][h], live.n_bf[r][h]) for h in range(H)] for r in range(B)]
    nf = [0] * B if n_fixed is None else list(n_fixed)
    work, part_off, gitems = plan(res, chunk_bf, chunk_i8, lpt, group_size, page_size, quant_block,
                                  nf, paths, node_len, old_bits,
                                  live if gen_tokens > 0 else None, chunk_group)
    t = Tables(bt, stride, lens, work, part_off, pages)
    t.gitems = gitems
    t.ring = [[len(pages[r][c][TIER_BF]) for c in range(C)] for r in range(B)]
    return t
