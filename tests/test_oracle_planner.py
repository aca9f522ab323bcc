"""Pins for the integer oracle (oracle/planner.py), independent of its code:
hand-worked golden tables, the radix lesson's printed block counts, a second
allocator built on a sorted free list, and invariants the rules imply."""
import bisect
import json
import os
import random

import numpy as np

import pytest

from oracle import planner as P
from workloads import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_hand_worked_budgets_clusters_tables_plan():
    g = _gold("planner_hand.json")["case_budgets"]
    res = P.reserve(g["head_rank"], g["ratio_hi_ppm"], g["ratio_lo_ppm"], g["n_clusters"],
                    g["recent_ppm"], g["quant_block"], g["n_comp"])
    assert res.budget == g["expect_budget"]
    assert res.cluster_of_head == g["expect_cluster_of_head"]
    assert res.slot_in_cluster == g["expect_slot_in_cluster"]
    assert res.cluster_size == g["expect_cluster_size"]
    pool = P.Pool([16, 16], [0, 0])
    t = P.build_tables(pool, res, g["page_size"], g["quant_block"], g["chunk_bf"], g["chunk_i8"], False)
    assert t.bt[0][P.TIER_BF] == g["expect_bt_c0_bf"]
    assert t.bt[1][P.TIER_BF] == g["expect_bt_c1_bf"]
    assert [list(w) for w in t.work] == g["expect_work"]
    assert t.part_off == g["expect_part_off"]
    work_lpt, off2, gi2 = P.plan(res, g["chunk_bf"], g["chunk_i8"], True)
    assert gi2 == []
    assert [w[5] for w in work_lpt] == g["expect_lpt_slots"]
    assert off2 == g["expect_part_off"]


def test_hand_worked_tier_split():
    g = _gold("planner_hand.json")["case_tiers"]
    res = P.reserve([0], 1_000_000, 1_000_000, 1, g["recent_ppm"], g["quant_block"],
                    [1] * len(g["L"]), [x - 1 for x in g["L"]])
    assert [row[0] for row in res.L] == g["L"]
    assert [row[0] for row in res.n_i8] == g["expect_n_i8"]
    assert [row[0] for row in res.n_bf] == g["expect_n_bf"]


def test_hand_worked_rounding_directions():
    """Two cases worked by hand where the rounding direction of the rules
    decides the result (R-rank, R-round, R-tier).

    Ratio band 0.5 .. 0.1 over H = 4 heads: rank 1 gets
    500000 - floor(400000 * 1 / 3) = 500000 - 133333 = 366667 ppm (rounding
    the step up would give 366666); for n = 3000 compressible tokens its
    budget is ceil(366667 * 3000 / 1e6) = ceil(1100.001) = 1101 (1100 with
    the other rounding).  Ranks 0, 2, 3: 500000, 233334, 100000 ppm ->
    1500, ceil(700.002) = 701, 300.

    Tier split of L = 585 rows keeping 12.5 % bf16 in 64-row blocks:
    n_bf0 = ceil(585 / 8) = ceil(73.125) = 74, the older 511 rows hold 7
    whole blocks, so n_i8 = 448 and n_bf = 137 (rounding n_bf0 down would
    leave 512 older rows: 8 blocks, n_i8 = 512)."""
    assert [P.ratio_ppm(k, 4, 500_000, 100_000) for k in range(4)] == [500_000, 366_667, 233_334, 100_000]
    res = P.reserve([0, 1, 2, 3], 500_000, 100_000, 1, 1_000_000, 64, [3000], None, None)
    assert res.budget == [[1500, 1101, 701, 300]]
    assert P.tier_split(585, 125_000, 64) == (448, 137)
    res = P.reserve([0], 1_000_000, 1_000_000, 1, 125_000, 64, [585], None, None)
    assert (res.n_i8, res.n_bf) == ([[448]], [[137]])


def test_tiered_128k_split_matches_workload_statement():
    g = _gold("planner_hand.json")["case_ttkv_128k"]
    res = P.reserve([0], 1_000_000, 1_000_000, 1, g["recent_ppm"], g["quant_block"], [g["L"]])
    assert res.n_i8[0][0] == g["expect_n_i8"] and res.n_bf[0][0] == g["expect_n_bf"]
    # newest 12.5% exactly, and the INT8 part is whole 64-token blocks
    assert res.n_bf[0][0] * 8 == g["L"] and res.n_i8[0][0] % 64 == 0


def _share_case():
    g = _gold("planner_hand.json")["case_share"]
    B = len(g["paths"])
    n_fixed = [sum(g["node_len"][n] for n in p) for p in g["paths"]]
    res = P.reserve([0, 1], 1_000_000, 1_000_000, 1, 1_000_000, g["quant_block"], g["n_comp"],
                    n_fixed, g["budget_override"])
    return g, res, n_fixed


def test_hand_worked_sharing_and_release():
    g, res, n_fixed = _share_case()
    assert res.L == g["expect_L"]
    need_bf, need_i8 = P.pages_needed(res, g["page_size"], g["quant_block"], n_fixed, g["paths"], g["node_len"])
    assert need_bf == [g["expect_pages_needed"]] and need_i8 == [0]
    pool = P.Pool([need_bf[0]], [0])
    t = P.build_tables(pool, res, g["page_size"], g["quant_block"], 4, 8, False, n_fixed, g["paths"], g["node_len"])
    assert t.bt[0][P.TIER_BF] == g["expect_bt"]
    for pid, cnt in g["expect_refcount"].items():
        assert pool.refcount(0, P.TIER_BF, int(pid)) == cnt
    P.release(pool, t.pages[0])
    a = g["after_release_r0_new_request"]
    res2 = P.reserve([0, 1], 1_000_000, 1_000_000, 1, 1_000_000, g["quant_block"], [a["n_comp"]],
                     [n_fixed[0]], a["budget"])
    pages = P.allocate(pool, res2, g["page_size"], g["quant_block"], [n_fixed[0]], [a["path"]], g["node_len"])
    assert pages[0][0][P.TIER_BF] == a["expect_pages"]


def test_enomem_rolls_back_completely():
    g, res, n_fixed = _share_case()
    pool = P.Pool([g["expect_pages_needed"] - 1], [0])
    before = pool._snapshot()
    with pytest.raises(P.OracleError) as e:
        P.build_tables(pool, res, g["page_size"], g["quant_block"], 4, 8, False, n_fixed, g["paths"], g["node_len"])
    assert e.value.code == "ENOMEM"
    assert pool._snapshot() == before


def test_radix_lesson_block_counts():
    g = _gold("radix_blocks.json")
    ps = g["page_size"]
    for e in g["blocks_to_hold"]:
        if not e["consistent"]:
            continue
        res = P.reserve([0], 1_000_000, 1_000_000, 1, 1_000_000, 64, [e["tokens"]])
        assert P.page_counts(res, ps, 64)[0][0][P.TIER_BF] == e["blocks"], e
    # whole pages of a page-aligned 500-token branch are the shared ones
    e = g["full_blocks_reused"][0]
    node_len = [2000, 500]
    res = P.reserve([0], 1_000_000, 1_000_000, 1, 1_000_000, 64, [30], [2500])
    shared = [j for j in range(P.page_counts(res, ps, 64)[0][0][P.TIER_BF])
              if P.share_key(res, 0, 0, P.TIER_BF, j, ps, 64, [2500], [[0, 1]], node_len) is not None]
    branch = [j for j in shared
              if P.share_key(res, 0, 0, P.TIER_BF, j, ps, 64, [2500], [[0, 1]], node_len)[2] == 1]
    assert len(branch) == e["blocks"]
    assert len(shared) - len(branch) == 2000 // ps


# ---------------------------------------------------------------- brute-force allocator
class SortedListPool:
    """Second allocator: a sorted Python list of free ids (bisect), refcount dict."""

    def __init__(self, cap):
        self.free = list(range(cap))
        self.ref = {}
        self.reg = {}
        self.key_of = {}

    def take(self, key):
        if key is not None and key in self.reg:
            pid = self.reg[key]
            self.ref[pid] += 1
            return pid
        pid = self.free.pop(0)
        self.ref[pid] = 1
        if key is not None:
            self.reg[key] = pid
            self.key_of[pid] = key
        return pid

    def drop(self, pid):
        self.ref[pid] -= 1
        if self.ref[pid] == 0:
            del self.ref[pid]
            bisect.insort(self.free, pid)
            k = self.key_of.pop(pid, None)
            if k is not None:
                del self.reg[k]


def test_allocator_matches_sorted_list_allocator_under_churn():
    rnd = random.Random(1234)
    node_len = [5, 3, 7, 2]
    ps = 4
    oracle_pool = P.Pool([400], [0])
    ref_pool = SortedListPool(400)
    live = []
    for step in range(60):
        if live and rnd.random() < 0.4:
            idx = rnd.randrange(len(live))
            pages_o, pages_r = live.pop(idx)
            P.release(oracle_pool, pages_o)
            for pid in pages_r:
                ref_pool.drop(pid)
            continue
        path = [0, rnd.choice([1, 2, 3])]
        nf = sum(node_len[n] for n in path)
        ncomp = rnd.randint(1, 9)
        b = [rnd.randint(1, ncomp), rnd.randint(1, ncomp)]
        res = P.reserve([0, 1], 1_000_000, 1_000_000, 1, 1_000_000, 8, [ncomp], [nf], b)
        pages = P.allocate(oracle_pool, res, ps, 8, [nf], [path], node_len)
        npg = -(-max(res.L[0]) // ps)
        expect = []
        for j in range(npg):
            key = None
            if j * ps + ps <= nf:
                acc, node = 0, None
                for n in path:
                    acc += node_len[n]
                    if j * ps + ps - 1 < acc:
                        node = n
                        break
                key = (node, j * ps)
            expect.append(ref_pool.take(key))
        assert pages[0][0][P.TIER_BF] == expect
        live.append((pages[0], expect))


# ---------------------------------------------------------------- invariants
def _small(name):
    over = {"tiny": {}, "llama8b": dict(B=6, ctx=("uniform", 300, 1200)),
            "ragged": dict(B=8, ctx=("loguniform", 100, 3000)),
            "tiered": dict(B=2, ctx=("fixed", 4000)),
            "radix": dict(B=12, share=dict(prefix=200, branch=50, n_branches=4, suffix=(8, 100)))}[name]
    return make_workload(name, **over)


@pytest.mark.parametrize("name", ["tiny", "llama8b", "ragged", "tiered", "radix"])
def test_invariants(name):
    w = _small(name)
    res = P.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                    w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    H, B = w.Hkv, w.B
    # budgets: bounded by the ratio band, non-increasing in rank
    for r in range(B):
        n = int(w.n_comp[r])
        for h in range(H):
            b = res.budget[r][h]
            assert 1 <= b <= n
            assert res.L[r][h] == b + int(w.n_fixed[r])
            if w.budget_override is None:
                assert -(-w.ratio_lo_ppm * n // 10**6) <= b <= -(-w.ratio_hi_ppm * n // 10**6)
        if w.budget_override is None:
            by_rank = [res.budget[r][h] for h in sorted(range(H), key=lambda h: w.head_rank[h])]
            assert by_rank == sorted(by_rank, reverse=True)
    # clusters: sizes sum to H, contiguous in rank, sizes differ by <= 1
    assert sum(res.cluster_size) == H and max(res.cluster_size) - min(res.cluster_size) <= 1
    order = sorted(range(H), key=lambda h: w.head_rank[h])
    assert [res.cluster_of_head[h] for h in order] == sorted(res.cluster_of_head)
    # tiers: INT8 part whole blocks, recent share kept in bf16
    for r in range(B):
        for h in range(H):
            assert res.n_i8[r][h] % w.quant_block == 0
            assert res.n_i8[r][h] + res.n_bf[r][h] == res.L[r][h]
            assert res.n_bf[r][h] * 10**6 >= res.L[r][h] * w.recent_ppm
    share = None if w.paths is None else (w.n_fixed, w.paths, w.node_len)
    need_bf, need_i8 = P.pages_needed(res, w.page_size, w.quant_block, *(share or ()))
    pool = P.Pool(need_bf, need_i8)
    t = P.build_tables(pool, res, w.page_size, w.quant_block, 4 * w.page_size, 2 * w.quant_block, True,
                       *(share or ()))
    # pool sized exactly: full afterwards; refcounts equal the number of referencing rows
    for c in range(w.n_clusters):
        for tt in (0, 1):
            assert pool.free_pages(c, tt) == 0
            counts = {}
            for r in range(B):
                for pid in t.pages[r][c][tt]:
                    counts[pid] = counts.get(pid, 0) + 1
            for pid, cnt in counts.items():
                assert pool.refcount(c, tt, pid) == cnt
                if cnt > 1:
                    assert (c, tt, pid) in pool.key_of
    # plan tiles every tier range exactly once; part_off is the CSR of slots
    seen = {}
    for (r, h, tier, t0, t1, slot) in t.work:
        assert 0 <= t0 < t1
        seen.setdefault((r, h, tier), []).append((t0, t1))
        assert t.part_off[r * H + h] <= slot < t.part_off[r * H + h + 1]
    assert sorted(s[5] for s in t.work) == list(range(len(t.work)))
    for r in range(B):
        for h in range(H):
            for tier, n in ((0, res.n_i8[r][h]), (1, res.n_bf[r][h])):
                iv = sorted(seen.get((r, h, tier), []))
                pos = 0
                for a, b in iv:
                    assert a == pos
                    pos = b
                assert pos == n
    # releasing everything restores an empty pool
    for r in range(B):
        P.release(pool, t.pages[r])
    for c in range(w.n_clusters):
        for tt in (0, 1):
            assert pool.free_pages(c, tt) == pool.cap[c][tt]
    assert not pool.registry


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("chunks", [(64, 128), (128, 192), (256, 64), (48, 320)])
def test_longest_first_order_follows_bytes_read(bits, chunks):
    """The longest-first order ranks items by the HBM bytes they read, priced
    from the page layout itself: a bf16 head page is ps rows of K and V at 2
    bytes a value; a quantised head block is qb rows of K and V codes at
    bits / 8 bytes a value plus one 2-byte scale per channel for K and for V.
    Equal bytes keep the natural (slot) order."""
    from fractions import Fraction
    w = make_workload("tiered", B=3, ctx=("fixed", 2900), recent_ppm=300_000)
    res = P.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                    w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    need_bf, need_i8 = P.pages_needed(res, w.page_size, w.quant_block)
    t = P.build_tables(P.Pool(need_bf, need_i8), res, w.page_size, w.quant_block, chunks[0], chunks[1], True,
                       old_bits=bits)
    d, ps, qb = w.d, w.page_size, w.quant_block
    per_row = {P.TIER_BF: Fraction(ps * 2 * d * 2, ps),
               P.TIER_I8: Fraction(qb * 2 * d * bits // 8 + 2 * d * 2, qb)}
    key = [(-(t1 - t0) * per_row[tier], slot) for (r, h, tier, t0, t1, slot) in t.work]
    assert key == sorted(key)
    # both tiers and several lengths take part, so the order is not trivial
    assert len({it[2] for it in t.work}) == 2 and len({it[4] - it[3] for it in t.work}) > 3


def test_rejects_bad_admission_inputs():
    with pytest.raises(P.OracleError):
        P.reserve([0, 0], 10, 10, 1, 10**6, 64, [5])
    with pytest.raises(P.OracleError):
        P.reserve([0, 1], 10, 20, 1, 10**6, 64, [5])
    with pytest.raises(P.OracleError):
        P.reserve([0, 1], 10, 10, 3, 10**6, 64, [5])
    with pytest.raises(P.OracleError):
        P.reserve([0, 1], 10, 10, 1, 10**6, 64, [0])
    with pytest.raises(P.OracleError):
        P.reserve([0, 1], 10, 10, 1, 10**6, 64, [5], None, [1, 6])


# ---------------------------------------------------------------- group items (R-group)
def test_hand_worked_group_items():
    g, res, n_fixed = _share_case()
    c = _gold("planner_hand.json")["case_group"]
    for lpt in (False, True):
        pool = P.Pool([g["expect_pages_needed"]], [0])
        t = P.build_tables(pool, res, g["page_size"], g["quant_block"], c["chunk_bf"], c["chunk_i8"], lpt,
                           n_fixed, g["paths"], g["node_len"], c["group_size"])
        assert t.part_off == c["expect_part_off"]
        assert [[list(x) for x in gi] for gi in t.gitems] == c["expect_gitems"]
        if not lpt:
            assert [list(w) for w in t.work] == c["expect_work"]
        else:
            order = ["g%d" % (-1 - w[0]) if w[0] < 0 else w[5] for w in t.work]
            assert order == c["expect_lpt_order"]
        # same pages as the ungrouped plan: grouping only changes the work list
        pool2 = P.Pool([g["expect_pages_needed"]], [0])
        t2 = P.build_tables(pool2, res, g["page_size"], g["quant_block"], c["chunk_bf"], c["chunk_i8"], lpt,
                            n_fixed, g["paths"], g["node_len"])
        assert t2.bt == t.bt and t2.gitems == []


def _group_check(w, res, t, gs):
    """Coverage, slot and page-identity invariants of a grouped plan."""
    H, B, ps = w.Hkv, w.B, w.page_size
    covered = {}
    slots = []
    for (r, h, tier, t0, t1, slot) in t.work:
        assert 0 <= t0 < t1
        if r >= 0:
            covered.setdefault((r, h, tier), []).append((t0, t1))
            slots.append(slot)
            assert t.part_off[r * H + h] <= slot < t.part_off[r * H + h + 1]
            continue
        assert slot == -1 and tier == P.TIER_BF
        mem = [m for m in t.gitems[-1 - r] if m[0] >= 0]
        assert 1 <= len(mem) <= gs and all(m == (-1, -1) for m in t.gitems[-1 - r][len(mem):])
        rs = [m[0] for m in mem]
        assert rs == sorted(set(rs))
        c = res.cluster_of_head[h]
        assert t0 % ps == 0 and t1 % ps == 0
        for (m, s) in mem:
            covered.setdefault((m, h, tier), []).append((t0, t1))
            slots.append(s)
            assert t.part_off[m * H + h] <= s < t.part_off[m * H + h + 1]
            # group rows lie in the fixed (shared) prefix of every member
            assert res.n_i8[m][h] + t1 <= w.n_fixed[m]
            assert res.n_i8[m][h] == res.n_i8[rs[0]][h]
        # every member reads the very same physical pages for these rows
        ref = t.bt[c][P.TIER_BF][rs[0]][t0 // ps:t1 // ps]
        for m in rs[1:]:
            assert t.bt[c][P.TIER_BF][m][t0 // ps:t1 // ps] == ref
    assert sorted(slots) == list(range(t.part_off[-1]))
    for r in range(B):
        for h in range(H):
            for tier, n in ((0, res.n_i8[r][h]), (1, res.n_bf[r][h])):
                pos = 0
                for a, b in sorted(covered.get((r, h, tier), [])):
                    assert a == pos
                    pos = b
                assert pos == n


@pytest.mark.parametrize("gs", [1, 2, 3, 8, 16, 32])
@pytest.mark.parametrize("recent_ppm", [1_000_000, 250_000])
def test_group_invariants(gs, recent_ppm):
    w = make_workload("radix", B=14, recent_ppm=recent_ppm,
                      share=dict(prefix=300, branch=70, n_branches=3, suffix=(8, 120)))
    res = P.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                    w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    share = (w.n_fixed, w.paths, w.node_len)
    need_bf, need_i8 = P.pages_needed(res, w.page_size, w.quant_block, *share)
    for chunk in (w.page_size, 3 * w.page_size, 64 * w.page_size):
        pool = P.Pool(need_bf, need_i8)
        t = P.build_tables(pool, res, w.page_size, w.quant_block, chunk, w.quant_block, True, *share, gs)
        _group_check(w, res, t, gs)
        n_group = sum(1 for it in t.work if it[0] < 0)
        assert n_group == len(t.gitems) and (n_group > 0) == (gs > 1)
        # the longest-first order keeps the group items ahead of all others
        assert all(it[0] < 0 for it in t.work[:n_group]) and all(it[0] >= 0 for it in t.work[n_group:])


# ---------------------------------------------------------------- decode-step growth (R-step)
def _n_bf_closed(L, rho, qb):
    """bf16 rows at length L written out: the recent share plus what is left
    of the older rows after whole blocks."""
    recent = -(-L * rho // 10**6)
    return recent + (L - recent) % qb


@pytest.mark.parametrize("rho,qb", [(125_000, 64), (300_000, 64), (10**6, 64), (0, 64), (500_000, 4), (1, 16)])
def test_append_steps_follow_the_tier_split(rho, qb):
    rnd = random.Random(rho + qb)
    for _ in range(40):
        L0, T = rnd.randint(1, 3000), rnd.randint(0, 400)
        i8, bf = P.tier_split(L0, rho, qb)
        aged = 0
        for k in range(1, T + 1):
            i8, bf, a = P.append_step(i8, bf, rho, qb)
            aged += a
            assert (i8, bf) == P.tier_split(L0 + k, rho, qb)
            assert bf == _n_bf_closed(L0 + k, rho, qb) and i8 % qb == 0
        assert aged * qb == i8 - P.tier_split(L0, rho, qb)[0]


def test_capacity_is_the_largest_split_on_the_way():
    res = P.reserve([0, 1, 2], 900_000, 300_000, 2, 125_000, 64, [700, 5000, 131], [17, 0, 3000])
    for T in (0, 1, 63, 64, 65, 1000):
        cap = P.capacity(res, T)
        for r in range(3):
            for h in range(3):
                L0 = res.L[r][h]
                assert cap.n_i8[r][h] == P.tier_split(L0 + T, 125_000, 64)[0]
                assert cap.n_bf[r][h] == max(_n_bf_closed(L, 125_000, 64) for L in range(L0, L0 + T + 1))


def test_incremental_blocks_equal_blocks_of_the_whole_sequence():
    """Quantising the oldest bf16 rows block by block as they age gives the
    same INT8 codes and scales as quantising the grown sequence at once."""
    from oracle import quant as Q
    rng = np.random.default_rng(5)
    qb, rho = 64, 125_000
    L0, T = 900, 700
    x = (rng.standard_normal((L0 + T, 16)) * 3).astype(np.float32)
    i8, bf = P.tier_split(L0, rho, qb)
    blocks = [Q.quantize_block(x[b * qb:(b + 1) * qb]) for b in range(i8 // qb)]
    for k in range(T):
        i8n, bf, aged = P.append_step(i8, bf, rho, qb)
        if aged:
            blocks.append(Q.quantize_block(x[i8:i8 + qb]))  # the oldest bf16 rows
        i8 = i8n
    qa, sa = Q.quantize_rows(x[:i8], qb)
    assert len(blocks) == i8 // qb
    assert np.array_equal(np.concatenate([b[0] for b in blocks]), qa)
    assert np.array_equal(np.stack([b[1] for b in blocks]), sa)


@pytest.mark.parametrize("T,chunks", [(1, (256, 512)), (128, (512, 1792)), (500, (256, 512)), (5000, (256, 512))])
def test_growth_plan_item_counts_follow_the_live_rows(T, chunks):
    """Room for T appended rows adds no items while it is small: each tier
    range of the growth plan has as many items as the same range of the plan
    of the live rows alone, unless that would make items longer than twice
    the chunk (then more, up to that bound); the items tile the reserved rows,
    near-equal in whole units, in order."""
    w = make_workload("tiered", B=3, ctx=("fixed", 2900), recent_ppm=200_000)
    res = P.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                    w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    cap = P.capacity(res, T)
    need_bf, need_i8 = P.pages_needed(cap, w.page_size, w.quant_block)
    g = P.build_tables(P.Pool(need_bf, need_i8), res, w.page_size, w.quant_block, chunks[0], chunks[1], False,
                       gen_tokens=T)
    need_bf, need_i8 = P.pages_needed(res, w.page_size, w.quant_block)
    plain = P.build_tables(P.Pool(need_bf, need_i8), res, w.page_size, w.quant_block, chunks[0], chunks[1], False)

    def ranges(t):
        out = {}
        for (r, h, tier, t0, t1, slot) in t.work:
            out.setdefault((r, h, tier), []).append((t0, t1))
        return out

    gi, pi = ranges(g), ranges(plain)
    grew = 0
    for (r, h, tier), its in gi.items():
        unit = w.page_size if tier == P.TIER_BF else w.quant_block
        c = (chunks[0] if tier == P.TIER_BF else chunks[1]) // unit
        full = cap.n_bf[r][h] if tier == P.TIER_BF else cap.n_i8[r][h]
        assert its[0][0] == 0 and its[-1][1] == full
        assert all(a[1] == b[0] for a, b in zip(its, its[1:]))
        sizes = [-(-(b - a) // unit) for a, b in its]
        assert max(sizes) - min(sizes) <= 1 and max(sizes) <= 2 * c
        n_plain = len(pi.get((r, h, tier), []))
        if len(its) != max(n_plain, 1):
            # only where keeping the live count would pass twice the chunk, and
            # then no more items than that bound needs
            u = -(-full // unit)
            assert u > 2 * c * max(n_plain, 1) and 2 * c * (len(its) - 1) < u
            grew += 1
    if T <= 500:
        assert grew == 0


def test_growth_tables_cover_capacity_and_keep_live_lengths():
    w = make_workload("tiered", B=2, ctx=("fixed", 3000))
    res = P.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                    w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    T = 500
    cap = P.capacity(res, T)
    need_bf, need_i8 = P.pages_needed(cap, w.page_size, w.quant_block)
    pool = P.Pool(need_bf, need_i8)
    t = P.build_tables(pool, res, w.page_size, w.quant_block, 256, 512, True, gen_tokens=T)
    for r in range(w.B):
        for h in range(w.Hkv):
            assert t.lens[r][h] == (res.n_i8[r][h], res.n_bf[r][h])
            assert t.ring[r][0] * w.page_size >= cap.n_bf[r][h]
    seen = {}
    for (r, h, tier, t0, t1, slot) in t.work:
        seen.setdefault((r, h, tier), []).append((t0, t1))
    for r in range(w.B):
        for h in range(w.Hkv):
            for tier, n in ((0, cap.n_i8[r][h]), (1, cap.n_bf[r][h])):
                assert sorted(seen[(r, h, tier)])[-1][1] == n
    with pytest.raises(P.OracleError):
        P.build_tables(P.Pool([100], [0]), res, w.page_size, w.quant_block, 256, 512, True,
                       [0, 0], [[0], [0]], [0], gen_tokens=T)


def test_hand_worked_group_chunk():
    """Group items cut with their own length (chunk_group), worked by hand.
    Three requests share one radix node of 40 rows (pages of 4 rows: one run
    of 10 shared pages per request), H = 1, own rows 5, 9 and 3; groups of 2.
    chunk_group 16 rows = 4 pages: k = ceil(10 / 4) = 3 items per group,
    starting at pages floor(i * 10 / 3) = 0, 3, 6, i.e. rows [0,12) [12,24)
    [24,40); groups {0, 1} then {2}.  Own items with chunk_bf 8 rows = 2
    pages: r0 rows 40..45 (2 pages, 1 item), r1 40..49 (3 pages: 2 items
    starting at pages 0 and floor(3/2) = 1, i.e. 40..44, 44..49), r2 40..43.
    Slots per request: its three memberships, then its own items."""
    n_comp = [5, 9, 3]
    res = P.reserve([0], 1_000_000, 1_000_000, 1, 1_000_000, 8, n_comp, [40, 40, 40], None)
    pool = P.Pool([60], [0])
    t = P.build_tables(pool, res, 4, 8, 8, 8, False, [40, 40, 40], [[0], [0], [0]], [40], group_size=2,
                       chunk_group=16)
    assert [list(w) for w in t.work] == [
        [-1, 0, 1, 0, 12, -1], [-2, 0, 1, 12, 24, -1], [-3, 0, 1, 24, 40, -1],
        [-4, 0, 1, 0, 12, -1], [-5, 0, 1, 12, 24, -1], [-6, 0, 1, 24, 40, -1],
        [0, 0, 1, 40, 45, 3], [1, 0, 1, 40, 44, 7], [1, 0, 1, 44, 49, 8], [2, 0, 1, 40, 43, 12]]
    assert t.part_off == [0, 4, 9, 13]
    pad = [(-1, -1)] * 30
    assert t.gitems == [[(0, 0), (1, 4)] + pad, [(0, 1), (1, 5)] + pad, [(0, 2), (1, 6)] + pad,
                        [(2, 9)] + [(-1, -1)] * 31, [(2, 10)] + [(-1, -1)] * 31, [(2, 11)] + [(-1, -1)] * 31]
    # chunk_group 0 takes chunk_bf for the group items too: 5 items per group
    pool2 = P.Pool([60], [0])
    t2 = P.build_tables(pool2, res, 4, 8, 8, 8, False, [40, 40, 40], [[0], [0], [0]], [40], group_size=2)
    assert [tuple(w[3:5]) for w in t2.work if w[0] < 0][:5] == [(0, 8), (8, 16), (16, 24), (24, 32), (32, 40)]
    with pytest.raises(P.OracleError):
        P.build_tables(P.Pool([60], [0]), res, 4, 8, 8, 8, False, [40, 40, 40], [[0], [0], [0]], [40],
                       group_size=2, chunk_group=6)


def test_hand_worked_growth_plan():
    """A plan with room for appended rows (R-step), worked by hand.  One
    request, H = 1, recent share 50 %, Qb 8, pages of 4 rows, L0 = 30:
    n_bf0 = ceil(15) = 15, old 15 -> n_i8 8, n_bf 22.  Six appends:
      L 31: n_bf0 16, old 15 -> i8 8, bf 23
      L 32: n_bf0 16, old 16 -> i8 16: rows 8..15 age, bf 24 - 8 = 16
      L 33..36: old 16..18 -> i8 16, bf 17, 18, 19, 20
    Capacity: INT8 rows of the final length (16) and the most bf16 rows on
    the way (23): 2 INT8 pages, ceil(23 / 4) = 6 bf16 pages (the ring).
    Plan, chunk 8 rows in both tiers: INT8 [0, 16) is 2 blocks, 1 live:
    k = max(1, ceil(1 / 1), ceil(2 / 2)) = 1 item [0, 16); bf16 [0, 23) is 6
    pages, 6 live (22 rows): k = max(1, ceil(6 / 2), ceil(6 / 4)) = 3 items at
    pages 0, 2, 4: [0, 8) [8, 16) [16, 23).  Live lengths stay (8, 22)."""
    res = P.reserve([0], 1_000_000, 1_000_000, 1, 500_000, 8, [30], None, None)
    assert (res.n_i8[0][0], res.n_bf[0][0]) == (8, 22)
    steps, state = [], (8, 22)
    for _ in range(6):
        i8, bf, aged = P.append_step(state[0], state[1], 500_000, 8)
        steps.append((i8, bf, aged))
        state = (i8, bf)
    assert steps == [(8, 23, False), (16, 16, True), (16, 17, False), (16, 18, False), (16, 19, False),
                     (16, 20, False)]
    cap = P.capacity(res, 6)
    assert (cap.n_i8[0][0], cap.n_bf[0][0]) == (16, 23)
    assert P.pages_needed(cap, 4, 8) == ([6], [2])
    pool = P.Pool([6], [2])
    t = P.build_tables(pool, res, 4, 8, 8, 8, False, gen_tokens=6)
    assert [list(w) for w in t.work] == [[0, 0, 0, 0, 16, 0], [0, 0, 1, 0, 8, 1], [0, 0, 1, 8, 16, 2],
                                         [0, 0, 1, 16, 23, 3]]
    assert t.part_off == [0, 4]
    assert t.lens[0][0] == (8, 22)
    assert t.ring == [[6]]
    assert pool.free_pages(0, 0) == 0 and pool.free_pages(0, 1) == 0
