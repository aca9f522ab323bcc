"""Host planner of libtg.so (C++) against the integer oracle, bit for bit.

Runs on the CPU: only host entry points are called.  Also checks that the
library loads and exports every function include/tg.h declares."""
import os
import random
import re

import numpy as np
import pytest

from oracle import planner as P
from workloads import make_workload
from workloads.gen import share_arrays

tg = pytest.importorskip("non_uniform_paged_amd")
from non_uniform_paged_amd import _lib  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tg.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(tg_[a-z_0-9]+)\s*\(", text))
    assert len(names) >= 14
    L = _lib.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)


def _both(w, chunk_bf=512, chunk_i8=1024, lpt=True, slack=0):
    res_o = P.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                      w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    res_g = tg.tg_reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                          w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    return res_o, res_g


def _compare_reservation(res_o, res_g):
    assert np.array_equal(res_g.budget, np.array(res_o.budget))
    assert np.array_equal(res_g.length, np.array(res_o.L))
    assert np.array_equal(res_g.n_i8, np.array(res_o.n_i8))
    assert np.array_equal(res_g.n_bf, np.array(res_o.n_bf))
    assert list(res_g.cluster_of_head) == res_o.cluster_of_head
    assert list(res_g.slot_in_cluster) == res_o.slot_in_cluster
    assert list(res_g.cluster_size) == res_o.cluster_size


def _share(w):
    if w.paths is None:
        return None, ()
    n_nodes, ids, node_len = share_arrays(w)
    return tg.Share(n_nodes, ids, node_len), (w.n_fixed, w.paths, w.node_len)


def _gitems_of(t_o):
    return np.array(t_o.gitems, dtype=np.int32).reshape(-1, 32, 2)


def _tables_parity(w, chunk_bf=512, chunk_i8=1024, lpt=True, slack=3, group_size=0, gen=0, chunk_group=0):
    res_o, res_g = _both(w)
    _compare_reservation(res_o, res_g)
    share, sh_o = _share(w)
    need_bf, need_i8 = P.pages_needed(P.capacity(res_o, gen), w.page_size, w.quant_block, *sh_o)
    sizes = tg.tg_size_tables(res_g, w.page_size, w.quant_block, share, chunk_bf, chunk_i8, lpt, group_size, gen,
                              chunk_group)
    assert [row[1] for row in sizes["pages_needed"]] == need_bf
    assert [row[0] for row in sizes["pages_needed"]] == need_i8
    pool_g = tg.Pool(res_g.cluster_size, w.d, w.page_size, w.quant_block,
                     [x + slack for x in need_bf], [x + slack for x in need_i8], old_bits=w.old_bits)
    pool_o = P.Pool([x + slack for x in need_bf], [x + slack for x in need_i8])
    t_g = tg.tg_build_tables(pool_g, res_g, share, chunk_bf, chunk_i8, lpt, group_size, gen, chunk_group)
    t_o = P.build_tables(pool_o, res_o, w.page_size, w.quant_block, chunk_bf, chunk_i8, lpt, *sh_o,
                         **({"group_size": group_size} if sh_o else {"gen_tokens": gen}), old_bits=w.old_bits,
                         chunk_group=chunk_group)
    for c in range(w.n_clusters):
        for t in range(2):
            assert t_g.stride[c][t] == t_o.stride[c][t]
            if t_o.stride[c][t]:
                assert np.array_equal(t_g.bt[c][t], np.array(t_o.bt[c][t], dtype=np.int32)), (c, t)
            assert pool_g.free_pages(c, t) == pool_o.free_pages(c, t)
    assert np.array_equal(t_g.len, np.array(t_o.lens, dtype=np.int32))
    assert np.array_equal(t_g.plan, np.array(t_o.work, dtype=np.int32).reshape(-1, 6))
    assert list(t_g.part_off) == t_o.part_off
    assert t_g.n_slots == t_o.part_off[-1] and t_g.n_gitems == len(t_o.gitems)
    assert np.array_equal(t_g.gitems, _gitems_of(t_o))
    assert np.array_equal(t_g.ring, np.array(t_o.ring, dtype=np.int32))
    tg.tg_check_tables(pool_g, res_g, t_g)  # the library's own consistency check agrees
    return res_o, res_g, pool_o, pool_g, t_o, t_g


@pytest.mark.parametrize("name,gen", [("tiny", 37), ("llama8b", 256), ("tiered", 1000), ("ragged", 64)])
def test_growth_tables_bit_exact(name, gen):
    w = make_workload(name)
    res_o, res_g, pool_o, pool_g, t_o, t_g = _tables_parity(w, gen=gen)
    assert np.array_equal(t_g.len[..., 0], np.array(res_o.n_i8)) and np.array_equal(t_g.len[..., 1], np.array(res_o.n_bf))


@pytest.mark.parametrize("name,gs", [("tiny", 0), ("llama8b", 0), ("ragged", 0), ("tiered", 0), ("tiered4", 0),
                                     ("radix", 0),
                                     ("radix", 2), ("radix", 8), ("radix", 32)])
def test_full_size_configs_bit_exact(name, gs):
    w = make_workload(name)
    res_o, res_g, pool_o, pool_g, t_o, t_g = _tables_parity(w, group_size=gs)
    if gs > 1:
        assert t_g.n_gitems > 0
    # refcounts agree page by page on a sample of pages
    for c in range(w.n_clusters):
        for t in range(2):
            cap = pool_g.capacity(c, t)
            for pid in range(0, cap, max(1, cap // 97)):
                assert pool_g.refcount(c, t, pid) == pool_o.refcount(c, t, pid)


@pytest.mark.parametrize("chunk_bf,chunk_group", [(256, 1008), (128, 0), (768, 512)])
def test_radix_group_chunk_bit_exact(chunk_bf, chunk_group):
    """Group items cut with their own length (chunk_group) while the
    requests' own items use chunk_bf, at full radix size."""
    w = make_workload("radix")
    res_o, res_g, pool_o, pool_g, t_o, t_g = _tables_parity(w, chunk_bf=chunk_bf, group_size=32,
                                                           chunk_group=chunk_group)
    assert t_g.n_gitems > 0


def test_release_and_reallocation_bit_exact():
    w = make_workload("radix", B=24, share=dict(prefix=100, branch=37, n_branches=3, suffix=(5, 90)))
    res_o, res_g, pool_o, pool_g, t_o, t_g = _tables_parity(w, chunk_bf=64, slack=40)
    rnd = random.Random(7)
    order = list(range(w.B))
    rnd.shuffle(order)
    for r in order[:15]:
        tg.tg_release(pool_g, t_g, r)
        P.release(pool_o, t_o.pages[r])
        for c in range(w.n_clusters):
            for t in range(2):
                assert pool_g.free_pages(c, t) == pool_o.free_pages(c, t)
        tg.tg_check_tables(pool_g, res_g, t_g)  # released rows are skipped, the rest stays consistent
    with pytest.raises(tg.TGError) as e:
        tg.tg_release(pool_g, t_g, order[0])
    assert e.value.name == "TG_EINVAL"
    # a second batch lands in the holes, lowest id first, identically
    w2 = make_workload("radix", B=9, share=dict(prefix=100, branch=37, n_branches=3, suffix=(5, 90)))
    res2_o, res2_g = _both(w2)
    share2, sh2_o = _share(w2)
    t2_g = tg.tg_build_tables(pool_g, res2_g, share2, 64, 1024, True)
    t2_o = P.build_tables(pool_o, res2_o, w2.page_size, w2.quant_block, 64, 1024, True, *sh2_o)
    for c in range(w2.n_clusters):
        assert np.array_equal(t2_g.bt[c][1], np.array(t2_o.bt[c][1], dtype=np.int32))


def test_randomised_small_cases_bit_exact():
    rnd = random.Random(2026)
    for case in range(120):
        H = rnd.choice([1, 2, 3, 4, 5, 8])
        C = rnd.randint(1, H)
        B = rnd.randint(1, 5)
        hi = rnd.randint(1, 10**6)
        lo = rnd.randint(1, hi)
        qb = rnd.choice([4, 8, 64])
        ps = rnd.choice([2, 4, 16])
        recent = rnd.choice([0, 1, 125_000, 500_000, 10**6])
        rank = list(range(H))
        rnd.shuffle(rank)
        n_comp = [rnd.randint(1, 300) for _ in range(B)]
        use_share = rnd.random() < 0.5
        node_len = [rnd.randint(0, 40) for _ in range(4)]
        paths = [[0, rnd.randint(1, 3)] for _ in range(B)] if use_share else None
        n_fixed = [sum(node_len[n] for n in p) for p in paths] if use_share else [0] * B
        override = [rnd.randint(1, n) for n in n_comp for _ in range(H)] if rnd.random() < 0.3 else None
        res_o = P.reserve(rank, hi, lo, C, recent, qb, n_comp, n_fixed, override)
        res_g = tg.tg_reserve(rank, hi, lo, C, recent, qb, n_comp, n_fixed, override)
        _compare_reservation(res_o, res_g)
        sh_o = (n_fixed, paths, node_len) if use_share else ()
        share = tg.Share([2] * B, [x for p in paths for x in p], node_len) if use_share else None
        chunk_bf = ps * rnd.randint(1, 6)
        chunk_i8 = qb * rnd.randint(1, 3)
        lpt = rnd.random() < 0.5
        gs = rnd.choice([0, 1, 2, 3, 16, 32])
        cg = ps * rnd.randint(1, 8) if rnd.random() < 0.5 else 0
        gen = 0 if use_share else rnd.choice([0, 0, 1, 70, 300])
        grp = {"group_size": gs} if use_share else {"gen_tokens": gen}
        need_bf, need_i8 = P.pages_needed(P.capacity(res_o, gen), ps, qb, *sh_o)
        cap_bf = [n + rnd.randint(-1, 2) for n in need_bf]
        cap_i8 = [n + rnd.randint(-1, 2) for n in need_i8]
        cap_bf = [max(0, x) for x in cap_bf]
        cap_i8 = [max(0, x) for x in cap_i8]
        bits = rnd.choice([8, 4])
        pool_g = tg.Pool(res_g.cluster_size, 16, ps, qb, cap_bf, cap_i8, old_bits=bits)
        pool_o = P.Pool(cap_bf, cap_i8)
        try:
            t_o = P.build_tables(pool_o, res_o, ps, qb, chunk_bf, chunk_i8, lpt, *sh_o, **grp, old_bits=bits,
                                 chunk_group=cg)
        except P.OracleError as e:
            assert e.code == "ENOMEM"
            with pytest.raises(tg.TGError) as ge:
                tg.tg_build_tables(pool_g, res_g, share, chunk_bf, chunk_i8, lpt, gs, gen, cg)
            assert ge.value.name == "TG_ENOMEM"
            for c in range(C):
                for t in range(2):
                    assert pool_g.free_pages(c, t) == pool_g.capacity(c, t)
            continue
        t_g = tg.tg_build_tables(pool_g, res_g, share, chunk_bf, chunk_i8, lpt, gs, gen, cg)
        assert np.array_equal(t_g.ring, np.array(t_o.ring, dtype=np.int32)), case
        for c in range(C):
            for t in range(2):
                if t_o.stride[c][t]:
                    assert np.array_equal(t_g.bt[c][t], np.array(t_o.bt[c][t], dtype=np.int32)), case
        assert np.array_equal(t_g.plan, np.array(t_o.work, dtype=np.int32).reshape(-1, 6)), case
        assert list(t_g.part_off) == t_o.part_off
        assert np.array_equal(t_g.gitems, _gitems_of(t_o)), case
        tg.tg_check_tables(pool_g, res_g, t_g)


def test_error_codes():
    w = make_workload("tiny")
    with pytest.raises(tg.TGError) as e:
        tg.tg_reserve([0, 0], 10, 10, 1, 10**6, 64, [5])
    assert e.value.name == "TG_EINVAL"
    with pytest.raises(tg.TGError) as e:
        tg.tg_reserve([0, 1], 10, 10, 1, 10**6, 64, [2**31 - 5], [10])
    assert e.value.name == "TG_EOVERFLOW"
    res = tg.tg_reserve(w.head_rank, 10**6, 10**6, 2, 10**6, 64, w.n_comp)
    with pytest.raises(tg.TGError) as e:
        tg.tg_size_tables(res, 16, 64, None, chunk_bf=24)
    assert e.value.name == "TG_EINVAL"
    with pytest.raises(tg.TGError) as e:
        tg.Pool([1, 1], 64, 0, 64, [1, 1], [0, 0])
    assert e.value.name == "TG_EINVAL"
    # share paths inconsistent with n_fixed
    with pytest.raises(tg.TGError) as e:
        tg.tg_size_tables(res, 16, 64, tg.Share([1, 1], [0, 0], [5]))
    assert e.value.name == "TG_EINVAL"
    with pytest.raises(tg.TGError) as e:
        tg.tg_size_tables(res, 16, 64, None, group_size=33)
    assert e.value.name == "TG_EINVAL"
    with pytest.raises(tg.TGError) as e:
        tg.tg_size_tables(res, 16, 64, None, gen_tokens=-1)
    assert e.value.name == "TG_EINVAL"
    # growth is not combined with shared pages
    wr = make_workload("radix", B=3, share=dict(prefix=40, branch=10, n_branches=2, suffix=(5, 30)))
    rr = tg.tg_reserve(wr.head_rank, wr.ratio_hi_ppm, wr.ratio_lo_ppm, wr.n_clusters, wr.recent_ppm,
                       wr.quant_block, wr.n_comp, wr.n_fixed, wr.budget_override)
    n_nodes, ids, node_len = share_arrays(wr)
    with pytest.raises(tg.TGError) as e:
        tg.tg_size_tables(rr, 16, 64, tg.Share(n_nodes, ids, node_len), gen_tokens=8)
    assert e.value.name == "TG_EINVAL"


def test_rounding_directions_match_the_hand_worked_cases():
    """The library's reservation on the oracle pins' hand-worked rounding
    cases (rank step floored, budget and bf16 share ceiled)."""
    r = tg.tg_reserve([0, 1, 2, 3], 500_000, 100_000, 1, 1_000_000, 64, [3000], None, None)
    assert r.budget.tolist() == [[1500, 1101, 701, 300]]
    r = tg.tg_reserve([0], 1_000_000, 1_000_000, 1, 125_000, 64, [585], None, None)
    assert (r.n_i8.tolist(), r.n_bf.tolist()) == ([[448]], [[137]])


def test_binding_signatures_follow_the_header():
    """Every ctypes signature has the header prototype's number of
    parameters, and a return type of the same size and kind, so that no
    argument is dropped or widened between Python and the library."""
    import ctypes
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    protos = {}
    for m in re.finditer(r"\b([A-Za-z_][A-Za-z_0-9 ]*?\**)\s*\b(tg_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        ret, name, params = m.group(1).strip(), m.group(2), " ".join(m.group(3).split())
        n = 0 if params in ("", "void") else params.count(",") + 1
        protos[name] = (ret, n)
    kinds = {"int": ctypes.c_int, "int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "size_t": ctypes.c_size_t,
             "void": None, "const char*": ctypes.c_char_p}
    assert set(protos) == set(_lib.SIGNATURES), set(protos) ^ set(_lib.SIGNATURES)
    for name, (ret, n) in protos.items():
        res, args = _lib.SIGNATURES[name]
        assert len(args) == n, (name, n, len(args))
        want = kinds[ret.replace(" *", "*")]
        if want is None:
            assert res is None, name
        else:
            assert res is not None and ctypes.sizeof(res) == ctypes.sizeof(want), (name, ret, res)


def test_hand_worked_growth_plan_from_c():
    """The library's tables for the hand-worked growth case of
    test_oracle_planner.test_hand_worked_growth_plan: one request, L0 = 30,
    recent 50 %, Qb 8, pages of 4 rows, room for 6 appended rows."""
    api = tg
    res = api.tg_reserve([0], 1_000_000, 1_000_000, 1, 500_000, 8, [30])
    sizes = api.tg_size_tables(res, 4, 8, None, 8, 8, False, 0, 6)
    assert [list(x) for x in sizes["pages_needed"]] == [[2, 6]]
    pool = api.Pool(res.cluster_size, 64, 4, 8, [6], [2])
    t = api.tg_build_tables(pool, res, None, 8, 8, False, 0, 6)
    assert t.plan.tolist() == [[0, 0, 0, 0, 16, 0], [0, 0, 1, 0, 8, 1], [0, 0, 1, 8, 16, 2], [0, 0, 1, 16, 23, 3]]
    assert t.part_off.tolist() == [0, 4]
    assert t.len.reshape(-1).tolist() == [8, 22]
    assert t.ring.tolist() == [[6]]
    assert pool.free_pages(0, 0) == 0 and pool.free_pages(0, 1) == 0
