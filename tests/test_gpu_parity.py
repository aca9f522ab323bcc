"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerance (stated by the workload specification): every fp32 output element
satisfies |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|.  Integer work (budgets,
tables, INT8 codes and scales) must match bit for bit."""
import sys

import numpy as np
import pytest

from oracle import attention as A
from oracle import quant as Q
from workloads import make_workload

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _prep(w, **kw):
    from non_uniform_paged_amd.runner import Prepared
    return Prepared(w, **kw)


def _check(got, ref, pairs, G, what):
    worst_abs = worst_rel = 0.0
    for r, h in pairs:
        g = got[r, h * G:(h + 1) * G]
        o = ref[r, h * G:(h + 1) * G]
        err = np.abs(g - o)
        assert np.all(np.isfinite(g)), (what, r, h)
        bad = err > ATOL + RTOL * np.abs(o)
        assert not bad.any(), f"{what}: (r={r}, h={h}) max err {err.max():.3g}"
        worst_abs = max(worst_abs, float(err.max()))
        big = np.abs(o) >= 1e-3
        if big.any():
            worst_rel = max(worst_rel, float((err[big] / np.abs(o[big])).max()))
    _say(f"{what}: max-abs {worst_abs:.3g} max-rel {worst_rel:.3g} over {len(pairs)} (r,h)")
    return worst_abs, worst_rel


def _run_and_compare(w, pairs=None, what="", **kw):
    _say(f"case {what or w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} C={w.n_clusters} {kw}")
    p = _prep(w, **kw)
    p.step()
    got = p.output()
    res_o = A.reserve_for(w)
    assert np.array_equal(p.res.length, np.array(res_o.L))
    if pairs is None:
        pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
    ref = A.decode(w, res_o, pairs)
    _check(got, ref, pairs, w.Hq // w.Hkv, what or w.name)
    return p, got


SMALL = {
    "tiny": {},
    "llama8b": dict(B=4, ctx=("uniform", 300, 1500)),
    "ragged": dict(B=8, ctx=("loguniform", 64, 4000)),
    "tiered": dict(B=2, ctx=("fixed", 5000)),
    "radix": dict(B=10, share=dict(prefix=200, branch=50, n_branches=4, suffix=(8, 300))),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_configs_all_outputs(name):
    _need_gpu()
    _run_and_compare(make_workload(name, **SMALL[name]), chunk_bf=64, chunk_i8=128)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_configs_default_plan(name):
    _need_gpu()
    _run_and_compare(make_workload(name, **SMALL[name]))


def _sample_pairs(w, k, seed):
    rnd = np.random.default_rng(seed)
    idx = rnd.choice(w.B * w.Hkv, size=min(k, w.B * w.Hkv), replace=False)
    return sorted((int(i) // w.Hkv, int(i) % w.Hkv) for i in idx)


@pytest.mark.parametrize("name,k", [("llama8b", 24), ("ragged", 24), ("tiered", 8), ("tiered4", 8),
                                    ("radix", 24)])
def test_full_size_configs_sampled(name, k):
    """Full sizes in the benchmark's launch configuration (its plan item
    lengths and group size), sampled (r, h) pairs against the oracle."""
    _need_gpu()
    from non_uniform_paged_amd.runner import PLAN_CHUNKS
    w = make_workload(name)
    chunk_bf, chunk_i8 = PLAN_CHUNKS[name]
    _run_and_compare(w, pairs=_sample_pairs(w, k, 11), what=f"{name}-full", chunk_bf=chunk_bf, chunk_i8=chunk_i8)


@pytest.mark.parametrize("name,k", [("ragged", 12), ("tiered", 6)])
def test_full_size_with_one_page_items(name, k):
    """The largest plans at full size: every item one bf16 page or one INT8
    block (ragged: 428369 items and partials, 107093 workgroups, ~209
    partials a pair through the four-wavefront merge), sampled pairs
    against the oracle."""
    _need_gpu()
    w = make_workload(name)
    p, _ = _run_and_compare(w, pairs=_sample_pairs(w, k, 5), what=f"{name}-one-page-items", chunk_bf=16,
                            chunk_i8=64)
    assert p.tables.n_items == p.tables.n_slots and p.tables.n_items > (400_000 if name == "ragged" else 90_000)


def test_single_row_returns_value_row_exactly():
    torch = _need_gpu()
    w = make_workload("llama8b", B=3, ctx=("uniform", 20, 40), budget=None)
    w.budget_override = np.ones(w.B * w.Hkv, np.int32)
    p = _prep(w)
    p.step()
    got = p.output()
    for r in range(w.B):
        for h in range(w.Hkv):
            K16, V16 = w.logical_kv(r, h, 1)
            v = A.bf16_to_f64(V16)[0].astype(np.float32)
            for g in range(4):
                assert np.array_equal(got[r, 4 * h + g], v)


def test_page_placement_invariance_bitwise():
    _need_gpu()
    w = make_workload("ragged", B=6, ctx=("loguniform", 100, 3000))
    a = _prep(w, chunk_bf=128)
    a.step()
    ga = a.output()
    b = _prep(w, chunk_bf=128, shift_pages=37)
    assert any((b.tables.bt[c][1] != a.tables.bt[c][1]).any() for c in range(w.n_clusters))
    b.step()
    gb = b.output()
    assert np.array_equal(ga, gb)


@pytest.mark.parametrize("C", [1, 2, 8])
def test_cluster_count_invariance(C):
    _need_gpu()
    w = make_workload("llama8b", B=3, ctx=("uniform", 400, 900), n_clusters=C)
    _run_and_compare(w, what=f"llama8b-C{C}")


@pytest.mark.parametrize("chunk", [16, 48, 4096])
def test_split_invariance(chunk):
    _need_gpu()
    w = make_workload("llama8b", B=2, ctx=("uniform", 600, 1200))
    _run_and_compare(w, what=f"chunk{chunk}", chunk_bf=chunk, lpt=chunk != 48)


def test_uniform_budgets_dense():
    _need_gpu()
    w = make_workload("llama8b", B=2, ctx=("uniform", 300, 700), ratio_ppm=(10**6, 10**6), n_clusters=1)
    _run_and_compare(w, what="dense")


def _read_i8_pages(p, r, h):
    """Codes and scales of (r, h)'s INT8 rows, read back from the device pool
    through the layout include/tg.h documents."""
    w = p.w
    d, qb = w.d, w.quant_block
    cl = int(p.res.cluster_of_head[h])
    s = int(p.res.slot_in_cluster[h])
    n8 = int(p.res.n_i8[r, h])
    hb = 2 * qb * d + 4 * d
    pool = p.cache.pools[cl][0].cpu().numpy()
    kq, vq, ks, vs = [], [], [], []
    t = np.arange(qb)[:, None]
    c = np.arange(d)[None, :]
    nl = d // 64
    koff = ((t >> 4) * nl + (c >> 6)) * 1024 + (((c >> 3) & 3) * 16 + (t & 15)) * 16 + ((c >> 5) & 1) * 8 + (c & 7)
    voff = ((t >> 4) * nl + (c >> 6)) * 1024 + (((t >> 2) & 3) * 16 + (c & 15)) * 16 + ((c >> 4) & 3) * 4 + (t & 3)
    assert sorted(koff.ravel()) == list(range(qb * d)) and sorted(voff.ravel()) == list(range(qb * d))
    for j in range(n8 // qb):
        pid = int(p.tables.bt[cl][0][r, j])
        base = p.cache.slot_offset(cl, 0, pid, s, p.pool)
        blk = pool[base:base + hb]
        kq.append(blk[:qb * d].view(np.int8)[koff])
        vq.append(blk[qb * d:2 * qb * d].view(np.int8)[voff])
        ks.append(blk[2 * qb * d:2 * qb * d + 2 * d].view(np.float16))
        vs.append(blk[2 * qb * d + 2 * d:].view(np.float16))
    return np.concatenate(kq), np.concatenate(vq), np.stack(ks), np.stack(vs)


def test_int8_codes_and_scales_bit_exact():
    _need_gpu()
    w = make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 3000))
    p = _prep(w)
    for r in range(w.B):
        for h in range(w.Hkv):
            n8 = int(p.res.n_i8[r, h])
            K16, V16 = w.logical_kv(r, h, int(p.res.length[r, h]))
            kq, vq, ks, vs = _read_i8_pages(p, r, h)
            from workloads import bf16_bits_to_f32
            okq, oks = Q.quantize_rows(bf16_bits_to_f32(K16[:n8]), 64)
            ovq, ovs = Q.quantize_rows(bf16_bits_to_f32(V16[:n8]), 64)
            assert np.array_equal(kq, okq) and np.array_equal(vq, ovq)
            assert np.array_equal(ks.view(np.uint16), oks.view(np.uint16))
            assert np.array_equal(vs.view(np.uint16), ovs.view(np.uint16))


class _ExactRows:
    """Rows that are integer multiples of 2^-5 with a +-127 code in the first
    row of every 64-row block, so symmetric absmax INT8 reproduces them
    exactly (step 2^-5)."""

    @staticmethod
    def make(base, recent_ppm):
        import dataclasses
        from workloads.gen import Workload, bf16_round

        class W(Workload):
            def stream_rows(self, key, n):
                tag, a, h = key
                rr = np.random.default_rng([0 if tag == "seq" else 1, a, h])
                k = rr.integers(-127, 128, size=(n, self.d))
                v = rr.integers(-127, 128, size=(n, self.d))
                k[::64] = 127
                v[::64] = -127
                return (bf16_round((k * 2.0 ** -5).astype(np.float32)),
                        bf16_round((v * 2.0 ** -5).astype(np.float32)))

        fields = {f.name: getattr(base, f.name) for f in dataclasses.fields(base)}
        fields["recent_ppm"] = recent_ppm
        return W(**fields)


def test_int8_tier_equals_bf16_tier_on_exact_values():
    _need_gpu()
    base = make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 1024))
    a = _prep(_ExactRows.make(base, 10**6))
    b = _prep(_ExactRows.make(base, 125_000))
    assert int(b.res.n_i8.min()) > 0 and int(a.res.n_i8.max()) == 0
    a.step()
    b.step()
    ga, gb = a.output(), b.output()
    _say(f"int8-vs-bf16 exact rows: max diff {np.max(np.abs(ga - gb)):.3g}")
    assert np.max(np.abs(ga - gb)) < 1e-5


@pytest.mark.parametrize("G,d,counts,n_empty", [
    (4, 128, [1, 3, 7, 0, 2, 16], 0),
    # 16 or more slots per pair on average: four wavefronts per row
    (4, 128, [40, 1, 0, 130, 17, 3], 9),
    (8, 64, [64, 64, 2, 95], 5),
    (1, 128, [33, 0, 70, 1], 4),
    (2, 64, [5, 1, 9, 2, 3], 3),
])
def test_merge_partials_against_lse_oracle(G, d, counts, n_empty):
    """Slots with no rows (m = -inf, l = 0, acc = 0, as an item past the end
    of its rows writes them) add nothing; a pair with no slots gives zeros."""
    torch = _need_gpu()
    from non_uniform_paged_amd import api
    rnd = np.random.default_rng(5 + G + d)
    n_slots = sum(counts)
    m = rnd.normal(0, 5, size=(n_slots, G)).astype(np.float32)
    l = rnd.uniform(0.5, 50, size=(n_slots, G)).astype(np.float32)
    acc = rnd.normal(0, 3, size=(n_slots, G, d)).astype(np.float32)
    empty = rnd.choice(n_slots, n_empty, replace=False)
    m[empty] = -np.inf
    l[empty] = 0
    acc[empty] = 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ws = np.concatenate([acc.reshape(-1), np.stack([m, l], -1).reshape(-1)]).astype(np.float32)
    out = torch.empty((len(counts) * G, d), dtype=torch.float32, device="cuda")
    api.tg_merge_partials(torch.from_numpy(ws).cuda(), n_slots, len(counts), G, d,
                          torch.from_numpy(off).cuda(), out)
    got = out.cpu().numpy().reshape(len(counts), G, d)
    for p_, cnt in enumerate(counts):
        if cnt == 0:
            assert np.all(got[p_] == 0)
            continue
        sl = slice(off[p_], off[p_ + 1])
        if np.all(m[sl] == -np.inf):
            continue  # no rows at all: any output is unconstrained
        ref = A.lse_merge(m[sl], l[sl], acc[sl])
        assert np.all(np.abs(got[p_] - ref) <= 1e-5 + 1e-5 * np.abs(ref))


@pytest.mark.parametrize("G,d,qd", [(1, 128, "bf16"), (8, 128, "bf16"), (2, 64, "bf16"), (8, 64, "f32"), (4, 128, "f32")])
def test_head_shapes(G, d, qd):
    _need_gpu()
    w = make_workload("llama8b", B=2, Hq=2 * G, Hkv=2, d=d, q_dtype=qd, ctx=("uniform", 200, 600),
                      n_clusters=2, recent_ppm=300_000)
    _run_and_compare(w, what=f"G{G}-d{d}-{qd}", chunk_bf=96, chunk_i8=64)


@pytest.mark.parametrize("name", ["llama8b", "tiered", "radix"])
def test_split_then_merge_equals_decode(name):
    """tg_decode_split + tg_merge_partials (the sharded form) gives the
    tg_decode_attn result, and repeated calls agree bit for bit."""
    torch = _need_gpu()
    from non_uniform_paged_amd import api
    p = _prep(make_workload(name, **SMALL[name]), chunk_bf=64, chunk_i8=128)
    p.step()
    fused = p.output().copy()
    p.step()
    assert np.array_equal(fused, p.output())
    ws = torch.empty_like(p.workspace)
    out = torch.empty_like(p.out)
    api.tg_decode_split(p.cache, p.q, ws, p.w.Hq)
    api.tg_merge_partials(ws, p.tables.n_slots, p.w.B * p.w.Hkv, p.w.Hq // p.w.Hkv, p.w.d,
                          p.cache.part_off, out)
    torch.cuda.synchronize()
    sep = out.cpu().numpy()
    assert np.array_equal(sep, fused)


def test_all_int8_and_empty_bf16_tier():
    _need_gpu()
    w = make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 640), recent_ppm=0)
    p, _ = _run_and_compare(w, what="int8-only")
    assert int(p.res.n_bf.max()) == 0


@pytest.mark.parametrize("gs,G,recent,qd", [(0, 4, 10**6, "bf16"), (1, 4, 10**6, "bf16"), (2, 4, 10**6, "bf16"),
                                            (4, 4, 10**6, "f32"), (3, 4, 250_000, "bf16"),
                                            (16, 1, 10**6, "bf16"), (8, 2, 250_000, "f32"),
                                            (2, 8, 10**6, "bf16"), (8, 4, 10**6, "bf16"),
                                            (5, 4, 250_000, "f32"), (32, 1, 10**6, "f32"),
                                            (16, 2, 10**6, "bf16"), (3, 8, 250_000, "bf16"),
                                            (4, 8, 10**6, "f32")])
def test_group_items(gs, G, recent, qd):
    """Shared-prefix group items (one pass over a shared page for all members,
    the four wavefronts of a workgroup scoring 32 / G members each) against
    the oracle, for several group sizes and head shapes."""
    _need_gpu()
    w = make_workload("radix", B=40, Hq=2 * G, Hkv=2, recent_ppm=recent, q_dtype=qd,
                      share=dict(prefix=200, branch=50, n_branches=3, suffix=(8, 300)))
    p, _ = _run_and_compare(w, what=f"group{gs}-G{G}-{recent}-{qd}", chunk_bf=48, group_size=gs)
    assert (p.tables.n_gitems > 0) == (gs > 1)


@pytest.mark.parametrize("gs,G,d,qd", [(32, 4, 128, "bf16"), (32, 8, 128, "bf16"), (24, 2, 128, "f32"),
                                        (13, 4, 128, "bf16"), (32, 4, 64, "bf16"), (32, 8, 64, "f32"),
                                        (32, 1, 64, "bf16")])
def test_group_items_wide(gs, G, d, qd):
    """Wide groups: every wavefront of the workgroup has members (G = 4, 32
    members), two passes over the pages (G = 8 takes 16 members a pass), a
    ragged last wavefront, and d = 64 (one page block per wavefront)."""
    _need_gpu()
    w = make_workload("radix", B=70, Hq=2 * G, Hkv=2, d=d, q_dtype=qd,
                      share=dict(prefix=230, branch=60, n_branches=2, suffix=(8, 200)))
    p, _ = _run_and_compare(w, what=f"wide{gs}-G{G}-d{d}-{qd}", chunk_bf=64, group_size=gs)
    assert p.tables.n_gitems > 0


@pytest.mark.parametrize("G,qd", [(4, "bf16"), (8, "f32")])
def test_group_items_past_one_page_window(G, qd):
    """Group items longer than the 64 pages whose ids a wavefront holds at
    once (a 1500-row prefix in one item: two windows, the second ending in a
    short pair) on the cooperative path."""
    _need_gpu()
    w = make_workload("radix", B=40, Hq=2 * G, Hkv=2, q_dtype=qd,
                      share=dict(prefix=1500, branch=200, n_branches=2, suffix=(8, 100)))
    p, _ = _run_and_compare(w, what=f"long-group-items-G{G}-{qd}", chunk_bf=4096, group_size=32)
    rows = p.tables.plan[:p.tables.n_gitems, 4] - p.tables.plan[:p.tables.n_gitems, 3]
    assert rows.max() > 64 * 16


@pytest.mark.parametrize("seed", [1, 2])
def test_group_items_in_any_plan_order(seed):
    """A plan whose group items do not lead (shuffled on the host) still
    decodes correctly: the leading workgroups hand ordinary items to one
    wavefront, and group items met later run on one wavefront, a tile of
    members at a time."""
    torch = _need_gpu()
    from non_uniform_paged_amd import api
    G = 4
    w = make_workload("radix", B=24, Hq=2 * G, Hkv=2,
                      share=dict(prefix=120, branch=40, n_branches=3, suffix=(8, 150)))
    p = _prep(w, chunk_bf=48, group_size=32)
    assert p.tables.n_gitems > 0
    plan = p.tables.plan.copy()
    perm = np.random.default_rng(seed).permutation(len(plan))
    assert (plan[perm][:p.tables.n_gitems, 0] >= 0).any()  # some leading entries are ordinary items
    p.cache.work.copy_(torch.from_numpy(np.ascontiguousarray(plan[perm])).to(p.cache.work.device))
    p.step()
    got = p.output()
    res_o = A.reserve_for(w)
    pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
    _check(got, A.decode(w, res_o, pairs), pairs, G, f"shuffled-plan-{seed}")


def test_replan_over_the_same_pages():
    """The runner's replan swaps in plans of other item lengths over the same
    pages (and tune_chunks picks the fastest of them): every plan decodes to
    the oracle's result, on an INT8-tier batch and a radix batch."""
    torch = _need_gpu()
    for w in (make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 3000)),
              make_workload("radix", B=12, Hq=8, Hkv=2, share=dict(prefix=150, branch=40, n_branches=2,
                                                                     suffix=(8, 120)))):
        p = _prep(w, chunk_bf=64, chunk_i8=128)
        res_o = A.reserve_for(w)
        pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
        ref = A.decode(w, res_o, pairs)
        for cb, ci in ((16, 64), (48, 192), (4096, 4096)):
            p.replan(cb, ci)
            p.step()
            _check(p.output(), ref, pairs, w.Hq // w.Hkv, f"replan-{w.name}-{cb}-{ci}")
        out = p.tune_chunks([(32, 64), (96, 256)], steps=2)
        assert {(a, b) for a, b, _ in out} == {(32, 64), (96, 256)}
        assert p.chunks == min(out, key=lambda x: x[2])[:2]
        p.step()
        _check(p.output(), ref, pairs, w.Hq // w.Hkv, f"tuned-{w.name}")


@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_custom_score_scale(scale):
    """A caller's score scale (instead of 1/sqrt(d)) reaches every path: bf16
    items, INT8 items (where the block's K scale is folded into q) and
    shared-prefix group items, against the oracle at the same scale."""
    _need_gpu()
    for w, kw in ((make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 2500)), dict(chunk_bf=64, chunk_i8=192)),
                  (make_workload("radix", B=20, Hq=8, Hkv=2, share=dict(prefix=150, branch=40, n_branches=2,
                                                                         suffix=(8, 120))),
                   dict(chunk_bf=48, group_size=32))):
        p = _prep(w, **kw)
        p.step(sm_scale=scale)
        res_o = A.reserve_for(w)
        pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
        ref = A.decode(w, res_o, pairs, scale=scale)
        _check(p.output(), ref, pairs, w.Hq // w.Hkv, f"scale-{scale}-{w.name}")


@pytest.mark.parametrize("head_major", [False, True])
def test_pages_beyond_4_gib(head_major):
    """Pages placed past byte 2^32 of their pools (bf16 and INT8 alike) give
    the same outputs, bit for bit, as the same batch in the lowest pages:
    page addresses are formed in 64 bits on every path (~13 GB of pools), in
    either pool layout (head-major: the second head slot's pages)."""
    _need_gpu()
    w = make_workload("tiered", B=1, Hq=8, Hkv=2, ctx=("fixed", 3000), n_clusters=1)
    a = _prep(w, chunk_bf=64, chunk_i8=192, head_major=head_major)
    a.step()
    ga = a.output()
    del a
    shift = (1 << 32) // (2 * 8192) + 64  # bf16 pages of 2 heads x 8 KiB: past 4 GiB
    b = _prep(w, chunk_bf=64, chunk_i8=192, shift_pages=shift, head_major=head_major)
    for tier in (0, 1):
        bt = b.tables.bt[0][tier]
        lo = int(bt[bt >= 0].min())
        if head_major:
            assert b.cache.slot_offset(0, tier, lo, 1, b.pool) >= 1 << 32, tier
        else:
            assert lo * b.pool.page_bytes(0, tier) >= 1 << 32, tier
    b.step()
    assert np.array_equal(ga, b.output())


def test_decode_step_replays_from_a_graph():
    """The decode step (split kernels, then the merge; no memory-set nodes)
    captured once in a HIP graph and replayed: every replay, with eager work
    and synchronisations between replays and new queries copied into the
    captured q buffer, equals the eager step bit for bit."""
    torch = _need_gpu()
    for w, kw in ((make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 2500)), dict(chunk_bf=64, chunk_i8=192)),
                  (make_workload("radix", B=20, Hq=8, Hkv=2, share=dict(prefix=150, branch=40, n_branches=2,
                                                                         suffix=(8, 120))),
                   dict(chunk_bf=48, group_size=32))):
        p = _prep(w, **kw)
        q0 = p.q.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
            p.step(stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            p.step()
        gen = torch.Generator(device="cpu").manual_seed(5)
        for k in range(4):
            qk = q0 if k == 0 else (q0.float() + 0.25 * torch.randn(q0.shape, generator=gen).to(q0.device)).to(q0.dtype)
            p.q.copy_(qk)
            p.step()  # eager reference with the same q
            want = p.output().copy()
            p.out.zero_()
            junk = torch.randn(1 << 20, device=q0.device).sum()  # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            got = p.output()
            assert np.isfinite(float(junk))
            assert np.array_equal(got, want), (w.name, k)
        # a replay with the workload's own q against the oracle
        p.q.copy_(q0)
        g.replay()
        res_o = A.reserve_for(w)
        pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
        _check(p.output(), A.decode(w, res_o, pairs), pairs, w.Hq // w.Hkv, f"graph-{w.name}")


def test_timed_split_equals_split_and_times_the_kernel():
    """tg_decode_split_timed writes the same partials as tg_decode_split, bit
    for bit, and its events bracket the kernel alone: a positive time no
    longer than that of an event pair recorded around the launch."""
    torch = _need_gpu()
    from non_uniform_paged_amd import api
    from non_uniform_paged_amd.runner import Prepared
    for name, w in (("llama8b", make_workload("llama8b", B=4, ctx=("uniform", 1000, 3000))),
                    ("tiered", make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 5000))),
                    ("tiered4", make_workload("tiered4", B=2, Hq=8, Hkv=2, ctx=("fixed", 3000))),
                    ("radix", make_workload("radix", B=24, Hq=8, Hkv=2,
                                            share=dict(prefix=300, branch=80, n_branches=3, suffix=(8, 300))))):
        p = Prepared(w, chunk_bf=256, chunk_i8=512)
        assert name != "radix" or p.tables.n_gitems > 0
        ws = torch.full_like(p.workspace, float("nan"))
        api.tg_decode_split(p.cache, p.q, ws, w.Hq)
        ref = ws.clone()
        ws.fill_(float("nan"))
        outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        inner = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        outer[0].record()
        api.tg_decode_split_timed(p.cache, p.q, ws, w.Hq, inner)
        outer[1].record()
        torch.cuda.synchronize()
        used = p.tables.n_slots * (w.Hq // w.Hkv) * (w.d + 2)
        assert torch.equal(ws[:used], ref[:used]), name
        t_in, t_out = inner[0].elapsed_time(inner[1]), outer[0].elapsed_time(outer[1])
        print(f"{name}: kernel {t_in * 1e3:.1f} us, event pair {t_out * 1e3:.1f} us", flush=True)
        assert 0 < t_in <= t_out, (t_in, t_out)
