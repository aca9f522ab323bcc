"""GPU parity of the decode-step append and tier ageing (tg_append_kv) and of
decoding a grown cache, against the CPU oracle.

The oracle side needs no step-by-step model: appending T rows one at a time
(the newest row bf16, the oldest block aged into INT8 whenever the tier split
of the new length says so) must leave exactly the cache that a fresh
admission at length L0 + T would hold (pinned on the CPU in
test_oracle_planner.py), so every check compares with the oracle at the grown
length: lengths exactly, INT8 codes and scales bit for bit, outputs within the
tolerance."""
import dataclasses

import numpy as np
import pytest

from oracle import attention as A
from oracle import planner as P
from oracle import quant as Q
from workloads import bf16_bits_to_f32, make_workload

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _grown(res, T):
    """The oracle reservation after T appended rows (R-step = R-tier of L + T)."""
    L = [[x + T for x in row] for row in res.L]
    split = [[P.tier_split(x, res.recent_ppm, res.quant_block) for x in row] for row in L]
    return dataclasses.replace(res, L=L, n_i8=[[s[0] for s in row] for row in split],
                               n_bf=[[s[1] for s in row] for row in split])


def _check_outputs(p, res_k, what):
    got = p.output()
    ref = A.decode(p.w, res_k)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    print(f"{what}: max-abs {err.max():.3g}", flush=True)
    assert np.all(np.isfinite(got)) and not bad.any(), f"{what}: max err {err.max():.3g}"


def _i8_block(p, r, h, j):
    """Codes and scales of INT8 block j of (r, h), read through the layout."""
    w = p.w
    d, qb = w.d, w.quant_block
    cl, s = int(p.res.cluster_of_head[h]), int(p.res.slot_in_cluster[h])
    hb = 2 * qb * d + 4 * d
    pid = int(p.tables.bt[cl][0][r, j])
    off = p.cache.slot_offset(cl, 0, pid, s, p.pool)
    blk = p.cache.pools[cl][0][off:off + hb].cpu().numpy()
    t, c = np.arange(qb)[:, None], np.arange(d)[None, :]
    nl = d // 64
    koff = ((t >> 4) * nl + (c >> 6)) * 1024 + (((c >> 3) & 3) * 16 + (t & 15)) * 16 + ((c >> 5) & 1) * 8 + (c & 7)
    voff = ((t >> 4) * nl + (c >> 6)) * 1024 + (((t >> 2) & 3) * 16 + (c & 15)) * 16 + ((c >> 4) & 3) * 4 + (t & 3)
    return (blk[:qb * d].view(np.int8)[koff], blk[qb * d:2 * qb * d].view(np.int8)[voff],
            blk[2 * qb * d:2 * qb * d + 2 * d].view(np.float16), blk[2 * qb * d + 2 * d:].view(np.float16))


CASES = {
    # tiered, few rows: several ageing events in 200 steps
    "tiered": (dict(B=2, Hq=8, Hkv=2, ctx=("fixed", 3000)), 200, [0, 1, 63, 64, 65, 130, 200]),
    # a small recent share: the bf16 ring wraps several times
    "wrap": (dict(B=2, Hq=8, Hkv=2, ctx=("fixed", 300), recent_ppm=100_000), 700, [0, 64, 333, 700]),
    # all bf16 (no ageing), ragged budgets, two clusters, d 64, G 2
    "bf16": (dict(B=3, Hq=8, Hkv=4, d=64, ctx=("uniform", 200, 900), recent_ppm=10**6), 150, [0, 150]),
    # q in fp32, G 8
    "g8": (dict(B=2, Hq=16, Hkv=2, q_dtype="f32", ctx=("fixed", 1000), recent_ppm=250_000), 130, [0, 130]),
    # ragged budgets in two clusters (each cluster its own bf16 ring) with ageing
    "clusters-ageing": (dict(B=3, Hq=8, Hkv=4, ctx=("uniform", 300, 1200), recent_ppm=250_000), 200,
                        [0, 37, 200]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_append_and_age_match_fresh_admission(case):
    torch = _need_gpu()
    from non_uniform_paged_amd.runner import Prepared
    base = "llama8b" if case in ("bf16", "clusters-ageing") else "tiered"
    over, T, checks = CASES[case]
    w = make_workload(base, **over)
    print(f"case {case}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} T={T}", flush=True)
    p = Prepared(w, chunk_bf=64, chunk_i8=128, gen_tokens=T)
    res0 = A.reserve_for(w)
    for k in range(T + 1):
        if k in checks:
            res_k = _grown(res0, k)
            lens = p.live_lengths()
            assert np.array_equal(lens[..., 0], np.array(res_k.n_i8)), k
            assert np.array_equal(lens[..., 1], np.array(res_k.n_bf)), k
            p.step()
            _check_outputs(p, res_k, f"{case} after {k} appended rows")
        if k < T:
            p.append()
    assert int(p.status.item()) == 0
    # every INT8 block, aged or written at admission, bit for bit
    res_T = _grown(res0, T)
    for r in range(w.B):
        for h in range(w.Hkv):
            n8 = res_T.n_i8[r][h]
            if not n8:
                continue
            K16, V16 = w.logical_kv(r, h, res_T.L[r][h])
            okq, oks = Q.quantize_rows(bf16_bits_to_f32(K16[:n8]), 64)
            ovq, ovs = Q.quantize_rows(bf16_bits_to_f32(V16[:n8]), 64)
            for j in range(n8 // 64):
                kq, vq, ks, vs = _i8_block(p, r, h, j)
                assert np.array_equal(kq, okq[64 * j:64 * j + 64]), (r, h, j)
                assert np.array_equal(vq, ovq[64 * j:64 * j + 64]), (r, h, j)
                assert np.array_equal(ks, oks[j].astype(np.float16)), (r, h, j)
                assert np.array_equal(vs, ovs[j].astype(np.float16)), (r, h, j)


def test_append_past_capacity_is_refused_and_flagged():
    torch = _need_gpu()
    from non_uniform_paged_amd import api
    from non_uniform_paged_amd.runner import Prepared
    w = make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 500), recent_ppm=200_000)
    T = 100
    p = Prepared(w, chunk_bf=64, chunk_i8=128, gen_tokens=T)
    for _ in range(T):
        p.append()
    assert int(p.status.item()) == 0
    # more rows than reserved: each (r, h) grows while its reserved pages last
    # (the bf16 ring is whole pages, so a little slack remains), then is
    # refused and flagged, and never written past its pages
    refused_any = False
    for extra in range(80):
        lens = p.live_lengths().copy()
        api.tg_append_kv(p.cache, p.appended[T - 1], p.status)
        torch.cuda.synchronize()
        after = p.live_lengths()
        grew = after.sum(-1) > lens.sum(-1)
        for r in range(w.B):
            for h in range(w.Hkv):
                cl = int(p.res.cluster_of_head[h])
                i8_pages = int((p.tables.bt[cl][0][r] >= 0).sum()) if p.tables.stride[cl][0] else 0
                n_bf = int(lens[r, h, 1]) + 1  # the new row lands before any ageing
                ages = P.tier_split(int(lens[r, h].sum()) + 1, w.recent_ppm, 64)[0] > lens[r, h, 0]
                ok = n_bf <= p.tables.ring[r, cl] * 16 and (not ages or lens[r, h, 0] // 64 < i8_pages)
                assert grew[r, h] == ok, (extra, r, h)
                if not ok:
                    assert np.array_equal(after[r, h], lens[r, h])
        refused_any |= not grew.all()
        assert int(p.status.item()) == int(refused_any)
    assert refused_any


def _random_growth_cases(n=24, seed=4242):
    """Seeded random shapes, tier shares, item lengths and pool layouts, each
    grown by a random number of appended rows within its reserved room."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        base = ["tiered", "llama8b", "tiered4"][i % 3]
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        d = 128 if base == "tiered4" else int(rng.choice([64, 128]))
        lo = int(rng.integers(50, 600))
        kw = dict(B=int(rng.integers(1, 5)), Hkv=Hkv, Hq=G * Hkv, d=d, n_clusters=int(rng.integers(1, Hkv + 1)),
                  ctx=("uniform", lo, lo + int(rng.integers(0, 1500))),
                  recent_ppm=int(rng.choice([100_000, 250_000, 500_000, 1_000_000])),
                  q_dtype=str(rng.choice(["bf16", "f32"])))
        T = int(rng.integers(1, 300))
        k = int(rng.integers(0, T + 1))
        hm = [(False, False), (True, True), (False, True), (True, False)][int(rng.integers(0, 4))]
        chunks = dict(chunk_bf=int(rng.choice([16, 64, 256])), chunk_i8=int(rng.choice([64, 128, 512])))
        cases.append((i, base, kw, T, k, hm, chunks))
    return cases


RANDOM_GROWTH = _random_growth_cases()


@pytest.mark.parametrize("i,base,kw,T,k,hm,chunks", RANDOM_GROWTH, ids=[f"{c[0]}-{c[1]}" for c in RANDOM_GROWTH])
def test_random_growth(i, base, kw, T, k, hm, chunks):
    """k appended rows on a random shape and pool layout: live lengths exact,
    outputs within the tolerance of the oracle at the grown length."""
    _need_gpu()
    from non_uniform_paged_amd.runner import Prepared
    print(f"case {i} {base}: {kw} T={T} k={k} layout {hm} {chunks}", flush=True)
    w = make_workload(base, **kw)
    p = Prepared(w, gen_tokens=T, head_major=hm, **chunks)
    for _ in range(k):
        p.append()
    res_k = _grown(A.reserve_for(w), k)
    lens = p.live_lengths()
    assert np.array_equal(lens[..., 0], np.array(res_k.n_i8))
    assert np.array_equal(lens[..., 1], np.array(res_k.n_bf))
    assert int(p.status.item()) == 0
    p.step()
    _check_outputs(p, res_k, f"case {i} after {k} appended rows")
