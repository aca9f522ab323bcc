"""GPU edge cases of the method, through the C ABI, against the CPU oracle.

* Placement freedom (Tangram page, "Three mechanisms", item 2: where a page
  sits is the allocator's choice): a seeded random permutation of the
  physical page ids of every (cluster, tier) pool, applied to the pool bytes
  and the block tables together, leaves every output bit for bit unchanged --
  bf16 pages, INT8 and INT4 blocks, shared radix pages read by group items,
  and the INT8 tier streamed from host memory.
* The online normaliser's exactness for any split (CAP survey page, section
  2.4.3, online normaliser [88]): keys whose scores climb by more than 2^8 (in
  base 2) on every page, so that the running maximum is passed -- and the
  accumulators rescaled -- on every page of every item, with the maximum on
  the last row of the last (ragged) page; and score scales 30 and 100 times
  1/sqrt(d).  On the bf16, INT8 and INT4 paths and on shared-prefix group
  items.
* Full sizes: every (request, KV-head) pair of the 128K tiered workloads and
  128 sampled pairs of the ragged and radix workloads, in the benchmark's
  launch configuration.

Tolerance: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| for every element."""
import concurrent.futures as cf
import dataclasses
import math
import sys

import numpy as np
import pytest

from oracle import attention as A
from workloads import Workload, make_workload
from workloads.gen import bf16_bits_to_f32, bf16_round

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


def _oracle(w, pairs, scale=None):
    """Oracle outputs of the given pairs, computed on a thread pool."""
    res = A.reserve_for(w)
    q = A.q_f64(w)
    G = w.Hq // w.Hkv
    out = np.full((w.B, w.Hq, w.d), np.nan)

    def one(rh):
        r, h = rh
        return rh, A.decode_pair(w, res, r, h, q, scale)

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        for (r, h), o in ex.map(one, pairs):
            out[r, h * G:(h + 1) * G] = o
    return out


def _check(got, ref, pairs, G, what):
    worst_abs = worst_rel = 0.0
    for r, h in pairs:
        g = got[r, h * G:(h + 1) * G]
        o = ref[r, h * G:(h + 1) * G]
        assert np.all(np.isfinite(g)), (what, r, h)
        err = np.abs(g - o)
        bad = err > ATOL + RTOL * np.abs(o)
        assert not bad.any(), f"{what}: (r={r}, h={h}) max err {err.max():.3g} at |ref| {np.abs(o)[bad].max():.3g}"
        worst_abs = max(worst_abs, float(err.max()))
        big = np.abs(o) >= 1e-3
        if big.any():
            worst_rel = max(worst_rel, float((err[big] / np.abs(o[big])).max()))
    _say(f"{what}: max-abs {worst_abs:.3g} max-rel {worst_rel:.3g} over {len(pairs)} (r,h)")
    return worst_abs, worst_rel


def _all_pairs(w):
    return [(r, h) for r in range(w.B) for h in range(w.Hkv)]


# ---------------------------------------------------------------------------- placement
def _permute_pages(p, seed):
    """Move every page of every (cluster, tier) pool to a seeded random new
    id: pool bytes and block tables (host and device copies) together."""
    torch = _need_gpu()
    g = np.random.default_rng(seed)
    moved = 0
    for c in range(p.res.C):
        for t in range(2):
            pool = p.cache.pools[c][t]
            if pool is None:
                continue
            cap, pb = p.pool.capacity(c, t), p.pool.page_bytes(c, t)
            perm = g.permutation(cap)  # page j goes to perm[j]
            new = torch.empty_like(pool)
            to = torch.from_numpy(perm).to(pool.device)
            if p.cache.struct.head_major[c][t]:  # [slot][page][head bytes]
                n_c = int(p.res.cluster_size[c])
                new.view(n_c, cap, -1)[:, to] = pool.view(n_c, cap, -1)
            else:  # [page][page bytes]
                new.view(cap, pb)[to] = pool.view(cap, pb)
            pool.copy_(new)
            del new
            bt = p.tables.bt[c][t]
            if bt.size:
                live = bt >= 0
                moved += int((perm[bt[live]] != bt[live]).sum())
                bt[live] = perm[bt[live]]
                p.cache.bt[c][t].copy_(torch.from_numpy(bt).to(pool.device))
    torch.cuda.synchronize()
    return moved


PERMUTED = {
    "ragged": (dict(B=12, ctx=("loguniform", 100, 4000)), dict(chunk_bf=128)),
    "tiered": (dict(B=2, ctx=("fixed", 6000)), dict(chunk_bf=128, chunk_i8=256)),
    "tiered4": (dict(B=2, ctx=("fixed", 6000)), dict(chunk_bf=128, chunk_i8=256)),
    "radix": (dict(B=40, share=dict(prefix=400, branch=100, n_branches=3, suffix=(8, 300))), dict(chunk_bf=96)),
    "radix-i8": (dict(B=24, recent_ppm=300_000, share=dict(prefix=400, branch=100, n_branches=3, suffix=(8, 300))),
                 dict(chunk_bf=96, chunk_i8=128)),
}


@pytest.mark.parametrize("case", list(PERMUTED))
def test_random_page_permutation_bitwise(case):
    _need_gpu()
    over, kw = PERMUTED[case]
    name = case.split("-")[0]
    w = make_workload(name, **over)
    _say(f"case permute {case}: B={w.B} {kw}")
    p = _prep(w, slack_pages=23, **kw)
    assert name != "radix" or p.tables.n_gitems > 0
    p.step()
    before = p.output().copy()
    moved = _permute_pages(p, seed=31)
    assert moved > 0
    p.step()
    after = p.output()
    assert np.array_equal(before, after), f"{case}: outputs differ after permuting {moved} page ids"
    if p.tables.stride_has_i8:
        # the INT8 tier streamed from host memory reads the permuted ids too
        # (no longer runs of consecutive pages)
        p.to_host_i8()
        p.step_streamed()
        assert np.array_equal(before, p.output()), f"{case}: streamed decode differs after the permutation"
    pairs = _all_pairs(w)
    _check(after, _oracle(w, pairs), pairs, w.Hq // w.Hkv, f"permuted-{case}")


# ---------------------------------------------------------------------------- softmax range
class _Ramp(Workload):
    """Scores that climb along each sequence: q is 4 in one channel per
    KV-head (and N(0, 1/4) elsewhere), and K's value in
    that channel grows by `step` per logical row (on top of its N(0, 1)
    draw), so q . k rises by about 4 * step * scale per row -- more than 2^8
    in base 2 per 16-row page at the default scale (checked per q-head).  Shared radix nodes and
    private suffixes continue the same ramp at their logical positions."""

    step = 1.2

    def _channel(self, h):
        return (37 * h + 5) % self.d

    def q(self):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([20260601, 77, self.cfg_id])))
        x = 0.5 * g.standard_normal((self.B, self.Hq, self.d), dtype=np.float32)
        for hq in range(self.Hq):
            x[:, hq, self._channel(hq // self.G)] = np.float32(4.0)
        return x if self.q_dtype == "f32" else bf16_round(x)

    def _start(self, key):
        tag, a, h = key
        if tag == "seq":
            return int(self.n_fixed[a]) if self.paths is not None else 0
        for path in self.paths:
            if a in path:
                return int(sum(int(self.node_len[n]) for n in path[:path.index(a)]))
        raise KeyError(key)

    def _stream(self, key, n, kind):
        bits = super()._stream(key, n, kind)
        if kind != "K":
            return bits
        x = bf16_bits_to_f32(bits)
        ch = self._channel(key[2])
        x[:, ch] = x[:, ch] + np.float32(self.step) * (self._start(key) + np.arange(n, dtype=np.float32))
        return bf16_round(x)


def _ramp(base):
    return _Ramp(**{f.name: getattr(base, f.name) for f in dataclasses.fields(Workload)})


RAMPS = {
    "bf16": (make_workload, "llama8b", dict(B=3, ctx=("uniform", 700, 1300)), dict(chunk_bf=256)),
    "bf16-f32q": (make_workload, "tiny", dict(), dict(chunk_bf=64)),
    "int8": (make_workload, "tiered", dict(B=2, ctx=("fixed", 3001)), dict(chunk_bf=128, chunk_i8=512)),
    "int4": (make_workload, "tiered4", dict(B=2, ctx=("fixed", 3001)), dict(chunk_bf=128, chunk_i8=512)),
    "group": (make_workload, "radix", dict(B=40, share=dict(prefix=403, branch=97, n_branches=3, suffix=(9, 300))),
              dict(chunk_bf=96)),
}


@pytest.mark.parametrize("case", list(RAMPS))
def test_scores_climbing_past_the_reference_max_on_every_page(case):
    _need_gpu()
    mk, name, over, kw = RAMPS[case]
    w = _ramp(mk(name, **over))
    _say(f"case ramp {case}: B={w.B} {kw}")
    # the climb per page, in base 2, at the default scale, for every q-head
    q = A.q_f64(w)
    scale = 1 / math.sqrt(w.d)
    for h in range(w.Hkv):
        ch = w._channel(h)
        rise = q[:, h * w.G:(h + 1) * w.G, ch].min() * w.step * 16 * scale * math.log2(math.e)
        assert rise > 8.5, rise
    p = _prep(w, **kw)
    assert case != "group" or p.tables.n_gitems > 0
    p.step()
    pairs = _all_pairs(w)
    _check(p.output(), _oracle(w, pairs), pairs, w.G, f"ramp-{case}")


SCALED = {
    "bf16": ("llama8b", dict(B=3, ctx=("uniform", 700, 1300)), dict(chunk_bf=256)),
    "bf16-f32q": ("tiny", dict(), dict(chunk_bf=64)),
    "int8": ("tiered", dict(B=2, ctx=("fixed", 3001)), dict(chunk_bf=128, chunk_i8=512)),
    "int4": ("tiered4", dict(B=2, ctx=("fixed", 3001)), dict(chunk_bf=128, chunk_i8=512)),
    "group": ("radix", dict(B=40, share=dict(prefix=403, branch=97, n_branches=3, suffix=(9, 300))), dict(chunk_bf=96)),
}


@pytest.mark.parametrize("mult", [30, 100])
@pytest.mark.parametrize("case", list(SCALED))
def test_large_score_scales(case, mult):
    """Score scales 30 and 100 times 1/sqrt(d): sharply peaked softmax whose
    maximum moves between pages and items."""
    _need_gpu()
    name, over, kw = SCALED[case]
    w = make_workload(name, **over)
    scale = mult / math.sqrt(w.d)
    _say(f"case scale x{mult} {case}: B={w.B} {kw}")
    p = _prep(w, **kw)
    p.step(sm_scale=scale)
    pairs = _all_pairs(w)
    _check(p.output(), _oracle(w, pairs, scale=scale), pairs, w.G, f"scale-x{mult}-{case}")


# ---------------------------------------------------------------------------- full sizes
@pytest.mark.parametrize("name,k", [("tiered", None), ("tiered4", None), ("ragged", 128), ("radix", 128),
                                    ("llama8b", 128)])
def test_full_size_wide_coverage(name, k):
    """Full sizes in the benchmark's launch configuration: every pair of the
    128K tiered workloads, 128 sampled pairs of the others."""
    _need_gpu()
    from non_uniform_paged_amd.runner import PLAN_CHUNKS
    w = make_workload(name)
    pairs = _all_pairs(w)
    if k is not None:
        rnd = np.random.default_rng(23)
        pairs = sorted(pairs[i] for i in rnd.choice(len(pairs), size=k, replace=False))
    cb, ci = PLAN_CHUNKS[name]
    _say(f"case full {name}: {len(pairs)} pairs, chunks {cb}/{ci}")
    p = _prep(w, chunk_bf=cb, chunk_i8=ci)
    p.step()
    got = p.output()
    del p
    _check(got, _oracle(w, pairs), pairs, w.G, f"full-{name}")
