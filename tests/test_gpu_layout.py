"""Pool layouts (include/tg.h): a head-major pool holds the bytes of the
page-major one with each head slot's pages gathered into one run, and every
entry point gives the same result on either, bit for bit.  Tangram page,
"Three mechanisms", item 2 fixes what a page holds (the slots of every head
of its cluster), not where in memory those slots sit."""
import numpy as np
import pytest

from workloads import make_workload

pytestmark = pytest.mark.gpu


def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _page_major(p, c, t):
    """Pool (c, t) of p's cache as page-major bytes."""
    pool = p.cache.pools[c][t]
    if not p.cache.struct.head_major[c][t]:
        return pool
    n_c, cap = int(p.res.cluster_size[c]), p.pool.capacity(c, t)
    return pool.view(n_c, cap, -1).transpose(0, 1).reshape(-1)


CASES = {
    # two clusters of four heads, bf16 only, ragged budgets
    "llama8b": ("llama8b", dict(B=6, ctx=("uniform", 300, 1500)), dict(chunk_bf=128)),
    # one cluster of two heads with an INT8 tier
    "tiered": ("tiered", dict(B=2, Hq=8, Hkv=2, ctx=("fixed", 3000)), dict(chunk_bf=128, chunk_i8=256)),
    # INT4 tier
    "tiered4": ("tiered4", dict(B=2, Hq=8, Hkv=2, ctx=("fixed", 3000)), dict(chunk_bf=128, chunk_i8=256)),
    # shared radix pages on cooperative group items, and an INT8 tier beside them
    "radix": ("radix", dict(B=40, share=dict(prefix=400, branch=100, n_branches=3, suffix=(8, 300))),
              dict(chunk_bf=96)),
    "radix-i8": ("radix", dict(B=24, recent_ppm=300_000,
                               share=dict(prefix=400, branch=100, n_branches=3, suffix=(8, 300))),
                 dict(chunk_bf=96, chunk_i8=128)),
    # d 64, G 8, fp32 q, three clusters
    "d64-g8": ("llama8b", dict(B=3, Hq=48, Hkv=6, d=64, q_dtype="f32", n_clusters=3, ctx=("uniform", 200, 900)),
               dict(chunk_bf=64)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_head_major_pools_hold_the_same_bytes_and_give_the_same_outputs(case):
    torch = _need_gpu()
    from non_uniform_paged_amd.runner import Prepared
    base, over, kw = CASES[case]
    w = make_workload(base, **over)
    print(f"case {case}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} clusters {w.n_clusters}", flush=True)
    a = Prepared(w, head_major=False, **kw)
    b = Prepared(w, head_major=True, **kw)
    assert not a.cache.struct.head_major[0][1] and b.cache.struct.head_major[0][1]
    for p in (a, b):  # bytes no row reaches: 0 in both
        p.rewrite_zeroed()
    multi = False
    for c in range(a.res.C):
        multi = multi or int(a.res.cluster_size[c]) > 1
        for t in range(2):
            if a.cache.pools[c][t] is None:
                continue
            assert torch.equal(_page_major(a, c, t), _page_major(b, c, t)), (c, t)
    assert multi  # at least one cluster where the layouts differ
    a.step()
    b.step()
    assert np.array_equal(a.output(), b.output())


def test_append_and_ageing_in_both_layouts():
    """Appended rows and blocks aged into INT8 land in the same bytes, and the
    grown caches decode alike, step after step."""
    torch = _need_gpu()
    from non_uniform_paged_amd.runner import Prepared
    w = make_workload("llama8b", B=3, Hq=8, Hkv=4, ctx=("uniform", 300, 1200), recent_ppm=250_000)
    T = 150
    a = Prepared(w, chunk_bf=64, chunk_i8=128, gen_tokens=T, head_major=False)
    b = Prepared(w, chunk_bf=64, chunk_i8=128, gen_tokens=T, head_major=True)
    for p in (a, b):
        p.rewrite_zeroed()
    for k in range(T):
        a.append()
        b.append()
        if k % 37 == 0 or k == T - 1:
            a.step()
            b.step()
            assert np.array_equal(a.output(), b.output()), k
    assert np.array_equal(a.live_lengths(), b.live_lengths())
    assert int(a.status.item()) == 0 and int(b.status.item()) == 0
    for c in range(a.res.C):
        for t in range(2):
            if a.cache.pools[c][t] is not None:
                assert torch.equal(_page_major(a, c, t), _page_major(b, c, t)), (c, t)


def test_streamed_decode_of_a_head_major_cache():
    """The INT8 pools of a head-major cache go to host memory page-major (the
    streamed decode copies whole pages); the bf16 pools stay head-major and
    the streamed step equals the resident one bit for bit."""
    _need_gpu()
    from non_uniform_paged_amd.runner import Prepared
    w = make_workload("tiered", B=3, Hq=8, Hkv=2, ctx=("fixed", 2600))
    p = Prepared(w, chunk_bf=128, chunk_i8=256, head_major=True)
    p.step()
    ref = p.output().copy()
    p.to_host_i8()
    assert not p.cache.struct.head_major[0][0] and p.cache.struct.head_major[0][1]
    p.step_streamed()
    assert np.array_equal(p.output(), ref)


def test_streamed_decode_refuses_head_major_int8_pools():
    _need_gpu()
    from non_uniform_paged_amd import api
    from non_uniform_paged_amd.runner import Prepared
    w = make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 1500))
    p = Prepared(w, chunk_bf=128, chunk_i8=256, head_major=True)
    p.to_host_i8()
    p.cache.struct.head_major[0][0] = 1  # as if the host pool were head-major
    with pytest.raises(api.TGError) as e:
        p.step_streamed()
    assert e.value.name == "TG_EUNSUPPORTED"
