"""GPU parity over seeded random shapes: workload kind, batch, heads, group
size G, head size, clusters, tier split (bf16 / INT8 / INT4), q precision,
item lengths, shared-prefix grouping and pool layout drawn from fixed seeds,
each case against the oracle over every output.  The draws stay inside the supported
set (d in {64, 128}, G in {1, 2, 4, 8}, INT4 at d = 128)."""
import numpy as np
import pytest

from oracle import attention as A
from workloads import make_workload

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def draw_cases(n=24, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = ["llama8b", "ragged", "tiered", "tiered4", "radix"][i % 5]
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        d = 128 if kind == "tiered4" else int(rng.choice([64, 128]))
        kw = dict(Hkv=Hkv, Hq=G * Hkv, d=d, n_clusters=int(rng.integers(1, min(Hkv, 4) + 1)),
                  q_dtype=str(rng.choice(["bf16", "f32"])))
        plan = dict(chunk_bf=int(rng.choice([16, 48, 64, 256, 1024])), chunk_i8=int(rng.choice([64, 128, 192, 1024])))
        if kind == "radix":
            kw["B"] = int(rng.integers(4, 40))
            kw["share"] = dict(prefix=int(rng.integers(16, 300)), branch=int(rng.integers(16, 120)),
                               n_branches=int(rng.integers(1, 5)), suffix=(8, int(rng.integers(20, 300))))
            kw["recent_ppm"] = int(rng.choice([1_000_000, 1_000_000, 250_000]))
            plan["group_size"] = int(rng.choice([0, 2, 5, 32]))
        else:
            lo = int(rng.integers(1, 400))
            kw["B"] = int(rng.integers(1, 7))
            kw["ctx"] = ("uniform", lo, lo + int(rng.integers(0, 2500)))
            if kind in ("tiered", "tiered4"):
                kw["recent_ppm"] = int(rng.choice([125_000, 500_000, 0]))
            else:
                kw["recent_ppm"] = int(rng.choice([1_000_000, 300_000]))
        cases.append((i, kind, kw, plan))
    return cases


CASES = draw_cases(60)


@pytest.mark.parametrize("i,kind,kw,plan", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_random_shape(i, kind, kw, plan):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_uniform_paged_amd.runner import Prepared
    # pool layout (INT8 pools, bf16 pools head-major) from a stream of its own
    hm = [(False, False), (True, True), (False, True), (True, False)][int(np.random.default_rng(7000 + i).integers(0, 4))]
    print(f"case {i} {kind}: {kw} {plan} layout {hm}", flush=True)
    w = make_workload(kind, **kw)
    p = Prepared(w, head_major=hm, **plan)
    p.step()
    got = p.output()
    res_o = A.reserve_for(w)
    pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
    ref = A.decode(w, res_o, pairs)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"case {i}: max err {err.max():.3g}"
