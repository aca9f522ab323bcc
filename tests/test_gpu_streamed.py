"""INT8 tier in pinned host memory, streamed through two HBM staging slots
per decode step (tg_decode_streamed): the same kernels on the same pages, so
the output must equal the HBM-resident decode bit for bit (and the oracle
within the tolerance)."""
import numpy as np
import pytest

from oracle import attention as A
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


CASES = {
    "tiered-b3": ("tiered", dict(B=3, Hq=8, Hkv=2, ctx=("fixed", 3000))),
    "two-clusters-b5": ("llama8b", dict(B=5, ctx=("uniform", 600, 2500), recent_ppm=250_000)),
    # INT4 codes in host memory: half the bytes cross per block
    "int4-b3": ("tiered4", dict(B=3, Hq=8, Hkv=2, ctx=("fixed", 3000))),
    "int4-two-clusters-b4": ("tiered4", dict(B=4, Hq=16, Hkv=4, n_clusters=2, ctx=("uniform", 700, 2600))),
    "d64-g8-f32": ("tiered", dict(B=4, Hq=16, Hkv=2, d=64, q_dtype="f32", ctx=("fixed", 1500))),
    # shared radix pages in both tiers: group items run before the streamed
    # INT8 items, and shared INT8 pages are staged once per request
    "radix-int8": ("radix", dict(B=12, Hq=8, Hkv=2, recent_ppm=250_000,
                                 share=dict(prefix=300, branch=80, n_branches=2, suffix=(8, 300)))),
}


@pytest.mark.parametrize("case", list(CASES))
def test_streamed_equals_resident_bitwise(case):
    _need_gpu()
    from non_uniform_paged_amd.runner import Prepared
    base, over = CASES[case]
    w = make_workload(base, **over)
    print(f"case {case}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} C={w.n_clusters}", flush=True)
    p = Prepared(w, chunk_bf=64, chunk_i8=128)
    assert p.tables.stride_has_i8
    p.step()
    resident = p.output().copy()
    p.to_host_i8()
    assert p.chunk_off[0] < p.tables.n_items
    for _ in range(2):  # the staging slots are reused within and across calls
        p.step_streamed()
        assert np.array_equal(p.output(), resident)
    ref = A.decode(w, A.reserve_for(w))
    err = np.abs(resident - ref)
    assert not (err > 2e-3 + 1e-2 * np.abs(ref)).any(), err.max()
