"""tg_decode_attn_noalloc through the C ABI: the decode step with its
partials in the library's fixed device array gives the outputs of
tg_decode_attn (same kernels, same plan) bit for bit, on two calls in a row,
the second with a smaller batch, and both match the CPU oracle within the
tolerance |gpu - oracle| <= 2e-3 + 1e-2 |oracle|.  The call allocates no
device memory through the caller's allocator."""
import ctypes

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


def _run_pair(w, **kw):
    torch = _need_gpu()
    from non_uniform_paged_amd import _lib as L
    from non_uniform_paged_amd import api
    from non_uniform_paged_amd.runner import Prepared
    print(f"case noalloc {w.name}: B={w.B} {kw}", flush=True)
    p = Prepared(w, **kw)
    G = w.Hq // w.Hkv
    assert api.tg_decode_workspace_bytes(p.tables.n_slots, G, w.d) <= L.TG_NOALLOC_SCRATCH_BYTES
    p.step()
    ref = p.output().copy()
    out = torch.full_like(p.out, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    a = api._decode_args(p.cache, p.q, out, None, w.Hq, 0.0)
    st = L.lib().tg_decode_attn_noalloc(ctypes.byref(p.cache.struct), ctypes.byref(a), None)
    assert st == L.TG_OK, st
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    got = out.cpu().numpy()
    assert np.array_equal(got, ref), f"{w.name}: noalloc differs from tg_decode_attn"
    pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
    oracle = A.decode(w, A.reserve_for(w), pairs)
    err = np.abs(got - oracle)
    assert np.all(err <= 2e-3 + 1e-2 * np.abs(oracle)), float(err.max())
    return p.tables.n_slots


def test_noalloc_equals_decode_attn_twice_second_smaller():
    n1 = _run_pair(make_workload("radix", B=40, share=dict(prefix=400, branch=100, n_branches=3, suffix=(8, 300))),
                   chunk_bf=96)
    n2 = _run_pair(make_workload("tiered", B=2, Hq=8, Hkv=2, ctx=("fixed", 2000)), chunk_bf=128, chunk_i8=256)
    assert n2 < n1


def test_noalloc_at_full_size_and_then_a_small_batch():
    """The benchmark's llama8b step (2031 plan items, 4.2 MB of partials),
    then Tiny: the small call reads none of the large call's stale partials."""
    from non_uniform_paged_amd.runner import PLAN_CHUNKS
    cb, ci = PLAN_CHUNKS["llama8b"]
    n1 = _run_pair(make_workload("llama8b"), chunk_bf=cb, chunk_i8=ci)
    n2 = _run_pair(make_workload("tiny"), chunk_bf=64)
    assert n2 < n1


def test_noalloc_refuses_partials_past_its_array():
    torch = _need_gpu()
    from non_uniform_paged_amd import _lib as L
    from non_uniform_paged_amd import api
    from non_uniform_paged_amd.runner import Prepared
    w = make_workload("llama8b", B=2, ctx=("uniform", 500, 900))
    p = Prepared(w, chunk_bf=64)
    a = api._decode_args(p.cache, p.q, p.out, None, w.Hq, 0.0)
    a.n_slots = L.TG_NOALLOC_SCRATCH_BYTES // (4 * (w.d + 2) * 4) + 1  # one slot past the array
    assert L.lib().tg_decode_attn_noalloc(ctypes.byref(p.cache.struct), ctypes.byref(a), None) == L.TG_EOVERFLOW
    torch.cuda.synchronize()
