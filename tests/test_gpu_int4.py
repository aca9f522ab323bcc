"""GPU parity of the INT4 slow tier (codes in [-7, 7], two per byte, one fp16
scale per 64-row block and channel): codes and scales bit for bit against the
oracle quantiser, read back through the layout include/tg.h documents;
decode outputs against the oracle; rows exactly representable in both tiers
give the bf16 tier's result; the append path ages into INT4; the host-DRAM
streamed decode equals the resident one."""
import dataclasses

import numpy as np
import pytest

from oracle import attention as A
from oracle import planner as P
from oracle import quant as Q
from workloads import Workload, bf16_bits_to_f32, make_workload

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _prep(w, **kw):
    from non_uniform_paged_amd.runner import Prepared
    return Prepared(w, **kw)


def _check(got, ref, what):
    err = np.abs(got - ref)
    print(f"{what}: max-abs {err.max():.3g}", flush=True)
    assert np.all(np.isfinite(got)) and not (err > ATOL + RTOL * np.abs(ref)).any(), f"{what}: {err.max():.3g}"


def _i4_block(p, r, h, j):
    """(K codes [64][d], V codes [64][d], K scales, V scales) of INT4 block j."""
    w = p.w
    d = w.d
    cl, s = int(p.res.cluster_of_head[h]), int(p.res.slot_in_cluster[h])
    pb, hb = p.pool.page_bytes(cl, 0), 64 * d + 4 * d
    assert pb == hb * p.res.cluster_size[cl]
    pid = int(p.tables.bt[cl][0][r, j])
    off = p.cache.slot_offset(cl, 0, pid, s, p.pool)
    blk = p.cache.pools[cl][0][off:off + hb].cpu().numpy()
    kw = blk[:32 * d].view(np.uint32)
    vw = blk[32 * d:64 * d].view(np.uint32)
    t = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    kword = ((t >> 4) * 64 + (t & 15) + 16 * ((c >> 3) & 3)) * 4 + (c >> 5)
    knib = ((c & 1) << 2) | ((c & 7) >> 1)
    vword = ((t >> 4) * 64 + (c & 15) + 16 * ((t >> 2) & 3)) * 4 + (c >> 5)
    vnib = ((t & 1) << 2) | (((c >> 4) & 1) << 1) | ((t & 3) >> 1)
    kq = ((kw[kword] >> (4 * knib)) & 15).astype(np.int64) - 8
    vq = ((vw[vword] >> (4 * vnib)) & 15).astype(np.int64) - 8
    return kq, vq, blk[64 * d:66 * d].view(np.float16), blk[66 * d:].view(np.float16)


def test_layout_is_a_bijection():
    d = 128
    t = np.arange(64)[:, None]
    c = np.arange(d)[None, :]
    for word, nib in ((((t >> 4) * 64 + (t & 15) + 16 * ((c >> 3) & 3)) * 4 + (c >> 5),
                       ((c & 1) << 2) | ((c & 7) >> 1)),
                      (((t >> 4) * 64 + (c & 15) + 16 * ((t >> 2) & 3)) * 4 + (c >> 5),
                       ((t & 1) << 2) | (((c >> 4) & 1) << 1) | ((t & 3) >> 1))):
        assert sorted((word * 8 + nib).ravel()) == list(range(64 * d))


def test_int4_codes_scales_and_decode():
    _need_gpu()
    w = make_workload("tiered4", B=2, Hq=8, Hkv=2, ctx=("fixed", 3000))
    p = _prep(w, chunk_bf=64, chunk_i8=128)
    for r in range(w.B):
        for h in range(w.Hkv):
            n8 = int(p.res.n_i8[r, h])
            K16, V16 = w.logical_kv(r, h, int(p.res.length[r, h]))
            okq, oks = Q.quantize_rows(bf16_bits_to_f32(K16[:n8]), 64, 4)
            ovq, ovs = Q.quantize_rows(bf16_bits_to_f32(V16[:n8]), 64, 4)
            for j in range(n8 // 64):
                kq, vq, ks, vs = _i4_block(p, r, h, j)
                assert np.array_equal(kq, okq[64 * j:64 * j + 64]), (r, h, j)
                assert np.array_equal(vq, ovq[64 * j:64 * j + 64]), (r, h, j)
                assert np.array_equal(ks, oks[j]) and np.array_equal(vs, ovs[j]), (r, h, j)
    p.step()
    _check(p.output(), A.decode(w, A.reserve_for(w)), "int4 tiered")


@pytest.mark.parametrize("G,qd", [(4, "bf16"), (1, "f32"), (8, "bf16"), (2, "f32")])
def test_int4_head_shapes(G, qd):
    _need_gpu()
    w = make_workload("tiered4", B=2, Hq=2 * G, Hkv=2, q_dtype=qd, ctx=("fixed", 2000))
    p = _prep(w, chunk_bf=96, chunk_i8=192)
    p.step()
    _check(p.output(), A.decode(w, A.reserve_for(w)), f"int4 G{G} {qd}")


@pytest.mark.parametrize("C", [1, 2])
def test_int4_under_shared_radix_pages(C):
    """The INT4 tier beside shared radix pages: group items over the shared
    bf16 pages, shared INT4 blocks referenced by many tables, and ragged
    clusters, against the oracle (which quantises the same rows to 4 bits)."""
    _need_gpu()
    w = make_workload("radix", B=24, Hq=8, Hkv=2, old_bits=4, recent_ppm=250_000, n_clusters=C,
                      share=dict(prefix=300, branch=80, n_branches=3, suffix=(8, 300)))
    p = _prep(w, chunk_bf=64, chunk_i8=128)
    assert p.tables.n_gitems > 0 and p.tables.stride_has_i8
    p.step()
    _check(p.output(), A.decode(w, A.reserve_for(w)), f"int4 radix C{C}")


class _ExactRows(Workload):
    """Rows that are multiples of 2^-3 within +-7 * 2^-3, with +-7 * 2^-3 in
    every 64-row block and channel: exact in bf16 and in INT4."""

    def stream_rows(self, key, n):
        # a stable seed from the stream key ("seq", r, h) or ("node", k, h):
        # the same rows in every process (str hashes are salted per process)
        tag = {"seq": 1, "node": 2}[key[0]]
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([20260601, 99, tag, *key[1:]])))
        out = []
        for _ in range(2):
            k = g.integers(-7, 8, size=(n, self.d))
            k[::64] = 7
            k[1::64] = -7
            x = (k * 2.0 ** -3).astype(np.float32)
            out.append((x.view(np.uint32) >> 16).astype(np.uint16))
        return out[0], out[1]


def test_int4_equals_bf16_on_exact_rows():
    _need_gpu()
    base = make_workload("tiered4", B=2, Hq=8, Hkv=2, ctx=("fixed", 1200))
    w4 = _ExactRows(**{f.name: getattr(base, f.name) for f in dataclasses.fields(Workload)})
    wb = dataclasses.replace(w4, old_bits=8, recent_ppm=10**6)
    p4 = _prep(w4, chunk_bf=64, chunk_i8=128)
    pb = _prep(wb, chunk_bf=64, chunk_i8=128)
    assert int(p4.res.n_i8.min()) > 0 and int(pb.res.n_i8.max()) == 0
    p4.step()
    pb.step()
    # the INT4 path feeds q * s_K and the weights to the matrix cores as one
    # fp16 part each (2^-11 relative), the bf16 path as two: the outputs
    # (|v| <= 7/8) agree to ~1e-5, while any wrong code would move a value by
    # at least 2^-3
    assert np.max(np.abs(p4.output() - pb.output())) < 2e-4


def test_int4_append_ageing_matches_fresh_admission():
    _need_gpu()
    w = make_workload("tiered4", B=2, Hq=8, Hkv=2, ctx=("fixed", 700), recent_ppm=150_000)
    T = 300
    p = _prep(w, chunk_bf=64, chunk_i8=128, gen_tokens=T)
    for _ in range(T):
        p.append()
    res0 = A.reserve_for(w)
    L = [[x + T for x in row] for row in res0.L]
    split = [[P.tier_split(x, res0.recent_ppm, 64) for x in row] for row in L]
    resT = dataclasses.replace(res0, L=L, n_i8=[[a for a, _ in row] for row in split],
                               n_bf=[[b for _, b in row] for row in split])
    lens = p.live_lengths()
    assert np.array_equal(lens[..., 0], np.array(resT.n_i8)) and int(p.status.item()) == 0
    for r in range(w.B):
        for h in range(w.Hkv):
            n8 = resT.n_i8[r][h]
            K16, V16 = w.logical_kv(r, h, resT.L[r][h])
            okq, oks = Q.quantize_rows(bf16_bits_to_f32(K16[:n8]), 64, 4)
            for j in range(n8 // 64):
                kq, vq, ks, vs = _i4_block(p, r, h, j)
                assert np.array_equal(kq, okq[64 * j:64 * j + 64]) and np.array_equal(ks, oks[j]), (r, h, j)
    p.step()
    _check(p.output(), A.decode(w, resT), "int4 after appends")


def test_int4_streamed_equals_resident():
    _need_gpu()
    w = make_workload("tiered4", B=3, Hq=8, Hkv=2, ctx=("fixed", 2500))
    p = _prep(w, chunk_bf=64, chunk_i8=128)
    p.step()
    resident = p.output().copy()
    p.to_host_i8()
    p.step_streamed()
    assert np.array_equal(p.output(), resident)
