"""Pins for the fp64 attention oracle (oracle/attention.py) against facts the
mathematics fixes: a library SDPA on dense tensors, closed forms, brute force
with math.fsum, invariances, INT8/bf16 equivalence, and split invariance of
the log-sum-exp merge."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import quant
from workloads import make_workload


def _bf16_value_from_fields(u: int) -> float:
    """Value of one bf16 bit pattern read from the format's fields: bit 15
    the sign, bits 14..7 the exponent (bias 127; 0 = subnormal, 255 = inf or
    NaN), bits 6..0 the fraction -- built with math.ldexp, not by moving the
    pattern into an fp32 word, so that it checks the oracle's decoder rather
    than restating it."""
    sign = -1.0 if (u >> 15) & 1 else 1.0
    e = (u >> 7) & 0xFF
    f = u & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


_BF16_TABLE = np.array([_bf16_value_from_fields(u) for u in range(1 << 16)])


def _bf16_table(u):
    return _BF16_TABLE[np.asarray(u, dtype=np.uint16).astype(np.int64)]


def _q_from_fields(w):
    q = w.q()
    return np.asarray(q, np.float64) if w.q_dtype == "f32" else _bf16_table(q)


def _sdpa_dense(w, res):
    """torch fp64 scaled_dot_product_attention over the full logical rows.
    Rows and queries are decoded from the bf16 fields (``_bf16_table``), not
    by the oracle's own decoder, so this pin also covers that decoder."""
    q = torch.from_numpy(_q_from_fields(w))
    G = w.Hq // w.Hkv
    out = np.zeros((w.B, w.Hq, w.d))
    for r in range(w.B):
        Ks, Vs = [], []
        for h in range(w.Hkv):
            K16, V16 = w.logical_kv(r, h, res.L[r][h])
            Ks.append(torch.from_numpy(_bf16_table(K16)))
            Vs.append(torch.from_numpy(_bf16_table(V16)))
        K = torch.stack(Ks).repeat_interleave(G, dim=0)      # [Hq, L, d]
        V = torch.stack(Vs).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(q[r][:, None, :], K, V)
        out[r] = o[:, 0, :].numpy()
    return out


@pytest.mark.parametrize("name,over", [
    ("tiny", dict(budget=None, n_clusters=1)),
    ("llama8b", dict(B=2, ctx=("uniform", 200, 500), ratio_ppm=(1_000_000, 1_000_000), n_clusters=1)),
])
def test_uniform_budgets_equal_dense_sdpa(name, over):
    w = make_workload(name, **over)
    res = A.reserve_for(w)
    assert all(res.L[r][h] == int(w.n_comp[r]) for r in range(w.B) for h in range(w.Hkv))
    o = A.decode(w, res)
    ref = _sdpa_dense(w, res)
    assert np.max(np.abs(o - ref)) < 1e-12


def test_single_row_returns_its_value_row():
    g = np.random.default_rng(0)
    q = g.standard_normal((4, 64))
    K = g.standard_normal((1, 64))
    V = g.standard_normal((1, 64))
    o = A.attend(q, K, V, 0.125)
    assert np.array_equal(o, np.repeat(V, 4, axis=0))


def test_closed_forms():
    g = np.random.default_rng(1)
    d = 32
    V = g.standard_normal((50, d))
    q = g.standard_normal((2, d))
    # all keys equal -> plain mean of V
    K = np.repeat(g.standard_normal((1, d)), 50, axis=0)
    assert np.allclose(A.attend(q, K, V, 0.3), V.mean(axis=0)[None], atol=1e-14, rtol=0)
    # zero query -> plain mean of V
    assert np.allclose(A.attend(np.zeros((1, d)), g.standard_normal((50, d)), V, 0.3),
                       V.mean(axis=0)[None], atol=1e-14, rtol=0)
    # all values equal -> that value
    c = g.standard_normal(d)
    assert np.allclose(A.attend(q, g.standard_normal((50, d)), np.tile(c, (50, 1)), 0.3), c[None], atol=1e-14)
    # two rows whose scores differ by ln 3 -> weights 3/4 and 1/4
    qq = np.zeros((1, d)); qq[0, 0] = math.sqrt(d)
    KK = np.zeros((2, d)); KK[0, 0] = math.log(3.0)
    VV = g.standard_normal((2, d))
    assert np.allclose(A.attend(qq, KK, VV, 1 / math.sqrt(d)), 0.75 * VV[0] + 0.25 * VV[1], atol=1e-15)


def test_matches_pure_python_brute_force():
    g = np.random.default_rng(2)
    for L, d, G in [(1, 4, 1), (7, 8, 2), (64, 16, 4), (33, 5, 3)]:
        q = g.standard_normal((G, d))
        K = g.standard_normal((L, d))
        V = g.standard_normal((L, d))
        sc = 1 / math.sqrt(d)
        o = A.attend(q, K, V, sc)
        for gi in range(G):
            s = [math.fsum(q[gi, i] * K[t, i] for i in range(d)) * sc for t in range(L)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for i in range(d):
                ref = math.fsum(e[t] * V[t, i] for t in range(L)) / z
                assert abs(o[gi, i] - ref) < 1e-12


def test_row_order_invariance():
    g = np.random.default_rng(3)
    q = g.standard_normal((4, 64))
    K = g.standard_normal((300, 64))
    V = g.standard_normal((300, 64))
    perm = g.permutation(300)
    assert np.max(np.abs(A.attend(q, K, V, 0.125) - A.attend(q, K[perm], V[perm], 0.125))) < 1e-13


def test_lse_merge_split_invariance():
    g = np.random.default_rng(4)
    q = g.standard_normal((4, 32))
    K = 3 * g.standard_normal((500, 32))
    V = g.standard_normal((500, 32))
    full = A.attend(q, K, V, 0.2)
    for cuts in ([250], [1, 2, 3, 499], sorted(g.choice(np.arange(1, 500), 17, replace=False))):
        b = [0, *cuts, 500]
        parts = [A.partial(q, K[b[i]:b[i + 1]], V[b[i]:b[i + 1]], 0.2) for i in range(len(b) - 1)]
        m = np.stack([p[0] for p in parts]); l = np.stack([p[1] for p in parts])
        acc = np.stack([p[2] for p in parts])
        assert np.max(np.abs(A.lse_merge(m, l, acc) - full)) < 1e-12


def test_int8_rows_equal_attention_over_same_bf16_values():
    # rows that are integer multiples of 2^-5 with absmax 127*2^-5 per channel
    # quantise exactly, so the INT8 tier must give the bf16 result
    g = np.random.default_rng(5)
    k = g.integers(-127, 128, size=(128, 64)); k[0] = 127; k[64] = -127
    v = g.integers(-127, 128, size=(128, 64)); v[3] = 127; v[70] = 127
    Kx = (k * 2.0 ** -5).astype(np.float32)
    Vx = (v * 2.0 ** -5).astype(np.float32)
    qk, sk = quant.quantize_rows(Kx, 64)
    qv, sv = quant.quantize_rows(Vx, 64)
    q = g.standard_normal((4, 64))
    a = A.attend(q, quant.dequantize_rows(qk, sk, 64), quant.dequantize_rows(qv, sv, 64), 0.125)
    b = A.attend(q, Kx.astype(np.float64), Vx.astype(np.float64), 0.125)
    assert np.max(np.abs(a - b)) < 1e-12


def test_workload_tier_rows_oldest_quantised_newest_exact():
    w = make_workload("tiered", B=1, Hkv=2, Hq=4, ctx=("fixed", 1000))
    res = A.reserve_for(w)
    n8 = res.n_i8[0][1]
    assert n8 == 832 and res.n_bf[0][1] == 168
    K, V = A.head_rows(w, res, 0, 1)
    K16, V16 = w.logical_kv(0, 1, res.L[0][1])
    Kb, Vb = A.bf16_to_f64(K16), A.bf16_to_f64(V16)
    assert np.array_equal(K[n8:], Kb[n8:]) and np.array_equal(V[n8:], Vb[n8:])
    for X, Xb in ((K, Kb), (V, Vb)):
        for blk in range(n8 // 64):
            sl = slice(64 * blk, 64 * blk + 64)
            step = np.abs(Xb[sl]).max(axis=0) / 127
            assert np.all(np.abs(X[sl] - Xb[sl]) <= step * (0.5 + 2.0 ** -10) + 1e-30)
        assert not np.array_equal(X[:n8], Xb[:n8])


def test_gqa_mapping_and_scale_default():
    # each q-head reads its own KV-head (hq // G), with scale 1/sqrt(d)
    w = make_workload("llama8b", B=1, ctx=("uniform", 64, 64), ratio_ppm=(1_000_000, 1_000_000), n_clusters=1)
    res = A.reserve_for(w)
    q = A.q_f64(w)
    o = A.decode(w, res)
    for hq in (0, 3, 4, 31):
        h = hq // 4
        K16, V16 = w.logical_kv(0, h, 64)
        ref = A.attend(q[0, hq:hq + 1], A.bf16_to_f64(K16), A.bf16_to_f64(V16), 1 / math.sqrt(128))
        assert np.max(np.abs(o[0, hq] - ref[0])) < 1e-14


def test_int4_workload_rows_within_half_a_step_and_exact_multiples():
    w = make_workload("tiered4", B=1, Hkv=2, Hq=4, ctx=("fixed", 1000))
    assert w.old_bits == 4
    res = A.reserve_for(w)
    n8 = res.n_i8[0][0]
    K, V = A.head_rows(w, res, 0, 0)
    K16, V16 = w.logical_kv(0, 0, res.L[0][0])
    Kb, Vb = A.bf16_to_f64(K16), A.bf16_to_f64(V16)
    assert np.array_equal(K[n8:], Kb[n8:])
    for X, Xb in ((K, Kb), (V, Vb)):
        for blk in range(n8 // 64):
            sl = slice(64 * blk, 64 * blk + 64)
            step = np.abs(Xb[sl]).max(axis=0) / 7
            assert np.all(np.abs(X[sl] - Xb[sl]) <= step * (0.5 + 2.0 ** -10) + 1e-30)
    # rows that are multiples of 2^-3 within +-7 * 2^-3 quantise exactly to 4 bits
    g = np.random.default_rng(6)
    k = g.integers(-7, 8, size=(128, 64)); k[0] = 7; k[64] = -7
    Kx = (k * 2.0 ** -3).astype(np.float32)
    qk, sk = quant.quantize_rows(Kx, 64, 4)
    assert np.array_equal(quant.dequantize_rows(qk, sk, 64), Kx.astype(np.float64))


def test_lse_merge_ignores_partials_with_no_rows():
    # a partial over no rows (m = -inf, l = 0, acc = 0) leaves the merge
    # unchanged, wherever it sits among the others
    g = np.random.default_rng(7)
    q = g.standard_normal((2, 16))
    K = g.standard_normal((90, 16))
    V = g.standard_normal((90, 16))
    parts = [A.partial(q, K[a:b], V[a:b], 0.25) for a, b in ((0, 30), (30, 31), (31, 90))]
    empty = (np.full(2, -np.inf), np.zeros(2), np.zeros((2, 16)))
    full = A.attend(q, K, V, 0.25)
    for at in (0, 2, 3):
        ps = parts[:at] + [empty] + parts[at:]
        o = A.lse_merge(np.stack([p[0] for p in ps]), np.stack([p[1] for p in ps]), np.stack([p[2] for p in ps]))
        assert np.max(np.abs(o - full)) < 1e-13


def test_bf16_decoder_on_fixed_patterns():
    """Hand-checked patterns of the bf16 format (sign, 8-bit exponent with
    bias 127, 7-bit fraction): the K/V bf16 rows of the fast tier (TTKV page,
    "Tier Layout") and bf16 queries enter the oracle through this decoder."""
    cases = {
        0x3F80: 1.0, 0xC040: -3.0, 0x4049: 3.140625, 0x3E80: 0.25, 0xBF00: -0.5,
        0x0001: 2.0 ** -133,                      # smallest subnormal
        0x0080: 2.0 ** -126,                      # smallest normal
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,   # largest finite
        0xFF7F: -(2.0 - 2.0 ** -7) * 2.0 ** 127,
        0x7F80: math.inf, 0xFF80: -math.inf, 0x0000: 0.0,
    }
    pats = np.array(list(cases), dtype=np.uint16)
    got = A.bf16_to_f64(pats)
    assert got.dtype == np.float64
    for u, g in zip(cases, got):
        assert g == cases[u], hex(u)
    neg0 = A.bf16_to_f64(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    assert math.isnan(A.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])


def test_bf16_decoder_on_every_pattern():
    """All 65536 patterns against the field-by-field reading of the format
    (NaN patterns must decode to NaN), and against the generator's fp32
    decoder, which must agree with it exactly."""
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        got = A.bf16_to_f64(allp)
    ref = _BF16_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    from workloads import bf16_bits_to_f32
    with np.errstate(invalid="ignore"):
        g32 = bf16_bits_to_f32(allp).astype(np.float64)
    assert np.array_equal(g32[~nan], ref[~nan])


@pytest.mark.parametrize("name", ["tiny", "llama8b", "tiered"])
def test_q_f64_decodes_the_query_bits(name):
    """q_f64: fp32 queries (Tiny) pass through unchanged, bf16 queries decode
    through the format fields."""
    w = make_workload(name, B=2) if name != "tiny" else make_workload(name)
    q = A.q_f64(w)
    assert q.dtype == np.float64 and q.shape == (w.B, w.Hq, w.d)
    raw = w.q()
    if w.q_dtype == "f32":
        assert np.array_equal(q, np.asarray(raw, np.float64))
    else:
        assert raw.dtype == np.uint16
        assert np.array_equal(q, _bf16_table(raw))
