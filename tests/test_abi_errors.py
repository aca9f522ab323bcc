"""Argument checks of the device entry points, on the CPU: each call below is
rejected by the library's host-side validation before anything reaches the
GPU, so these run without one.  The returned code is the one include/tg.h
documents for that mistake."""
import ctypes

import numpy as np
import pytest

from non_uniform_paged_amd import _lib as L


def _cache(d=128, B=2, H=2, C=1, page=16, qb=64, old_bits=8):
    c = L.Cache()
    c.B, c.n_kv_heads, c.head_dim = B, H, d
    c.page_size, c.quant_block, c.n_clusters = page, qb, C
    c.old_bits = old_bits
    c.recent_ppm = 1_000_000
    return c


def _args(**kw):
    a = L.DecodeArgs()
    a.n_q_heads = kw.get("n_q_heads", 4)
    a.q_dtype = kw.get("q_dtype", L.TG_Q_BF16)
    for k, v in kw.items():
        if k not in ("n_q_heads", "q_dtype"):
            setattr(a, k, v)
    return a


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_decode_rejects_missing_and_unsupported_arguments():
    lib = L.lib()
    assert lib.tg_decode_attn(None, None, None) == L.TG_EINVAL
    c = _cache()
    # no cluster tables, no q
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(_args()), None) == L.TG_EINVAL
    # q-heads not a multiple of the KV-heads
    c.cluster_of_head = c.slot_in_cluster = c.len = FAKE.value
    a = _args(n_q_heads=3, q=FAKE.value, out=FAKE.value, part_off=FAKE.value)
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL
    # head size and group size outside the supported set
    for d, nq in ((96, 4), (128, 6), (128, 32)):
        c2 = _cache(d=d)
        c2.cluster_of_head = c2.slot_in_cluster = c2.len = FAKE.value
        a = _args(n_q_heads=nq, q=FAKE.value, out=FAKE.value, part_off=FAKE.value)
        assert lib.tg_decode_attn(ctypes.byref(c2), ctypes.byref(a), None) == L.TG_EUNSUPPORTED, (d, nq)
    # INT4 is laid out for d = 128 only
    c3 = _cache(d=64, old_bits=4)
    c3.cluster_of_head = c3.slot_in_cluster = c3.len = FAKE.value
    a = _args(q=FAKE.value, out=FAKE.value, part_off=FAKE.value)
    assert lib.tg_decode_attn(ctypes.byref(c3), ctypes.byref(a), None) == L.TG_EUNSUPPORTED
    # bad q dtype; items without a workspace; a workspace too small for the slots
    a = _args(q_dtype=7, q=FAKE.value, out=FAKE.value, part_off=FAKE.value)
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL
    # the score scale must be finite and non-negative (0 = 1/sqrt(d))
    for bad in (-0.125, float("nan"), float("inf")):
        a = _args(q=FAKE.value, out=FAKE.value, part_off=FAKE.value, sm_scale=bad)
        assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL, bad
    a = _args(q=FAKE.value, out=FAKE.value, part_off=FAKE.value, n_items=5, work=FAKE.value, n_slots=5)
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL
    need = lib.tg_decode_workspace_bytes(5, 2, 128)
    assert need == 5 * 2 * (128 + 2) * 4
    a = _args(q=FAKE.value, out=FAKE.value, part_off=FAKE.value, n_items=5, work=FAKE.value, n_slots=5,
              workspace=FAKE.value, workspace_bytes=need - 4)
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL
    # group items without their member table
    a = _args(q=FAKE.value, out=FAKE.value, part_off=FAKE.value, n_gitems=1)
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL


def test_merge_write_append_reject_bad_arguments():
    lib = L.lib()
    assert lib.tg_merge_partials(None, 4, 2, 4, 96, None, None, None) == L.TG_EUNSUPPORTED
    assert lib.tg_merge_partials(None, 4, 2, 4, 128, None, None, None) == L.TG_EINVAL
    assert lib.tg_merge_partials(None, -1, 0, 4, 128, None, None, None) == L.TG_EINVAL
    assert lib.tg_write_kv(None, None, None, None, None) == L.TG_EINVAL
    c = _cache()
    c.cluster_of_head = c.slot_in_cluster = c.len = FAKE.value
    assert lib.tg_write_kv(ctypes.byref(c), None, None, None, None) == L.TG_EINVAL
    c64 = _cache(d=96)
    c64.cluster_of_head = c64.slot_in_cluster = c64.len = FAKE.value
    assert lib.tg_write_kv(ctypes.byref(c64), FAKE, FAKE, FAKE, None) == L.TG_EUNSUPPORTED
    # appending needs the growth ring
    assert lib.tg_append_kv(ctypes.byref(c), FAKE, None, None) == L.TG_EINVAL
    c.ring = c.bf_base = FAKE.value
    c.recent_ppm = 2_000_000
    assert lib.tg_append_kv(ctypes.byref(c), FAKE, None, None) == L.TG_EINVAL


def test_codec_and_read_aid_reject_bad_sizes():
    lib = L.lib()
    assert lib.tg_zip_bound(-1) == 0 and lib.tg_zip_workspace_bytes(-1) == 0
    n = 1 << 12
    assert lib.tg_zip_bound(n) >= 256 + n + n // 2
    for bad_n in (0, 7, 12, (1 << 32) + 8):
        assert lib.tg_zip_encode(FAKE, bad_n, FAKE, 1 << 40, FAKE, 1 << 40, None) == L.TG_EINVAL, bad_n
        assert lib.tg_zip_decode(FAKE, bad_n, FAKE, None) == L.TG_EINVAL, bad_n
    # destination or workspace smaller than the bounds
    assert lib.tg_zip_encode(FAKE, n, FAKE, lib.tg_zip_bound(n) - 1, FAKE, 1 << 40, None) == L.TG_EINVAL
    assert lib.tg_zip_encode(FAKE, n, FAKE, 1 << 40, FAKE, lib.tg_zip_workspace_bytes(n) - 1, None) == L.TG_EINVAL
    # misaligned pointers
    odd = ctypes.c_void_p(0x1008)
    assert lib.tg_zip_encode(odd, n, FAKE, 1 << 40, FAKE, 1 << 40, None) == L.TG_EINVAL
    assert lib.tg_zip_decode(FAKE, n, odd, None) == L.TG_EINVAL
    assert lib.tg_bench_read(FAKE, 24, FAKE, None, None, None) == L.TG_EINVAL
    # the timed split needs both events (checked before the arguments)
    c, a = _cache(), _args()
    assert lib.tg_decode_split_timed(ctypes.byref(c), ctypes.byref(a), None, FAKE, None) == L.TG_EINVAL
    assert lib.tg_decode_split_timed(ctypes.byref(c), ctypes.byref(a), FAKE, None, None) == L.TG_EINVAL
    assert lib.tg_bench_read(None, 32, FAKE, None, None, None) == L.TG_EINVAL
    # the paged-stream read: buffer of whole 8 KiB chunks, aligned, tables present
    for args in ((FAKE, 8192 + 16, FAKE, FAKE, 1), (FAKE, 0, FAKE, FAKE, 1), (odd, 8192, FAKE, FAKE, 1),
                 (FAKE, 8192, None, FAKE, 1), (FAKE, 8192, FAKE, None, 1), (FAKE, 8192, FAKE, FAKE, -1)):
        assert lib.tg_bench_streams(*args, FAKE, None, None, None) == L.TG_EINVAL, args
    assert lib.tg_bench_streams(FAKE, 8192, FAKE, FAKE, 1, None, None, None, None) == L.TG_EINVAL
    assert lib.tg_bench_streams(FAKE, 8192, None, None, 0, None, None, None, None) == L.TG_OK  # nothing to read


def test_status_strings_cover_every_code():
    lib = L.lib()
    lib.tg_strerror.restype = ctypes.c_char_p
    seen = set()
    for code in L.STATUS_NAMES:
        s = lib.tg_strerror(code)
        assert s and s not in seen
        seen.add(s)
    assert np.all([isinstance(x, bytes) for x in seen])


def test_python_binding_refuses_unfit_buffers():
    """The binding checks what the C calls cannot see behind a raw pointer:
    device placement, contiguity, dtype and size of every buffer, so that a
    short or host buffer is refused before any launch (CPU only: every case
    fails before the library is called)."""
    torch = pytest.importorskip("torch")
    from types import SimpleNamespace
    from non_uniform_paged_amd import api
    cache = SimpleNamespace(B=2, H=2, d=64, work=torch.zeros(6, dtype=torch.int32), n_items=1, part_off=None,
                            gitems=None, n_gitems=0, n_slots=1)
    q = torch.zeros(2 * 4 * 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be a device tensor"):
        api._decode_args(cache, q, None, q, 4, 0.0)
    with pytest.raises(TypeError, match="q must be float32 or bfloat16"):
        api._decode_args(cache, q.to(torch.float16), None, q, 4, 0.0)
    with pytest.raises(ValueError, match="rows must be a device tensor"):
        api.tg_append_kv(cache, torch.zeros(8, dtype=torch.int16))
    with pytest.raises(ValueError, match="workspace must be a device tensor"):
        api.tg_merge_partials(torch.zeros(4), 1, 1, 2, 64, torch.zeros(2, dtype=torch.int32), torch.zeros(128))
    with pytest.raises(ValueError, match="src must be a device tensor"):
        api.tg_zip_decode(torch.zeros(8, dtype=torch.int16), 8, torch.zeros(8, dtype=torch.int16))
    with pytest.raises(ValueError, match="rows must be a device tensor"):
        api.tg_write_kv(cache, torch.zeros(4, dtype=torch.int16), torch.zeros(1, dtype=torch.int32),
                        torch.zeros(5, dtype=torch.int64))


def test_pool_create_checks():
    """tg_pool_create: INT4 codes pack two to a byte, so a block of qb rows of
    d channels needs qb * d even; the other arguments as documented."""
    lib = L.lib()
    one = (ctypes.c_int32 * 1)(2)
    pages = (ctypes.c_int64 * 1)(3)
    neg = (ctypes.c_int64 * 1)(-1)

    def create(d, ps, qb, bits, n_c=one, pb=pages, pi=pages):
        out = ctypes.c_void_p()
        rc = lib.tg_pool_create(1, n_c, d, ps, qb, bits, pb, pi, ctypes.byref(out))
        if rc == L.TG_OK:
            lib.tg_pool_destroy(out)
        return rc

    assert create(128, 16, 64, 4) == L.TG_OK
    assert create(5, 16, 3, 4) == L.TG_EINVAL       # 15 codes: half a byte left over
    assert create(5, 16, 4, 4) == L.TG_OK
    assert create(6, 16, 3, 4) == L.TG_OK
    assert create(5, 16, 3, 8) == L.TG_OK           # INT8 codes: any shape
    assert create(128, 16, 64, 6) == L.TG_EINVAL    # only 8 or 4 bits
    assert create(128, 0, 64, 8) == L.TG_EINVAL
    assert create(128, 16, 64, 8, n_c=(ctypes.c_int32 * 1)(0)) == L.TG_EINVAL
    assert create(128, 16, 64, 8, pi=neg) == L.TG_EINVAL
    assert create(1 << 30, 16, 64, 8, pb=(ctypes.c_int64 * 1)(1 << 40)) == L.TG_EOVERFLOW


def test_noalloc_refuses_oversized_partials_before_any_launch():
    """tg_decode_attn_noalloc checks the partials' size against its fixed
    array on the host: more slots than fit give TG_EOVERFLOW, malformed head
    counts TG_EINVAL, without touching the device."""
    lib = L.lib()
    assert lib.tg_decode_attn_noalloc(None, None, None) == L.TG_EINVAL
    c = _cache()
    a = _args(n_q_heads=4)
    a.n_slots = L.TG_NOALLOC_SCRATCH_BYTES // (2 * 130 * 4) + 1  # G = 2, d = 128
    assert lib.tg_decode_attn_noalloc(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EOVERFLOW
    a.n_q_heads = 3  # not a multiple of the KV-heads
    assert lib.tg_decode_attn_noalloc(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL


def test_pool_layout_flags_are_checked():
    """tg_cache.head_major is 0 or 1 per (cluster, tier); anything else is
    refused by the decode, cache fill and append calls alike, and a page size
    that is not a whole number of head slots is refused too."""
    lib = L.lib()
    c = _cache()
    c.cluster_of_head = c.slot_in_cluster = c.len = FAKE.value
    c.ring = c.bf_base = FAKE.value
    a = _args(q=FAKE.value, out=FAKE.value, part_off=FAKE.value)
    for bad in (2, -1):
        c.head_major[0][1] = bad
        assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL, bad
        assert lib.tg_write_kv(ctypes.byref(c), FAKE, FAKE, FAKE, None) == L.TG_EINVAL, bad
        assert lib.tg_append_kv(ctypes.byref(c), FAKE, FAKE, None) == L.TG_EINVAL, bad
    c.head_major[0][1] = 1
    # a bf16 page of 1.5 head slots (d 128: 8 KiB a slot)
    c.stride[0][1] = 4
    c.bt[0][1] = c.pool[0][1] = FAKE.value
    c.page_bytes[0][1] = 3 * 4096
    c.n_pages[0][1] = 8
    assert lib.tg_decode_attn(ctypes.byref(c), ctypes.byref(a), None) == L.TG_EINVAL
    assert lib.tg_write_kv(ctypes.byref(c), FAKE, FAKE, FAKE, None) == L.TG_EINVAL
    assert lib.tg_append_kv(ctypes.byref(c), FAKE, FAKE, None) == L.TG_EINVAL
