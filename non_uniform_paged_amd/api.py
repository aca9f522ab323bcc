"""Python binding of the C ABI in include/tg.h -- argument marshalling only.

Every computation happens in ``libtg.so``: the host planner (reservation,
pools, tables, plan) and the HIP kernels (cache fill, split decode, merge).
PyTorch is used here only to own device memory and to name the stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _lib as L
from ._lib import TG_BENCH_READ_BLOCKS, TG_GROUP_WIDTH, TG_Q_BF16, TG_Q_F32, TG_TIER_BF16, TG_TIER_I8, TGError, check, lib

__all__ = [
    "TGError", "TG_TIER_I8", "TG_TIER_BF16", "TG_Q_F32", "TG_Q_BF16", "TG_GROUP_WIDTH",
    "Reservation", "Share", "Pool", "Tables", "DeviceCache",
    "tg_reserve", "tg_size_tables", "tg_build_tables", "tg_release", "tg_check_tables",
    "tg_write_kv", "tg_decode_workspace_bytes", "tg_decode_attn", "tg_decode_attn_noalloc", "tg_decode_split",
    "tg_decode_split_timed",
    "tg_merge_partials", "tg_bench_read", "tg_bench_streams", "TG_BENCH_READ_BLOCKS", "tg_append_kv",
    "tg_stream_order", "tg_stream_staging_bytes", "tg_decode_streamed",
    "tg_zip_bound", "tg_zip_workspace_bytes", "tg_zip_encode", "tg_zip_decode", "zip_compressed_bytes",
]


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _p32(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(L.P32)


# --------------------------------------------------------------------------- host
class Reservation:
    """Output of ``tg_reserve`` as numpy arrays (kept alive with the struct)."""

    def __init__(self, B: int, H: int, C: int):
        self.B, self.H, self.C = B, H, C
        self.budget = np.zeros((B, H), np.int32)
        self.length = np.zeros((B, H), np.int32)
        self.n_i8 = np.zeros((B, H), np.int32)
        self.n_bf = np.zeros((B, H), np.int32)
        self.cluster_of_head = np.zeros(H, np.int32)
        self.slot_in_cluster = np.zeros(H, np.int32)
        self.cluster_size = np.zeros(C, np.int32)
        self.struct = L.Reservation(0, 0, 0, _p32(self.budget), _p32(self.length), _p32(self.n_i8),
                                    _p32(self.n_bf), _p32(self.cluster_of_head),
                                    _p32(self.slot_in_cluster), _p32(self.cluster_size))


def tg_reserve(head_rank: Sequence[int], ratio_hi_ppm: int, ratio_lo_ppm: int, n_clusters: int,
               recent_ppm: int, quant_block: int, n_comp: Sequence[int],
               n_fixed: Optional[Sequence[int]] = None,
               budget_override: Optional[Sequence[int]] = None) -> Reservation:
    rank = _i32(head_rank)
    nc = _i32(n_comp)
    nf = None if n_fixed is None else _i32(n_fixed)
    ov = None if budget_override is None else _i32(budget_override)
    H, B = int(rank.size), int(nc.size)
    if nf is not None and nf.size != B:
        raise ValueError("n_fixed must have B entries")
    if ov is not None and ov.size != B * H:
        raise ValueError("budget_override must have B*H entries")
    res = Reservation(B, H, max(int(n_clusters), 1))
    tb = L.BudgetTable(H, _p32(rank), int(ratio_hi_ppm), int(ratio_lo_ppm), int(n_clusters),
                       int(recent_ppm), int(quant_block))
    check(lib().tg_reserve(ctypes.byref(tb), B, _p32(nc), _p32(nf), _p32(ov), ctypes.byref(res.struct)),
          "tg_reserve")
    return res


class Share:
    """Radix paths of the batch (``tg_share_desc``)."""

    def __init__(self, n_nodes: Sequence[int], node_ids: Sequence[int], node_len: Sequence[int]):
        self.n_nodes = _i32(n_nodes)
        self.node_ids = _i32(node_ids)
        self.node_len = _i32(node_len)
        self.struct = L.ShareDesc(_p32(self.n_nodes), _p32(self.node_ids), int(self.node_len.size),
                                  _p32(self.node_len))


def _share_ptr(share: Optional[Share]):
    return None if share is None else ctypes.byref(share.struct)


class Pool:
    """Host bookkeeping of the (cluster, tier) page pools (``tg_pool``)."""

    def __init__(self, cluster_size: Sequence[int], head_dim: int, page_size: int, quant_block: int,
                 pages_bf: Sequence[int], pages_i8: Sequence[int], old_bits: int = 8):
        cs = _i32(cluster_size)
        self.C = int(cs.size)
        self.cluster_size = cs.copy()
        self.head_dim, self.page_size, self.quant_block = int(head_dim), int(page_size), int(quant_block)
        self.old_bits = int(old_bits)
        pb = np.ascontiguousarray(pages_bf, dtype=np.int64)
        pi = np.ascontiguousarray(pages_i8, dtype=np.int64)
        if pb.size != self.C or pi.size != self.C:
            raise ValueError("pages_bf and pages_i8 need one entry per cluster")
        h = ctypes.c_void_p()
        check(lib().tg_pool_create(self.C, _p32(cs), self.head_dim, self.page_size, self.quant_block,
                                   self.old_bits, pb.ctypes.data_as(L.P64), pi.ctypes.data_as(L.P64),
                                   ctypes.byref(h)),
              "tg_pool_create")
        self.handle = h

    def page_bytes(self, c: int, tier: int) -> int:
        return int(lib().tg_pool_page_bytes(self.handle, c, tier))

    def capacity(self, c: int, tier: int) -> int:
        return int(lib().tg_pool_capacity(self.handle, c, tier))

    def free_pages(self, c: int, tier: int) -> int:
        return int(lib().tg_pool_free_pages(self.handle, c, tier))

    def refcount(self, c: int, tier: int, page: int) -> int:
        return int(lib().tg_pool_refcount(self.handle, c, tier, page))

    def close(self):
        if self.handle:
            lib().tg_pool_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tg_size_tables(res: Reservation, page_size: int, quant_block: int, share: Optional[Share] = None,
                   chunk_bf: int = 1024, chunk_i8: int = 1024, lpt: bool = True,
                   group_size: int = 0, gen_tokens: int = 0, chunk_group: int = 0) -> dict:
    opts = L.PlanOpts(int(chunk_bf), int(chunk_i8), int(bool(lpt)), int(group_size), int(gen_tokens),
                      int(chunk_group))
    sz = L.TableSizes()
    check(lib().tg_size_tables(ctypes.byref(res.struct), int(page_size), int(quant_block),
                               _share_ptr(share), ctypes.byref(opts), ctypes.byref(sz)), "tg_size_tables")
    C = res.C
    return {"stride": [[sz.stride[c][t] for t in range(2)] for c in range(C)],
            "n_items": int(sz.n_items), "n_gitems": int(sz.n_gitems), "n_slots": int(sz.n_slots),
            "pages_needed": [[int(sz.pages_needed[c][t]) for t in range(2)] for c in range(C)]}


class Tables:
    """Block tables, lengths and plan filled by ``tg_build_tables`` (numpy)."""

    def __init__(self, res: Reservation, sizes: dict):
        B, H, C = res.B, res.H, res.C
        self.B, self.H, self.C = B, H, C
        self.stride = sizes["stride"]
        self.n_items = sizes["n_items"]
        self.n_gitems = sizes["n_gitems"]
        self.n_slots = sizes["n_slots"]
        self.bt = [[np.full((B, self.stride[c][t]), -1, np.int32) for t in range(2)] for c in range(C)]
        self.len = np.zeros((B, H, 2), np.int32)
        self.work = np.zeros((max(self.n_items, 1), 6), np.int32)
        self.part_off = np.zeros(B * H + 1, np.int32)
        self.released = np.zeros(B, np.int32)
        self.gitems_buf = np.full((max(self.n_gitems, 1), L.TG_GROUP_WIDTH, 2), -1, np.int32)
        self.ring = np.zeros((B, C), np.int32)
        self.gen_tokens = 0
        s = L.Tables()
        for c in range(C):
            for t in range(2):
                s.bt[c][t] = _p32(self.bt[c][t]) if self.stride[c][t] else None
                s.stride[c][t] = self.stride[c][t]
        s.len = _p32(self.len)
        s.work = _p32(self.work)
        s.n_items = self.n_items
        s.part_off = _p32(self.part_off)
        s.released = _p32(self.released)
        s.gitems = _p32(self.gitems_buf)
        s.n_gitems = self.n_gitems
        s.ring = _p32(self.ring)
        self.struct = s

    @property
    def plan(self) -> np.ndarray:
        return self.work[:self.n_items]

    @property
    def gitems(self) -> np.ndarray:
        """[n_gitems][TG_GROUP_WIDTH][2] member table (request, slot)."""
        return self.gitems_buf[:self.n_gitems]

    @property
    def stride_has_i8(self) -> bool:
        return any(self.stride[c][0] > 0 for c in range(self.C))


def tg_build_tables(pool: Pool, res: Reservation, share: Optional[Share] = None, chunk_bf: int = 1024,
                    chunk_i8: int = 1024, lpt: bool = True, group_size: int = 0,
                    gen_tokens: int = 0, chunk_group: int = 0) -> Tables:
    sizes = tg_size_tables(res, pool.page_size, pool.quant_block, share, chunk_bf, chunk_i8, lpt, group_size,
                           gen_tokens, chunk_group)
    t = Tables(res, sizes)
    t.gen_tokens = int(gen_tokens)
    opts = L.PlanOpts(int(chunk_bf), int(chunk_i8), int(bool(lpt)), int(group_size), int(gen_tokens),
                      int(chunk_group))
    check(lib().tg_build_tables(pool.handle, ctypes.byref(res.struct), _share_ptr(share),
                                ctypes.byref(opts), ctypes.byref(t.struct)), "tg_build_tables")
    t.sizes = sizes
    return t


def tg_release(pool: Pool, tables: Tables, r: int) -> None:
    if not 0 <= r < tables.B:
        raise IndexError(r)
    check(lib().tg_release(pool.handle, ctypes.byref(tables.struct), int(r)), "tg_release")


def tg_check_tables(pool: Pool, res: Reservation, tables: Tables) -> None:
    """Host consistency check of built (or edited) tables; raises TGError
    with the library's description of the first failed check."""
    buf = ctypes.create_string_buffer(512)
    st = lib().tg_check_tables(pool.handle, ctypes.byref(res.struct), ctypes.byref(tables.struct), buf,
                               ctypes.sizeof(buf))
    if st != L.TG_OK:
        raise L.TGError(st, "tg_check_tables: " + buf.value.decode())


def tg_decode_workspace_bytes(n_slots: int, G: int, d: int) -> int:
    return int(lib().tg_decode_workspace_bytes(int(n_slots), int(G), int(d)))


# --------------------------------------------------------------------------- device
def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class DeviceCache:
    """Device memory of one populated cache: the (cluster, tier) pools sized
    from ``pool`` and the uploaded tables, plus the ``tg_cache`` view.
    ``head_major``: pools head-major (each head slot's pages contiguous)
    instead of page-major, for every pool (a bool) or by tier (a pair: INT8
    pools, bf16 pools); the same bytes, pages and outputs either way."""

    def __init__(self, pool: Pool, res: Reservation, tables: Tables, device="cuda",
                 share: Optional[Share] = None, head_major=False):
        torch = _torch()
        self.device = torch.device(device)
        hm = tuple(head_major) if isinstance(head_major, (tuple, list)) else (head_major, head_major)
        self.head_major = (bool(hm[0]), bool(hm[1]))
        self.G_hint = None
        C = res.C
        self.pools = [[None, None] for _ in range(C)]
        self.bt = [[None, None] for _ in range(C)]
        c_s = L.Cache()
        c_s.B, c_s.n_kv_heads, c_s.head_dim = res.B, res.H, pool.head_dim
        c_s.page_size, c_s.quant_block, c_s.n_clusters = pool.page_size, pool.quant_block, C
        for c in range(C):
            for t in range(2):
                cap = pool.capacity(c, t)
                pb = pool.page_bytes(c, t)
                if cap > 0:
                    self.pools[c][t] = torch.empty(cap * pb, dtype=torch.uint8, device=self.device)
                if tables.stride[c][t] > 0:
                    self.bt[c][t] = torch.from_numpy(tables.bt[c][t]).to(self.device)
                c_s.pool[c][t] = _ptr(self.pools[c][t])
                c_s.page_bytes[c][t] = pb
                c_s.n_pages[c][t] = cap
                c_s.head_major[c][t] = int(self.head_major[t])
                c_s.bt[c][t] = _ptr(self.bt[c][t])
                c_s.stride[c][t] = tables.stride[c][t]
        self.cluster_of_head = torch.from_numpy(res.cluster_of_head).to(self.device)
        self.slot_in_cluster = torch.from_numpy(res.slot_in_cluster).to(self.device)
        self.len = torch.from_numpy(tables.len.reshape(-1).copy()).to(self.device)
        self.work = torch.from_numpy(tables.plan.copy()).to(self.device)
        self.part_off = torch.from_numpy(tables.part_off).to(self.device)
        self.n_items = tables.n_items
        self.n_gitems = tables.n_gitems
        self.n_slots = tables.n_slots
        self.gitems = (torch.from_numpy(tables.gitems.reshape(-1).copy()).to(self.device)
                       if tables.n_gitems else None)
        c_s.cluster_of_head = _ptr(self.cluster_of_head)
        c_s.slot_in_cluster = _ptr(self.slot_in_cluster)
        c_s.len = _ptr(self.len)
        self.n_fixed = None
        nf = res.length[:, 0] - res.budget[:, 0]
        if share is not None and int(nf.max()) > 0:
            self.n_fixed = torch.from_numpy(np.ascontiguousarray(nf, dtype=np.int32)).to(self.device)
        c_s.n_fixed = _ptr(self.n_fixed)
        # decode-step growth: the bf16 ring and its offsets
        self.ring = self.bf_base = None
        if tables.gen_tokens > 0:
            self.ring = torch.from_numpy(tables.ring.reshape(-1).copy()).to(self.device)
            self.bf_base = torch.zeros(res.B * res.H, dtype=torch.int32, device=self.device)
        c_s.ring = _ptr(self.ring)
        c_s.bf_base = _ptr(self.bf_base)
        c_s.recent_ppm = int(res.struct.recent_ppm)
        c_s.old_bits = pool.old_bits
        self.struct = c_s
        self.B, self.H, self.d = res.B, res.H, pool.head_dim

    def slot_offset(self, c: int, t: int, page: int, slot: int, pool: "Pool") -> int:
        """Byte offset of head slot ``slot`` of page ``page`` in pool (c, t)."""
        pb, cap = pool.page_bytes(c, t), pool.capacity(c, t)
        hb = pb // int(pool.cluster_size[c])
        if self.struct.head_major[c][t]:
            return (slot * cap + page) * hb
        return page * pb + slot * hb

    def pool_bytes(self) -> int:
        return sum(int(p.numel()) for row in self.pools for p in row if p is not None)


def tg_write_kv(cache: DeviceCache, rows, index, offsets, stream=None) -> None:
    torch = _torch()
    _dev(rows, "rows")
    _dev(index, "index", 0, (torch.int32,))
    _dev(offsets, "offsets", (int(cache.B) * int(cache.H) + 1) * 8, (torch.int64,))
    check(lib().tg_write_kv(ctypes.byref(cache.struct), _ptr(rows), _ptr(index), _ptr(offsets),
                            _stream_ptr(stream)), "tg_write_kv")


def _dev(t, name: str, min_bytes: int = 0, dtypes=None):
    """Check that ``t`` is a contiguous device tensor of at least
    ``min_bytes`` bytes (and of one of ``dtypes``): the C calls take raw
    pointers and cannot see a buffer's size, so a short buffer would be read
    or written past its end on the device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {[str(d) for d in dtypes]}, not {t.dtype}")
    if t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {min_bytes}")
    return t


def _decode_args(cache, q, out, workspace, n_q_heads, sm_scale, work=None):
    torch = _torch()
    if q.dtype == torch.float32:
        qd = TG_Q_F32
    elif q.dtype == torch.bfloat16:
        qd = TG_Q_BF16
    else:
        raise TypeError("q must be float32 or bfloat16")
    rows = int(cache.B) * int(n_q_heads) * int(cache.d)
    _dev(q, "q", rows * q.element_size())
    if out is not None:
        _dev(out, "out", rows * 4, (torch.float32,))
    if workspace is not None:
        _dev(workspace, "workspace")
    _dev(cache.work if work is None else work, "work", int(cache.n_items) * 24, (torch.int32,))
    a = L.DecodeArgs()
    a.n_q_heads = int(n_q_heads)
    a.q_dtype = qd
    a.q = _ptr(q)
    a.work = _ptr(cache.work if work is None else work)
    a.n_items = int(cache.n_items)
    a.part_off = _ptr(cache.part_off)
    a.gitems = _ptr(cache.gitems)
    a.n_gitems = int(cache.n_gitems)
    a.n_slots = int(cache.n_slots)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    a.out = _ptr(out)
    a.sm_scale = float(sm_scale)
    return a


def tg_decode_attn(cache: DeviceCache, q, out, workspace, n_q_heads: int, sm_scale: float = 0.0,
                   stream=None) -> None:
    """Enqueue one decode step with the plan uploaded with the cache.  ``q``
    is fp32 or bf16 [B][Hq][d] on the device; ``out`` fp32 [B][Hq][d];
    ``workspace`` fp32 of at least ``tg_decode_workspace_bytes(n_slots)``
    bytes."""
    a = _decode_args(cache, q, out, workspace, n_q_heads, sm_scale)
    check(lib().tg_decode_attn(ctypes.byref(cache.struct), ctypes.byref(a), _stream_ptr(stream)),
          "tg_decode_attn")


def tg_decode_attn_noalloc(cache: DeviceCache, q, out, n_q_heads: int, sm_scale: float = 0.0,
                           stream=None) -> None:
    """tg_decode_attn with the partials in the library's fixed device array
    (no workspace argument, nothing allocated by the call); TGError
    TG_EOVERFLOW when the plan's partials exceed TG_NOALLOC_SCRATCH_BYTES."""
    a = _decode_args(cache, q, out, None, n_q_heads, sm_scale)
    check(lib().tg_decode_attn_noalloc(ctypes.byref(cache.struct), ctypes.byref(a), _stream_ptr(stream)),
          "tg_decode_attn_noalloc")


def tg_decode_split(cache: DeviceCache, q, workspace, n_q_heads: int, sm_scale: float = 0.0,
                    stream=None) -> None:
    """Enqueue the split stage alone (partials into ``workspace``)."""
    a = _decode_args(cache, q, None, workspace, n_q_heads, sm_scale)
    check(lib().tg_decode_split(ctypes.byref(cache.struct), ctypes.byref(a), _stream_ptr(stream)),
          "tg_decode_split")


def _event_ptr(ev, stream):
    """Raw hipEvent_t of a torch.cuda.Event (created by a first record on
    ``stream`` if it has none yet), for the launches that record a kernel's own
    start and end into it."""
    if ev.cuda_event == 0:
        ev.record(stream)
    return ctypes.c_void_p(ev.cuda_event)


def _events(events, stream):
    if events is None:
        return None, None
    start, stop = events
    return _event_ptr(start, stream), _event_ptr(stop, stream)


def tg_decode_split_timed(cache: DeviceCache, q, workspace, n_q_heads: int, events, sm_scale: float = 0.0,
                          stream=None) -> None:
    """tg_decode_split with the split kernel's own start and end recorded
    into ``events`` (two torch.cuda.Event with timing enabled), so that
    ``events[0].elapsed_time(events[1])`` is the kernel's execution alone."""
    a = _decode_args(cache, q, None, workspace, n_q_heads, sm_scale)
    e0, e1 = _events(events, _torch().cuda.current_stream() if stream is None else stream)
    check(lib().tg_decode_split_timed(ctypes.byref(cache.struct), ctypes.byref(a), e0, e1, _stream_ptr(stream)),
          "tg_decode_split_timed")


def tg_merge_partials(workspace, n_slots: int, n_pairs: int, G: int, d: int, part_off, out,
                      stream=None) -> None:
    torch = _torch()
    _dev(workspace, "workspace", int(n_slots) * int(G) * (int(d) + 2) * 4)
    _dev(part_off, "part_off", (int(n_pairs) + 1) * 4, (torch.int32,))
    _dev(out, "out", int(n_pairs) * int(G) * int(d) * 4, (torch.float32,))
    check(lib().tg_merge_partials(_ptr(workspace), int(n_slots), int(n_pairs), int(G), int(d),
                                  _ptr(part_off), _ptr(out), _stream_ptr(stream)), "tg_merge_partials")


def tg_bench_read(src, sink, stream=None, events=None) -> None:
    """Streaming read of the whole of ``src`` (a device tensor, size a
    multiple of 16 bytes); ``sink`` is a device int32 tensor of at least
    TG_BENCH_READ_BLOCKS elements.  ``events``: None, or two torch.cuda.Event
    that receive the kernel's own start and end."""
    if sink.numel() * sink.element_size() < 4 * TG_BENCH_READ_BLOCKS:
        raise ValueError("sink too small")
    e0, e1 = _events(events, _torch().cuda.current_stream() if stream is None else stream)
    check(lib().tg_bench_read(_ptr(src), int(src.numel() * src.element_size()), _ptr(sink), e0, e1,
                              _stream_ptr(stream)), "tg_bench_read")


def tg_bench_streams(src, chunk, off, sink, stream=None, events=None) -> None:
    """Independent streams of 8 KiB chunks of ``src`` (device tensor, size a
    multiple of 8192 bytes): stream w reads chunk[off[w]:off[w + 1]] (device
    int32 tensors) one wavefront at a time, as a decode item reads its pages;
    ``sink`` (device int32, len(off) - 1 elements) receives each stream's XOR
    fold.  ``events``: as for ``tg_bench_read``."""
    torch = _torch()
    n = int(off.numel()) - 1
    if n < 0 or sink.numel() < n:
        raise ValueError("off must have n_streams + 1 entries and sink n_streams")
    _dev(src, "src")
    _dev(chunk, "chunk", 0, (torch.int32,))
    _dev(off, "off", 0, (torch.int32,))
    _dev(sink, "sink", 4 * n)
    e0, e1 = _events(events, torch.cuda.current_stream() if stream is None else stream)
    check(lib().tg_bench_streams(_ptr(src), int(src.numel() * src.element_size()), _ptr(chunk), _ptr(off), n,
                                 _ptr(sink), e0, e1, _stream_ptr(stream)), "tg_bench_streams")


def tg_append_kv(cache: DeviceCache, rows, status=None, stream=None) -> None:
    """Append one row per (r, h) (device uint16/int16 [B*H][2][d] bf16 bits)
    and age the oldest bf16 block into INT8 where the tier split says so;
    ``status`` (device int32, optional) gets bit 0 if a (r, h) ran out of the
    reserved capacity."""
    _dev(rows, "rows", int(cache.B) * int(cache.H) * 2 * int(cache.d) * 2)
    if status is not None:
        _dev(status, "status", 4)
    check(lib().tg_append_kv(ctypes.byref(cache.struct), _ptr(rows), _ptr(status), _stream_ptr(stream)),
          "tg_append_kv")


def tg_stream_order(tables: Tables):
    """(work [n_items][6] int32, chunk_off [B+1] int32): the plan reordered
    for tg_decode_streamed."""
    work = np.zeros((max(tables.n_items, 1), 6), np.int32)
    off = np.zeros(tables.B + 1, np.int32)
    check(lib().tg_stream_order(ctypes.byref(tables.struct), tables.B, _p32(work), _p32(off)), "tg_stream_order")
    return work[:tables.n_items], off


def tg_stream_staging_bytes(cache: DeviceCache, tables: Tables) -> int:
    return int(lib().tg_stream_staging_bytes(ctypes.byref(cache.struct), ctypes.byref(tables.struct)))


def tg_decode_streamed(cache: DeviceCache, tables: Tables, q, out, workspace, n_q_heads: int, work, chunk_off,
                       staging, sm_scale: float = 0.0, stream=None) -> None:
    """Decode step with the INT8 pages in pinned host memory (the cache's
    INT8 pool pointers), streamed through ``staging``; ``work`` is the device
    copy of ``tg_stream_order``'s plan, ``chunk_off`` its host offsets."""
    a = _decode_args(cache, q, out, workspace, n_q_heads, sm_scale, work=work)
    off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    check(lib().tg_decode_streamed(ctypes.byref(cache.struct), ctypes.byref(tables.struct), ctypes.byref(a),
                                   _p32(off), _ptr(staging), int(staging.numel() * staging.element_size()),
                                   _stream_ptr(stream)), "tg_decode_streamed")


# --------------------------------------------------------------------------- lossless codec
def tg_zip_bound(n: int) -> int:
    return int(lib().tg_zip_bound(int(n)))


def tg_zip_workspace_bytes(n: int) -> int:
    return int(lib().tg_zip_workspace_bytes(int(n)))


def tg_zip_encode(src, dst, workspace, stream=None) -> None:
    """Compress ``src`` (device int16/uint16 tensor of bf16 bits, size a
    multiple of 8) into ``dst`` (device, >= tg_zip_bound bytes)."""
    _dev(src, "src")
    _dev(dst, "dst")
    _dev(workspace, "workspace")
    check(lib().tg_zip_encode(_ptr(src), int(src.numel()), _ptr(dst), int(dst.numel() * dst.element_size()),
                              _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                              _stream_ptr(stream)), "tg_zip_encode")


def tg_zip_decode(src, n: int, dst, stream=None) -> None:
    _dev(src, "src")
    _dev(dst, "dst", int(n) * 2)
    check(lib().tg_zip_decode(_ptr(src), int(n), _ptr(dst), _stream_ptr(stream)), "tg_zip_decode")


def zip_compressed_bytes(buf) -> int:
    """Size of a compressed buffer from its header (reads 16 bytes back)."""
    h = buf[:16].cpu().numpy().view(np.int64)
    return 256 + int(h[0]) + int(h[0]) // 2 + 5 * int(h[1])
