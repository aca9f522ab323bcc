"""Drive one seeded workload through the library: admission, cache fill and
decode steps on one GPU.

This is the harness used by the GPU tests, ``smoke()`` and ``bench.py``; it
only marshals arguments into the C ABI (``api``) and owns device memory
through PyTorch.  ``w`` is any object with the fields of
``workloads.Workload``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import api


def tune_candidates(w, has_quantised: bool):
    """(chunk_bf, chunk_i8) pairs tune_chunks tries: bf16 item lengths from
    256 to 6144 rows, and with a quantised tier INT8 / INT4 lengths from 1024
    to 3072 rows against the shorter bf16 lengths."""
    if not has_quantised:
        return [(cb, 1024) for cb in (256, 384, 512, 640, 768, 832, 896, 960, 1024, 1280, 1536, 2048, 3072,
                                      4096, 6144)]
    return [(cb, ci) for cb in (384, 512, 768, 1024) for ci in (1024, 1536, 1792, 2048, 2304, 2560, 3072)]


# Plan item lengths (bf16 rows, quantised-tier rows) per workload, chosen by
# sweeping the split-kernel time on MI355X: the best length depends on how
# the item count falls against the ~2048 resident wavefronts and on the
# length mix.  The benchmark and the full-size parity tests both use them.
PLAN_CHUNKS = {"tiny": (1024, 1024), "llama8b": (896, 1024), "ragged": (4096, 1024),
               "tiered": (512, 1792), "tiered4": (512, 2048), "radix": (768, 1024)}


def reserve_workload(w) -> api.Reservation:
    return api.tg_reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                          w.quant_block, w.n_comp, w.n_fixed, w.budget_override)


def share_of(w) -> Optional[api.Share]:
    if getattr(w, "paths", None) is None:
        return None
    n_nodes = [len(p) for p in w.paths]
    ids = [n for p in w.paths for n in p]
    return api.Share(n_nodes, ids, w.node_len)


class Prepared:
    """A populated cache plus the buffers of one decode step."""

    def __init__(self, w, chunk_bf: int = 1024, chunk_i8: int = 1024, lpt: bool = True,
                 slack_pages: int = 0, shift_pages: int = 0, device: str = "cuda",
                 group_size: Optional[int] = None, gen_tokens: int = 0, chunk_group: int = 0,
                 head_major=None):
        """``group_size`` None: group shared-prefix pages for as many requests
        as a workgroup's four wavefronts score at once (two 16-column tiles
        each: 128 / G, at most 32) when the batch shares a radix prefix, else
        no groups.  ``gen_tokens`` > 0 reserves room for that
        many appended rows per (r, h) and stages them (the continuation of
        each sequence) on the device for ``append``.  ``chunk_group`` cuts
        group items with their own length (0: chunk_bf).  ``head_major``:
        pool layout (include/tg.h), a bool for every pool or a pair (INT8
        pools, bf16 pools); None chooses by measurement: bf16 pools
        head-major when the cache has no quantised tier (faster there), every
        other pool page-major (head-major bf16 pools beside a quantised tier
        measured no faster, and slower when the slot stride is a power of
        two)."""
        import torch

        self.w = w
        dev = torch.device(device)
        self.res = reserve_workload(w)
        self.share = share_of(w)
        G = w.Hq // w.Hkv
        if group_size is None:
            group_size = min(128 // G, api.TG_GROUP_WIDTH) if self.share is not None else 0
        self.group_size = group_size
        self.gen_tokens = gen_tokens
        self.chunk_group = chunk_group
        sizes = api.tg_size_tables(self.res, w.page_size, w.quant_block, self.share, chunk_bf, chunk_i8, lpt,
                                   group_size, gen_tokens, chunk_group)
        need = sizes["pages_needed"]
        C = self.res.C
        extra = slack_pages + shift_pages
        self.pool = api.Pool(self.res.cluster_size, w.d, w.page_size, w.quant_block,
                             [need[c][1] + extra for c in range(C)], [need[c][0] + extra for c in range(C)],
                             getattr(w, "old_bits", 8))
        fillers = []
        if shift_pages:
            # occupy the lowest shift_pages pages of both tiers first so that
            # this batch lands elsewhere: one all-bf16 and one all-INT8 request
            for recent, rows in ((10**6, w.page_size), (0, w.quant_block)):
                filler = api.tg_reserve(w.head_rank, 10**6, 10**6, C, recent, w.quant_block,
                                        [shift_pages * rows], None, None)
                fillers.append(api.tg_build_tables(self.pool, filler, None, w.page_size * 4, w.quant_block * 4,
                                                   False))
        self.tables = api.tg_build_tables(self.pool, self.res, self.share, chunk_bf, chunk_i8, lpt, group_size,
                                          gen_tokens, chunk_group)
        self.chunks = (chunk_bf, chunk_i8)
        for ftab in fillers:
            api.tg_release(self.pool, ftab, 0)
        if head_major is None:
            head_major = (False, int(self.res.n_i8.max()) == 0)
        self.cache = api.DeviceCache(self.pool, self.res, self.tables, dev, self.share, head_major)

        rows, index, offsets = w.source_buffer(self.res.length + gen_tokens)
        self.appended = None
        if gen_tokens > 0:
            # row L0 + k of every (r, h), step-major: [T][B*H][2][d]
            L0 = self.res.length.reshape(-1).astype(np.int64)
            src = index[offsets[:-1][None, :] + L0[None, :] + np.arange(gen_tokens)[:, None]]
            self.appended = torch.from_numpy(rows[src].view(np.int16)).to(dev)
            self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.steps_appended = 0
        self._write(rows, index, offsets)
        del rows

        qn = w.q()
        if w.q_dtype == "f32":
            self.q = torch.from_numpy(np.ascontiguousarray(qn, dtype=np.float32)).to(dev)
        else:
            self.q = torch.from_numpy(qn.view(np.int16)).to(dev).view(torch.bfloat16)
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        ws = api.tg_decode_workspace_bytes(self.tables.n_slots, G, w.d)
        self.workspace = torch.empty(max(ws // 4, 1), dtype=torch.float32, device=dev)

    def _write(self, rows, index, offsets) -> None:
        import torch
        dev = self.cache.device
        rows_t = torch.from_numpy(rows.view(np.uint16).reshape(-1).view(np.int16)).to(dev)
        index_t = torch.from_numpy(index).to(dev)
        off_t = torch.from_numpy(offsets).to(dev)
        api.tg_write_kv(self.cache, rows_t, index_t, off_t)
        torch.cuda.synchronize(dev)

    def rewrite_zeroed(self) -> None:
        """Zero every device pool and write the admitted rows again (bytes no
        row reaches are then 0 rather than whatever the allocation held)."""
        for row in self.cache.pools:
            for pool in row:
                if pool is not None:
                    pool.zero_()
        rows, index, offsets = self.w.source_buffer(self.res.length + self.gen_tokens)
        self._write(rows, index, offsets)

    # ------------------------------------------------------------------ plan
    def replan(self, chunk_bf: int, chunk_i8: int, lpt: bool = True) -> None:
        """Swap in the plan of other item lengths over the same pages: the
        tables are rebuilt on a fresh host pool of the same capacities (page
        allocation does not depend on the item lengths, so the block tables
        come out identical, which is checked) and the plan, its slot CSR and
        member table replace the device ones."""
        import torch
        w, C = self.w, self.res.C
        pool = api.Pool(self.res.cluster_size, w.d, w.page_size, w.quant_block,
                        [self.pool.capacity(c, api.TG_TIER_BF16) for c in range(C)],
                        [self.pool.capacity(c, api.TG_TIER_I8) for c in range(C)], getattr(w, "old_bits", 8))
        t = api.tg_build_tables(pool, self.res, self.share, chunk_bf, chunk_i8, lpt, self.group_size,
                                self.gen_tokens, self.chunk_group)
        for c in range(C):
            for tier in range(2):
                if not np.array_equal(t.bt[c][tier], self.tables.bt[c][tier]):
                    raise RuntimeError("replan: the block tables differ (pool not built from empty)")
        dev = self.cache.device
        self.cache.work = torch.from_numpy(t.plan.copy()).to(dev)
        self.cache.part_off = torch.from_numpy(t.part_off).to(dev)
        self.cache.gitems = torch.from_numpy(t.gitems.reshape(-1).copy()).to(dev) if t.n_gitems else None
        self.cache.n_items, self.cache.n_gitems, self.cache.n_slots = t.n_items, t.n_gitems, t.n_slots
        G = w.Hq // w.Hkv
        need = api.tg_decode_workspace_bytes(t.n_slots, G, w.d) // 4
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.float32, device=dev)
        self.tables = t
        self.chunks = (chunk_bf, chunk_i8)

    def tune_chunks(self, candidates, evict=None, steps: int = 8, stream=None):
        """Time the split stage for each (chunk_bf, chunk_i8) candidate over
        the same pages (``evict()`` runs before every timed step) and keep
        the fastest plan.  Returns [(chunk_bf, chunk_i8, median us)]."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        G = self.w.Hq // self.w.Hkv
        out = []
        for cb, ci in candidates:
            self.replan(cb, ci)
            ts = []
            for i in range(steps + 2):
                if evict is not None:
                    evict()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                api.tg_decode_split(self.cache, self.q, self.workspace, self.w.Hq, stream=s)
                e1.record(s)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            out.append((cb, ci, float(np.median([a.elapsed_time(b) for a, b in ts[2:]])) * 1e3))
        best = min(out, key=lambda x: x[2])
        self.replan(best[0], best[1])
        return out

    # ------------------------------------------------------------------ run
    def step(self, stream=None, sm_scale: float = 0.0):
        """One decode step over the uploaded plan; ``sm_scale`` 0 means 1/sqrt(d)."""
        if getattr(self, "host_i8", False):
            raise RuntimeError("the INT8 pages are in host memory: use step_streamed")
        api.tg_decode_attn(self.cache, self.q, self.out, self.workspace, self.w.Hq, sm_scale, stream=stream)

    # ------------------------------------------------------------------ INT8 tier in host DRAM
    def to_host_i8(self):
        """Move the INT8 pools to pinned host memory (page-major: the
        streamed decode copies whole pages) and prepare the streamed decode
        (its reordered plan on the device and its staging buffer); afterwards
        only ``step_streamed`` decodes."""
        import torch
        dev = self.cache.device
        self.host_pools = []
        for c in range(self.res.C):
            dp = self.cache.pools[c][0]
            if dp is None:
                continue
            if self.cache.struct.head_major[c][0]:
                n_c, cap = int(self.res.cluster_size[c]), self.pool.capacity(c, 0)
                dp = dp.view(n_c, cap, -1).transpose(0, 1).contiguous().view(-1)
            hp = torch.empty(dp.numel(), dtype=torch.uint8, pin_memory=True)
            hp.copy_(dp)
            self.host_pools.append(hp)
            self.cache.struct.pool[c][0] = hp.data_ptr()
            self.cache.struct.head_major[c][0] = 0
            self.cache.pools[c][0] = None
        torch.cuda.synchronize(dev)
        work, self.chunk_off = api.tg_stream_order(self.tables)
        self.stream_work = torch.from_numpy(np.ascontiguousarray(work)).to(dev)
        nbytes = api.tg_stream_staging_bytes(self.cache, self.tables)
        self.staging = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.host_i8 = True

    def step_streamed(self, stream=None):
        api.tg_decode_streamed(self.cache, self.tables, self.q, self.out, self.workspace, self.w.Hq,
                               self.stream_work, self.chunk_off, self.staging, stream=stream)

    def host_i8_bytes(self) -> int:
        """INT8 page bytes one streamed step copies to the device."""
        t = self.tables
        n = 0
        for c in range(self.res.C):
            if t.stride[c][0]:
                n += int((t.bt[c][0] >= 0).sum()) * self.pool.page_bytes(c, 0)
        return n

    def append(self, stream=None):
        """Append the next staged row to every (r, h) (tg_append_kv)."""
        if self.appended is None or self.steps_appended >= self.gen_tokens:
            raise ValueError("no staged rows left")
        api.tg_append_kv(self.cache, self.appended[self.steps_appended], self.status, stream=stream)
        self.steps_appended += 1

    def live_lengths(self) -> np.ndarray:
        """[B][H][2] (n_i8, n_bf) as the device holds them."""
        import torch
        torch.cuda.synchronize()
        return self.cache.len.cpu().numpy().reshape(self.w.B, self.w.Hkv, 2)

    def output(self) -> np.ndarray:
        import torch
        torch.cuda.synchronize()
        return self.out.cpu().numpy()

    # ------------------------------------------------------------------ accounting
    def traffic(self) -> dict:
        """Algorithmic bytes of one step.

        ``effective``: every (r, h) pays for the rows it attends over (a row
        is 4d bytes bf16, 2d bytes INT8 or d bytes INT4, plus 4d bytes of
        scales per quantised block), plus q, o and the tables it reads.  ``roofline``: the same, but
        a shared page's head block counts once however many sequences read
        it.  Flops: 4 * d * G per retained row per KV-head.
        """
        w, res, t = self.w, self.res, self.tables
        d, G = w.d, w.Hq // w.Hkv
        qbytes = 4 if w.q_dtype == "f32" else 2
        n_i8 = res.n_i8.astype(np.int64)
        n_bf = res.n_bf.astype(np.int64)
        bits = getattr(w, "old_bits", 8)
        kv_eff = int((n_bf * 4 * d).sum() + (n_i8 * 2 * d * bits // 8).sum() + (n_i8 // w.quant_block * 4 * d).sum())
        # unique page blocks: (cluster, tier, page id, head slot) -> rows read
        seen = {}
        for r in range(w.B):
            for h in range(w.Hkv):
                c = int(res.cluster_of_head[h])
                s = int(res.slot_in_cluster[h])
                for tier, n, S in ((0, int(n_i8[r, h]), w.quant_block), (1, int(n_bf[r, h]), w.page_size)):
                    npg = -(-n // S)
                    ids = t.bt[c][tier][r, :npg]
                    for j, pid in enumerate(ids):
                        rows = min(S, n - j * S)
                        key = (c, tier, int(pid), s)
                        if seen.get(key, 0) < rows:
                            seen[key] = rows
        kv_roof = 0
        for (c, tier, pid, s), rows in seen.items():
            kv_roof += rows * 4 * d if tier == 1 else rows * 2 * d * bits // 8 + 4 * d
        q_o = w.B * w.Hq * d * (qbytes + 4)
        tables = t.n_items * 24 + t.n_gitems * 128 + (w.B * w.Hkv + 1) * 4 + sum(
            int(-(-n_bf[r, h] // w.page_size) + n_i8[r, h] // w.quant_block) * 4
            for r in range(w.B) for h in range(w.Hkv))
        rows_total = int(n_bf.sum() + n_i8.sum())
        return {"kv_effective": kv_eff, "kv_roofline": kv_roof, "q_o": q_o, "tables": tables,
                "effective": kv_eff + q_o + tables, "roofline": kv_roof + q_o + tables,
                "head_rows": rows_total, "flops": 4 * d * G * rows_total,
                "n_items": t.n_items, "n_gitems": t.n_gitems, "n_slots": t.n_slots}


def allocated_bytes(w, n_clusters: int, chunk_bf: int = 1024, chunk_i8: int = 1024) -> int:
    """Device bytes of the page pools a batch needs from empty pools when its
    KV-heads are cut into ``n_clusters`` clusters (host computation only)."""
    res = api.tg_reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, n_clusters, w.recent_ppm,
                         w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    need = api.tg_size_tables(res, w.page_size, w.quant_block, share_of(w), chunk_bf, chunk_i8)["pages_needed"]
    pool = api.Pool(res.cluster_size, w.d, w.page_size, w.quant_block, [0] * res.C, [0] * res.C,
                    getattr(w, "old_bits", 8))
    return sum(need[c][t] * pool.page_bytes(c, t) for c in range(res.C) for t in range(2))
