#!/usr/bin/env python3
"""Benchmark: effective KV GB/s of one ragged-paged decode step on one GPU.

    python bench.py [--steps K] [--warmup W] [--config ragged] [--configs tiny,llama8b,...]

One step = the whole decode hot path over one batch: the split-K kernel over
every plan item (bf16 pages and INT8 blocks) and the log-sum-exp merge, on a
cache that is already resident in HBM.  The headline line is the largest
workload that fits one GPU (``ragged``: batch 256, context 2K-32K); every
other workload is measured the same way after it and listed under
``configs``, each with its split kernel's roofline and an oracle check of
every output it computed.  Before every timed step a 1 GiB
device read evicts L2 and the 256 MB last-level cache with clean lines
(outside the timed events; ``--flush write`` uses a 1 GiB write instead, whose
dirty lines then drain to HBM during the timed kernels).  Each step is
bracketed by HIP events on the stream the kernels run on; the K steps together
are bracketed by device synchronisation.

Prints one JSON line (see the ``result`` dict at the end).  ``--gpus`` above 1
is refused: the measurement runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
# device pool layouts (include/tg.h), as (INT8 pools, bf16 pools) head-major
# flags; "auto" is the runner's measured choice (bf16 pools head-major when
# the cache has no quantised tier, all else page-major)
LAYOUTS = {"auto": None, "page-major": (False, False), "head-major": (True, True),
           "bf16-head-major": (False, True)}
METRIC = "effective KV GB/s (and % of HBM peak) in ragged-paged decode attention"
DESCRIPTIONS = {
    "tiny": "tiny: 2 requests, 4/2 heads, d 64, ctx 256, budgets in {32..256}, 2 clusters",
    "llama8b": "Llama-3-8B-shaped layer: batch 64, 32/8 heads, d 128, ctx U[4096,16384], ratio 0.50->0.10 by head rank, 2 clusters, page 16, bf16",
    "ragged": "high raggedness: batch 256, 32/8 heads, d 128, ctx log-U[2048,32768], ratio 0.60->0.05, 8 clusters, 1% K outlier channels x8",
    "tiered": "TTKV tiered: batch 4, ctx 131072, 32/8 heads, d 128, newest 12.5% bf16, rest INT8 64-token blocks",
    "tiered4": "TTKV tiered, 4-bit slow tier: batch 4, ctx 131072, 32/8 heads, d 128, newest 12.5% bf16, rest INT4 64-token blocks",
    "radix": "prefix-shared radix: batch 256, 2000-token prefix + 1 of 4 500-token branches + 80..1000 suffix, ratio 0.60->0.20 on suffix",
}
# HBM bytes per split stage from rocprofv3 counter runs, one file per workload
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_kernel_{config}_traffic.txt")
# sources of the split kernels (the dominant kernels of every workload)
KERNEL_SRCS = [os.path.join(ROOT, "non_uniform_paged_amd", "csrc", f)
               for f in ("tg_split.hip", "tg_item_bf16.h", "tg_item_i8.h", "tg_device.h")]


def _kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_record(config: str):
    """HBM bytes per split launch from the committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    path = TRAFFIC_FILE.format(config=config)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != _kernel_hash() or rec.get("workload") != config:
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def codec_bench(prep, args, stream):
    """The lossless bf16 exponent codec over the whole bf16 page pool of the
    cache (the KV pages as they sit in HBM): compressed size, encode and
    decode rates (input and output bytes of bf16 per second), and a
    bit-exact check of the round trip."""
    import numpy as np
    import torch

    from non_uniform_paged_amd import api

    pools = [p[1] for p in prep.cache.pools if p[1] is not None]
    src = pools[0].view(torch.int16) if len(pools) == 1 else torch.cat([p.view(torch.int16) for p in pools])
    n = src.numel() - src.numel() % 8
    src = src[:n]
    dst = torch.empty(api.tg_zip_bound(n), dtype=torch.uint8, device="cuda")
    ws = torch.empty(api.tg_zip_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(src)
    api.tg_zip_encode(src, dst, ws, stream=stream)
    api.tg_zip_decode(dst, n, out, stream=stream)
    torch.cuda.synchronize()
    exact = bool(torch.equal(out, src))
    size = api.zip_compressed_bytes(dst)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    enc, dec = [], []
    for _ in range(args.zip_reps):
        ev[0].record(stream)
        api.tg_zip_encode(src, dst, ws, stream=stream)
        ev[1].record(stream)
        api.tg_zip_decode(dst, n, out, stream=stream)
        ev[2].record(stream)
        torch.cuda.synchronize()
        enc.append(ev[0].elapsed_time(ev[1]))
        dec.append(ev[1].elapsed_time(ev[2]))
    e_ms, d_ms = float(np.median(enc)), float(np.median(dec))
    n_esc = (size - 256 - n - n // 2) // 5
    res = {"values": n, "bf16_bytes": 2 * n, "compressed_bytes": size, "ratio": round(2 * n / size, 4),
           "escapes": n_esc, "encode_ms": round(e_ms, 4), "decode_ms": round(d_ms, 4),
           "encode_GBps": round(2 * n / (e_ms * 1e-3) / 1e9, 1), "decode_GBps": round(2 * n / (d_ms * 1e-3) / 1e9, 1),
           "round_trip_bit_exact": exact,
           "pages_quote_GBps": {"encode": 613, "decode": 2181, "hardware": "not stated"}}
    del dst, ws, out
    torch.cuda.empty_cache()
    return res


def append_bench(w, args, evict, stream):
    """Decode steps that each append one row per (r, h) first (tg_append_kv,
    with the ageing of the oldest bf16 block into INT8 where the tier split
    moves), on a cache built with room for them; the append and the decode
    are timed separately with HIP events."""
    import numpy as np
    import torch

    from non_uniform_paged_amd.runner import Prepared

    K = args.append_steps
    gp = Prepared(w, chunk_bf=args.chunk_bf, chunk_i8=args.chunk_i8, gen_tokens=K,
                  head_major=LAYOUTS[args.layout])
    lens0 = gp.live_lengths().copy()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for k in range(K):
        evict(k)
        ev[k][0].record(stream)
        gp.append(stream=stream)
        ev[k][1].record(stream)
        gp.step(stream=stream)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    app_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    lens = gp.live_lengths()
    L0 = lens0.sum(-1)
    # the tier split of the grown lengths (INT8: whole blocks of the rows older
    # than the recent share)
    Lk = L0 + K
    n_i8 = (Lk - (Lk * w.recent_ppm + 999_999) // 1_000_000) // w.quant_block * w.quant_block
    expect = np.stack([n_i8, Lk - n_i8], -1)
    d = w.d
    aged = int((lens[..., 0] - lens0[..., 0]).sum()) // w.quant_block
    # algorithmic bytes: each new row written (K and V, bf16), and per aged
    # block its bf16 rows read and its codes and scales written
    nbytes = K * w.B * w.Hkv * 4 * d + aged * (w.quant_block * 4 * d + w.quant_block * 2 * d + 4 * d)
    out = {"steps": K, "append_us_mean": round(float(app_ms.mean()) * 1e3, 2),
           "append_us_median": round(float(np.median(app_ms)) * 1e3, 2),
           "decode_us_mean_after_append": round(float(dec_ms.mean()) * 1e3, 2),
           "aged_blocks": aged, "append_bytes": nbytes,
           "append_GBps": round(nbytes / (app_ms.sum() * 1e-3) / 1e9, 2),
           "lengths_match_tier_split": bool(np.array_equal(lens, expect)),
           "capacity_flag": int(gp.status.item())}
    del gp
    torch.cuda.empty_cache()
    return out


def _layout_name(prep) -> str:
    """Layout of the prepared cache's pools, by tier."""
    hm = prep.cache.head_major
    return {(False, False): "page-major", (True, True): "head-major",
            (False, True): "bf16-head-major", (True, False): "int8-head-major"}[hm]


def host_tier_bench(prep, args, stream, resident_ms):
    """The same decode step with the INT8 pages in pinned host memory,
    streamed per request through two HBM staging slots (tg_decode_streamed):
    step time, INT8 bytes crossing to the device per step, their rate, the
    plain host-to-device copy rate of the same bytes, the step's rate as a
    fraction of it, and the time the step spends beyond the copies alone
    (the compute the pipeline does not hide)."""
    import numpy as np
    import torch

    resident_out = prep.output().copy()
    prep.to_host_i8()
    nbytes = prep.host_i8_bytes()
    # plain copy rate: every host pool to a device buffer once, pinned source
    dst = torch.empty(max(hp.numel() for hp in prep.host_pools), dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for hp in prep.host_pools:
        dst[:hp.numel()].copy_(hp, non_blocking=True)
    e0.record(stream)
    for hp in prep.host_pools:
        dst[:hp.numel()].copy_(hp, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    pool_bytes = sum(hp.numel() for hp in prep.host_pools)
    copy_gbps = pool_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    prep.step_streamed(stream=stream)
    torch.cuda.synchronize()
    identical = bool(np.array_equal(prep.output(), resident_out))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.host_steps)]
    for k in range(args.host_steps):
        ev[k][0].record(stream)
        prep.step_streamed(stream=stream)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    step_ms = float(np.median(ms))
    copy_ms = nbytes / (copy_gbps * 1e9) * 1e3
    return {"steps": args.host_steps, "step_ms_median": round(step_ms, 4),
            "int8_bytes_to_device_per_step": nbytes,
            "int8_GBps": round(nbytes / (step_ms * 1e-3) / 1e9, 2),
            "plain_h2d_copy_GBps": round(copy_gbps, 2),
            "copy_only_ms": round(copy_ms, 4), "resident_step_ms": round(resident_ms, 4),
            "fraction_of_copy_rate": round(copy_ms / step_ms, 4),
            "exposed_ms_beyond_copy": round(step_ms - copy_ms, 4),
            "bit_identical_to_resident": identical}


def stream_read_bench(w, prep, evict, stream, reps: int = 5) -> dict:
    """Time tg_bench_streams over the chunk counts of the plan: the rate the
    split kernels' access pattern (independent per-item page streams, two
    pages in flight) allows on this device, with no arithmetic."""
    import numpy as np
    import torch

    from non_uniform_paged_amd import api
    plan = prep.tables.plan
    t0, t1 = plan[:, 3].astype(np.int64), plan[:, 4].astype(np.int64)
    page = 4 * w.page_size * w.d                              # K and V of one head's bf16 page
    block = 2 * w.quant_block * w.d * getattr(w, "old_bits", 8) // 8 + 4 * w.d  # one INT8 block
    bf = plan[:, 2] == api.TG_TIER_BF16
    nbytes = np.where(bf, (-(-t1 // w.page_size) - t0 // w.page_size) * page,
                      (-(-t1 // w.quant_block) - t0 // w.quant_block) * block)
    n_chunks = -(-nbytes // 8192)
    total = int(n_chunks.sum())
    off = np.zeros(len(n_chunks) + 1, np.int32)
    off[1:] = np.cumsum(n_chunks)
    ids = np.random.default_rng(0).permutation(total).astype(np.int32)
    buf = torch.ones(total * 8192, dtype=torch.uint8, device="cuda")
    d_ids, d_off = torch.from_numpy(ids).cuda(), torch.from_numpy(off).cuda()
    sink = torch.empty(len(n_chunks), dtype=torch.int32, device="cuda")
    api.tg_bench_streams(buf, d_ids, d_off, sink, stream=stream)
    ts = []
    for i in range(reps):
        evict(i)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        api.tg_bench_streams(buf, d_ids, d_off, sink, stream=stream, events=ev)  # kernel start / end
        ts.append(ev)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
    del buf
    return {"streams": int(len(n_chunks)), "bytes": total * 8192, "ms": round(ms, 5),
            "GBps": round(total * 8192 / (ms * 1e-3) / 1e9, 1)}


def _device_record(torch) -> dict:
    """What the runtime reports about the GPU (to check the published
    figures the roofline uses: compute units, memory, caches)."""
    p = torch.cuda.get_device_properties(0)
    out = {}
    for k in ("name", "gcnArchName", "multi_processor_count", "total_memory", "L2_cache_size",
              "max_threads_per_multi_processor", "warp_size", "clock_rate", "memory_clock_rate",
              "memory_bus_width"):
        v = getattr(p, k, None)
        if v is not None:
            out[k] = v if isinstance(v, (int, float, str)) else str(v)
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def cpu_baseline(w, prep, min_s: float = 10.0, keep_bytes: float = 2e9):
    """The oracle, untuned, on this host's cores, in two parts.

    Check: every (r, h) pair of the step is decoded by the fp64 oracle from
    its raw rows and compared with the GPU output element by element, pass
    iff |g - r| <= 2e-3 + 1e-2 |r| everywhere (max-abs, and max-rel over
    |r| >= 1e-3, reported).  Timing: a bounded sample of the pairs (rows
    generated first and not timed, up to keep_bytes of them) is decoded again
    until min_s of wall time; GB/s over the rows decoded.  One pair per task
    on a pool of N threads (N = the cores this process may use, at most 16;
    numpy releases the interpreter lock in its kernels) with BLAS pinned to
    one thread each."""
    import concurrent.futures as cf

    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    from oracle import attention as A

    res = A.reserve_for(w)
    q = A.q_f64(w)
    G = w.Hq // w.Hkv
    scale = 1.0 / math.sqrt(w.d)
    n_threads = _threads()
    gpu_out = prep.output()
    bits = getattr(w, "old_bits", 8)

    def nbytes_of(r, h):
        n8, nb = res.n_i8[r][h], res.n_bf[r][h]
        return nb * 4 * w.d + n8 * 2 * w.d * bits // 8 + (n8 // w.quant_block) * 4 * w.d

    def check(rh):
        r, h = rh
        K16, V16 = w.logical_kv(r, h, res.L[r][h])
        ref = A.decode_rows(q[r, h * G:(h + 1) * G], K16, V16, res.n_i8[r][h], w.quant_block, scale, bits)
        got = gpu_out[r, h * G:(h + 1) * G]
        err = np.abs(got - ref)
        big = np.abs(ref) >= 1e-3
        rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
        ok = bool(np.all(err <= 2e-3 + 1e-2 * np.abs(ref)))
        return ok, float(err.max()), rel

    order = np.random.default_rng(7).permutation(w.B * w.Hkv)
    sample, total = [], 0
    for i in order:
        r, h = divmod(int(i), w.Hkv)
        size = int(res.L[r][h]) * 4 * w.d
        if sample and total + size > keep_bytes:
            break
        sample.append((r, h))
        total += size

    def gen(rh):
        r, h = rh
        K16, V16 = w.logical_kv(r, h, res.L[r][h])
        return r, h, K16, V16, nbytes_of(r, h)

    def run(task):
        r, h, K16, V16, _ = task
        return A.decode_rows(q[r, h * G:(h + 1) * G], K16, V16, res.n_i8[r][h], w.quant_block, scale, bits)

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        with cf.ThreadPoolExecutor(max_workers=n_threads) as ex:
            t0 = time.perf_counter()
            checks = list(ex.map(check, [(r, h) for r in range(w.B) for h in range(w.Hkv)]))
            check_s = time.perf_counter() - t0
            tasks = list(ex.map(gen, sample))
            wall, passes = 0.0, 0
            while passes == 0 or wall < min_s:
                t0 = time.perf_counter()
                list(ex.map(run, tasks))
                wall += time.perf_counter() - t0
                passes += 1
    finally:
        if ctx is not None and hasattr(ctx, "unregister"):
            ctx.unregister()
    nbytes = passes * sum(t[4] for t in tasks)
    return {"value": round(nbytes / wall / 1e9, 4), "unit": "GB/s", "cores": n_threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"timing: {passes} pass(es) over {len(tasks)} of the {w.B * w.Hkv} (request, KV-head) pairs "
                      f"of the step, fp64 numpy, {n_threads} threads with one BLAS thread each, {wall:.1f} s wall",
            "check": {"pairs": len(checks), "of_pairs": w.B * w.Hkv,
                      "criterion": "|gpu - oracle| <= 2e-3 + 1e-2 |oracle| for every output element",
                      "pass": all(c[0] for c in checks), "max_abs": max(c[1] for c in checks),
                      "max_rel": max(c[2] for c in checks), "wall_s": round(check_s, 2)}}


def measure(name, args, evict, stream, read_gbps=None, headline=False):
    """Time one workload's decode step (split kernel(s) + merge) and return
    its record: step times, the split kernel timed alone, its roofline on the
    algorithmic bytes, the page-stream read of its plan, and the oracle check
    and baseline.  Extra measurements of the path's other parts (append,
    codec, host-DRAM tier) go into the records that exercise them."""
    import numpy as np
    import torch

    from non_uniform_paged_amd import api
    from non_uniform_paged_amd.runner import PLAN_CHUNKS, Prepared, allocated_bytes, tune_candidates
    from workloads import make_workload

    w = make_workload(name)
    chunk_bf = args.chunk_bf if (headline and args.chunk_bf) else PLAN_CHUNKS[name][0]
    chunk_i8 = args.chunk_i8 if (headline and args.chunk_i8) else PLAN_CHUNKS[name][1]
    t_prep = time.perf_counter()
    prep = Prepared(w, chunk_bf=chunk_bf, chunk_i8=chunk_i8, group_size=args.group_size if headline else None,
                    head_major=LAYOUTS[args.layout])
    t_prep = time.perf_counter() - t_prep
    G = w.Hq // w.Hkv
    tuned = None
    if headline and args.tune:  # outside the timed region: pick the plan item lengths on the device
        cands = tune_candidates(w, prep.tables.stride_has_i8)
        tuned = sorted(prep.tune_chunks(cands, evict=lambda: evict(0), stream=stream), key=lambda x: x[2])
        chunk_bf, chunk_i8 = prep.chunks
    tr = prep.traffic()

    def one_step(evs=None):
        # the decode step: tg_decode_attn (split kernel(s), then the merge)
        if evs is not None:
            evs[0].record(stream)
        api.tg_decode_attn(prep.cache, prep.q, prep.out, prep.workspace, w.Hq, stream=stream)
        if evs is not None:
            evs[1].record(stream)

    def split_step(evs):
        # the same step issued as its two halves, the split kernel's own start
        # and end recorded into evs[0] and evs[1] (no dispatch latency of a
        # separately recorded event in its time); the tests check that the
        # two forms give bit-identical outputs
        api.tg_decode_split_timed(prep.cache, prep.q, prep.workspace, w.Hq, evs[:2], stream=stream)
        api.tg_merge_partials(prep.workspace, prep.tables.n_slots, w.B * w.Hkv, G, w.d,
                              prep.cache.part_off, prep.out, stream=stream)
        evs[2].record(stream)

    for i in range(args.warmup):
        evict(i)
        one_step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        evict(i + 1)
        one_step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    ms = float(step_ms.mean())
    med = float(np.median(step_ms))
    # kernel timing: as many steps again, split and merge timed separately
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        evict(i + 1)
        split_step(kev[i])
    torch.cuda.synchronize()
    split_ms_all = np.array([e[0].elapsed_time(e[1]) for e in kev])
    merge_ms_all = np.array([e[1].elapsed_time(e[2]) for e in kev])

    # algorithmic bytes of the split kernel(s), the dominant kernels: retained
    # rows (each page block once), q and the tables they read.  The partials
    # they write for the merge are overhead of the split, not algorithmic
    # bytes, and are listed apart.
    q_bytes = w.B * w.Hq * w.d * (4 if w.q_dtype == "f32" else 2)
    split_bytes = tr["kv_roofline"] + q_bytes + tr["tables"]
    partial_bytes = prep.tables.n_slots * G * (w.d + 2) * 4
    split_ms = float(split_ms_all.mean())
    achieved = split_bytes / (split_ms * 1e-3) / 1e9
    streams = stream_read_bench(w, prep, evict, stream)
    traffic = _traffic_record(name)
    rec = {
        "name": name,
        "workload": DESCRIPTIONS[name],
        "config": {"batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d, "clusters": w.n_clusters,
                   "page": w.page_size, "pool_layout": _layout_name(prep), "chunk_bf": chunk_bf,
                   "chunk_i8": chunk_i8,
                   "plan_items": prep.tables.n_items, "group_items": prep.tables.n_gitems,
                   "group_size": prep.group_size, "slots": prep.tables.n_slots,
                   "retained_head_rows": tr["head_rows"],
                   "chunks_tuned": None if tuned is None else [[a, b, round(c, 1)] for a, b, c in tuned[:5]]},
        "effective_bytes": tr["effective"],
        "roofline_bytes": tr["roofline"],
        "effective_GBps": round(tr["effective"] / (ms * 1e-3) / 1e9, 2),
        "step_ms_mean": round(ms, 5),
        "step_ms_median": round(med, 5),
        "p10_ms": round(float(np.percentile(step_ms, 10)), 5),
        "p90_ms": round(float(np.percentile(step_ms, 90)), 5),
        "steps_per_s": round(1e3 / med, 2),
        "step_frac_roofline_bytes": round(tr["roofline"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "split_ms": round(split_ms, 5),
        "merge_ms": round(float(merge_ms_all.mean()), 5),
        "partials_bytes_written": partial_bytes,
        "wall_s_timed_region": round(wall, 4),
        "prepare_s": round(t_prep, 2),
        "stream_read": dict(streams, split_time_frac=round(streams["ms"] / split_ms, 4)),
        "roofline": {
            "kernel": "split_bf16_kernel" if not prep.tables.stride_has_i8 else "split_tiered_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": split_bytes,
        },
    }
    if read_gbps:
        rec["split_frac_of_read_ceiling"] = round(achieved / read_gbps, 4)
    if headline:
        # pool bytes the batch needs at the configured cluster count, one
        # cluster and one cluster per KV-head, against the bytes it retains
        alloc = {str(C): allocated_bytes(w, C, chunk_bf, chunk_i8) for C in sorted({w.n_clusters, 1, w.Hkv})}
        rec["fragmentation"] = {"retained_bytes": tr["kv_roofline"], "allocated_bytes_by_clusters": alloc,
                                "ratio_by_clusters": {k: round(v / tr["kv_roofline"], 4) for k, v in alloc.items()}}
        if args.append_steps > 0 and w.paths is None:
            args_a = argparse.Namespace(**vars(args))
            args_a.chunk_bf, args_a.chunk_i8 = chunk_bf, chunk_i8
            rec["append"] = append_bench(w, args_a, evict, stream)
        if args.zip_reps > 0:
            rec["codec"] = codec_bench(prep, args, stream)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, prep, min_s=args.cpu_seconds if headline else args.cpu_seconds_sub)
    if args.host_steps > 0 and prep.tables.stride_has_i8 and (headline or name == "tiered"):
        rec["host_tier"] = host_tier_bench(prep, args, stream, med)
    del prep
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="ragged", choices=sorted(DESCRIPTIONS),
                    help="headline workload (default: the largest single-GPU one, ragged)")
    ap.add_argument("--configs", default="tiny,llama8b,tiered,tiered4,radix",
                    help="comma-separated workloads measured after the headline, each a sub-record ('' = none)")
    ap.add_argument("--chunk-bf", type=int, default=None, help="bf16 rows per plan item (default per workload)")
    ap.add_argument("--chunk-i8", type=int, default=None, help="INT8 rows per plan item (default per workload)")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read")
    ap.add_argument("--layout", choices=sorted(LAYOUTS), default="auto",
                    help="device pool layout (include/tg.h); outputs are identical")
    ap.add_argument("--append-steps", type=int, default=128,
                    help="decode steps with tg_append_kv timed on a second cache built for growth (0: skip)")
    ap.add_argument("--host-steps", type=int, default=10,
                    help="decode steps with the INT8 tier in pinned host memory, streamed (0: skip)")
    ap.add_argument("--zip-reps", type=int, default=5,
                    help="timed encode/decode passes of the lossless codec over the bf16 pool (0: skip)")
    ap.add_argument("--group-size", type=int, default=None,
                    help="requests per shared-prefix group item (default min(32, 128 / G) when pages are shared)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle timing per headline (s)")
    ap.add_argument("--cpu-seconds-sub", type=float, default=2.0, help="oracle timing per sub-record (s)")
    ap.add_argument("--tune", action="store_true",
                    help="time candidate plan item lengths on the device first and keep the fastest")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the decode step would shard by request with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        print(json.dumps({"copy_bytes_each_way": n, "copies": 5, "ms_per_copy": round(dt * 1e3, 4),
                          "GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)
        return

    from non_uniform_paged_amd import api

    torch.cuda.set_device(0)
    t_all = time.perf_counter()
    stream = torch.cuda.current_stream()
    flush = None if args.flush == "none" else torch.ones(1 << 30, dtype=torch.uint8, device="cuda")

    def evict(i):
        if args.flush == "read":
            torch.amax(flush)
        elif args.flush == "write":
            flush.fill_(i & 0xFF)

    # achievable streaming-read rate of this device (2 GiB, non-temporal
    # loads), the practical ceiling besides the 8 TB/s peak
    rbuf = torch.ones(1 << 31, dtype=torch.uint8, device="cuda")
    sink = torch.empty(api.TG_BENCH_READ_BLOCKS, dtype=torch.int32, device="cuda")
    api.tg_bench_read(rbuf, sink, stream=stream)
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(5)]
    for k in range(5):
        api.tg_bench_read(rbuf, sink, stream=stream, events=rev[k])  # kernel start / end
    torch.cuda.synchronize()
    read_ms = float(np.median([a.elapsed_time(b) for a, b in rev]))
    read_gbps = rbuf.numel() / (read_ms * 1e-3) / 1e9
    del rbuf
    torch.cuda.empty_cache()

    head = measure(args.config, args, evict, stream, read_gbps, headline=True)
    print(f"# {args.config}: split {head['split_ms'] * 1e3:.1f} us, frac {head['roofline']['frac']}",
          file=sys.stderr, flush=True)
    subs = []
    for name in [c for c in args.configs.split(",") if c and c != args.config]:
        subs.append(measure(name, args, evict, stream, read_gbps))
        print(f"# {name}: split {subs[-1]['split_ms'] * 1e3:.1f} us, frac {subs[-1]['roofline']['frac']}",
              file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": head["effective_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q; no datasets or weights)",
        "config": dict(workload=head["workload"], name=head["name"], parallelism="single GPU", **head["config"]),
        "hbm_frac_roofline_bytes": head["step_frac_roofline_bytes"],
        "kernel_timing": "split and read kernels: HIP events recorded at each kernel's own start and end "
                         "(hipExtLaunchKernel); merge_ms: split end to an event after the merge; steps: event "
                         "pairs around each tg_decode_attn call",
        "cache_eviction_between_steps": args.flush,
        "device": _device_record(torch),
        "read_ceiling_GBps": round(read_gbps, 1),
    }
    for k, v in head.items():
        if k not in ("name", "workload", "config") and k not in result:
            result[k] = v
    result["configs"] = subs
    result["bench_wall_s"] = round(time.perf_counter() - t_all, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
