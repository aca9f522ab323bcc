"""Seeded synthetic inputs for ragged-paged decode attention.

Every random number the workloads use is drawn here, from numpy PCG64 streams
keyed by ``SeedSequence([20260601, cfg_id, purpose, *ids])``.  Each stream is
independent, so one (request, KV-head) can be regenerated alone, and a stream
is prefix-stable: its first ``n`` rows do not depend on how many rows are
drawn.

What is drawn, per workload:

* admission inputs: context lengths, the head-importance ranking, optional
  per-(request, KV-head) budget overrides, radix-tree branch choices;
* the query vectors ``q[B][Hq][d]`` (fp32, or bf16 bit patterns);
* the K/V rows of each logical sequence, as bf16 bit patterns (uint16),
  drawn N(0, 1) in fp32 and rounded to nearest-even.

The module knows nothing of budgets, clusters, tiers, pages or quantisation:
callers pass in how many rows a sequence holds.

Workload shapes follow the five synthetic stand-ins for the pages' workloads:
Tangram's multi-turn histories (per-head budgets, clustered page tables), the
TTKV 128K-context tiered cache, and RadixAttention's shared system prompt plus
document branches.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

SEED_ROOT = 20260601

# purposes of the independent random streams
P_CTX, P_RANK, P_BUDGET, P_BRANCH, P_OUTLIER, P_Q, P_K, P_V, P_NODE_K, P_NODE_V = range(1, 11)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, *key])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite (normal draws); NaN handling is not needed here.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    b >>= np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------
# workload specifications
# --------------------------------------------------------------------------

SPECS: Dict[str, dict] = {
    # 1 layer, 2 requests, 4 q-heads / 2 KV-heads, d 64, context 256; one
    # budget per (request, KV-head) drawn from {32, 48, ..., 256}.
    "tiny": dict(cfg_id=1, B=2, Hq=4, Hkv=2, d=64, ctx=("fixed", 256),
                 ratio_ppm=(1_000_000, 1_000_000), budget=("override", 32, 256, 16),
                 n_clusters=2, page_size=16, quant_block=64, q_dtype="f32",
                 recent_ppm=1_000_000, rank="identity", outlier=None, share=None),
    # Llama-3-8B-shaped single layer: 32/8 heads, d 128, batch 64, context
    # uniform in [4096, 16384], retention ratio 0.50 -> 0.10 by head rank.
    "llama8b": dict(cfg_id=2, B=64, Hq=32, Hkv=8, d=128, ctx=("uniform", 4096, 16384),
                    ratio_ppm=(500_000, 100_000), budget=None, n_clusters=2,
                    page_size=16, quant_block=64, q_dtype="bf16", recent_ppm=1_000_000,
                    rank="seeded", outlier=None, share=None),
    # High raggedness: batch 256, context log-uniform in [2048, 32768], ratio
    # 0.60 -> 0.05, 8 clusters, K with 1% outlier channels scaled 8x.
    "ragged": dict(cfg_id=3, B=256, Hq=32, Hkv=8, d=128, ctx=("loguniform", 2048, 32768),
                   ratio_ppm=(600_000, 50_000), budget=None, n_clusters=8,
                   page_size=16, quant_block=64, q_dtype="bf16", recent_ppm=1_000_000,
                   rank="seeded", outlier=(0.01, 8.0), share=None),
    # Tiered long context: batch 4, context 131072, newest 12.5% bf16, the rest
    # INT8 in 64-token blocks.
    "tiered": dict(cfg_id=4, B=4, Hq=32, Hkv=8, d=128, ctx=("fixed", 131072),
                   ratio_ppm=(1_000_000, 1_000_000), budget=None, n_clusters=1,
                   page_size=16, quant_block=64, q_dtype="bf16", recent_ppm=125_000,
                   rank="seeded", outlier=None, share=None),
    # The tiered workload with a 4-bit slow tier (same seed, same rows).
    "tiered4": dict(cfg_id=4, B=4, Hq=32, Hkv=8, d=128, ctx=("fixed", 131072),
                    ratio_ppm=(1_000_000, 1_000_000), budget=None, n_clusters=1,
                    page_size=16, quant_block=64, q_dtype="bf16", recent_ppm=125_000,
                    rank="seeded", outlier=None, share=None, old_bits=4),
    # Prefix-shared radix layout: 256 requests share a 2000-token prefix, then
    # one of 4 shared 500-token branches, then a unique 80..1000-token suffix;
    # budgets (ratio 0.60 -> 0.20) apply to the suffix only.
    "radix": dict(cfg_id=5, B=256, Hq=32, Hkv=8, d=128, ctx=None,
                  ratio_ppm=(600_000, 200_000), budget=None, n_clusters=2,
                  page_size=16, quant_block=64, q_dtype="bf16", recent_ppm=1_000_000,
                  rank="seeded", outlier=None,
                  share=dict(prefix=2000, branch=500, n_branches=4, suffix=(80, 1000))),
}

WORKLOAD_NAMES = tuple(SPECS)


@dataclasses.dataclass
class Workload:
    """One seeded synthetic workload (one decode step of one layer)."""

    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    quant_block: int
    n_clusters: int
    q_dtype: str
    ratio_hi_ppm: int
    ratio_lo_ppm: int
    recent_ppm: int
    head_rank: np.ndarray            # int32 [Hkv] permutation, 0 = most important
    n_comp: np.ndarray               # int32 [B] compressible tokens per request
    n_fixed: np.ndarray              # int32 [B] always-kept shared-path tokens
    budget_override: Optional[np.ndarray]  # int32 [B*Hkv] or None
    node_len: Optional[np.ndarray]   # int32 [n_nodes] radix node lengths
    paths: Optional[List[List[int]]]  # per request: node ids, root first
    outlier_channels: Optional[np.ndarray]  # int32 [Hkv, n_out] or None
    outlier_scale: float
    spec: dict
    old_bits: int = 8                # code width of the slow (quantised) tier: 8 or 4

    # ------------------------------------------------------------------ Q
    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def q(self) -> np.ndarray:
        """Query vectors [B][Hq][d]: fp32 values, or bf16 bit patterns."""
        x = _rng(self.cfg_id, P_Q).standard_normal((self.B, self.Hq, self.d), dtype=np.float32)
        return x if self.q_dtype == "f32" else bf16_round(x)

    def q_f32(self) -> np.ndarray:
        q = self.q()
        return q if self.q_dtype == "f32" else bf16_bits_to_f32(q)

    # ------------------------------------------------------------------ K/V
    def _stream(self, key: Tuple, n: int, kind: str) -> np.ndarray:
        tag, a, h = key
        if tag == "seq":
            purpose = P_K if kind == "K" else P_V
        else:
            purpose = P_NODE_K if kind == "K" else P_NODE_V
        x = _rng(self.cfg_id, purpose, a, h).standard_normal((n, self.d), dtype=np.float32)
        if kind == "K" and self.outlier_channels is not None:
            x[:, self.outlier_channels[h]] *= np.float32(self.outlier_scale)
        return bf16_round(x)

    def stream_rows(self, key: Tuple, n: int) -> Tuple[np.ndarray, np.ndarray]:
        """First ``n`` K and V rows (bf16 bits, [n][d]) of stream ``key``.

        ``key`` is ``("seq", r, h)`` for the rows private to (r, h), or
        ``("node", k, h)`` for radix node ``k`` as seen by KV-head ``h``.
        """
        return self._stream(key, n, "K"), self._stream(key, n, "V")

    def segments(self, r: int, h: int, L: int) -> List[Tuple[Tuple, int]]:
        """The logical sequence of (r, h) with ``L`` rows, oldest first, as
        (stream key, row count) pieces: the shared radix path first (if any),
        then the rows private to (r, h)."""
        segs: List[Tuple[Tuple, int]] = []
        used = 0
        if self.paths is not None:
            for nid in self.paths[r]:
                n = int(self.node_len[nid])
                segs.append((("node", nid, h), n))
                used += n
            if L < used:
                raise ValueError("sequence shorter than its shared path")
        if L - used > 0:
            segs.append((("seq", r, h), L - used))
        return segs

    def logical_kv(self, r: int, h: int, L: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V rows (bf16 bits, [L][d]) of (r, h) in logical order."""
        ks, vs = [], []
        for key, n in self.segments(r, h, L):
            k, v = self.stream_rows(key, n)
            ks.append(k)
            vs.append(v)
        return np.concatenate(ks), np.concatenate(vs)

    def source_buffer(self, L: np.ndarray, threads: Optional[int] = None):
        """Deduplicated row store plus a per-token gather index.

        ``L`` is int [B][Hkv], the row count of each logical sequence.

        Returns ``(rows, index, offsets)``: ``rows`` is uint16
        [n_rows][2][d] (K row then V row, bf16 bits); the logical row ``i`` of
        (r, h) is ``rows[index[offsets[r*Hkv+h] + i]]``; ``offsets`` is int64
        [B*Hkv + 1].  Each stream is stored once, however many sequences use
        it.
        """
        L = np.asarray(L, dtype=np.int64).reshape(self.B, self.Hkv)
        need: Dict[Tuple, int] = {}
        segs = {}
        for r in range(self.B):
            for h in range(self.Hkv):
                s = self.segments(r, h, int(L[r, h]))
                segs[(r, h)] = s
                for key, n in s:
                    need[key] = max(need.get(key, 0), n)
        keys = list(need)
        start = {}
        tot = 0
        for key in keys:
            start[key] = tot
            tot += need[key]
        rows = np.empty((tot, 2, self.d), dtype=np.uint16)

        def fill(key):
            k, v = self.stream_rows(key, need[key])
            s = start[key]
            rows[s:s + need[key], 0, :] = k
            rows[s:s + need[key], 1, :] = v

        with _cf.ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(fill, keys))

        offsets = np.zeros(self.B * self.Hkv + 1, dtype=np.int64)
        offsets[1:] = np.cumsum(L.reshape(-1))
        index = np.empty(int(offsets[-1]), dtype=np.int32)
        if tot > np.iinfo(np.int32).max:
            raise OverflowError("row store too large for int32 row indices")
        for r in range(self.B):
            for h in range(self.Hkv):
                o = int(offsets[r * self.Hkv + h])
                for key, n in segs[(r, h)]:
                    index[o:o + n] = np.arange(start[key], start[key] + n, dtype=np.int32)
                    o += n
        return rows, index, offsets


def make_workload(name: str, **overrides) -> Workload:
    """Build workload ``name`` (one of ``WORKLOAD_NAMES``).

    Keyword overrides replace entries of the spec (e.g. ``B=4`` or
    ``ctx=("uniform", 300, 900)``) to make smaller seeded variants for tests.
    """
    spec = dict(SPECS[name])
    spec.setdefault("old_bits", 8)
    unknown = set(overrides) - set(spec)
    if unknown:
        raise KeyError(f"unknown workload fields: {sorted(unknown)}")
    spec.update(overrides)
    cid = spec["cfg_id"]
    B, Hq, Hkv, d = spec["B"], spec["Hq"], spec["Hkv"], spec["d"]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")

    if spec["rank"] == "identity":
        rank = np.arange(Hkv, dtype=np.int32)
    else:
        rank = _rng(cid, P_RANK).permutation(Hkv).astype(np.int32)

    node_len = paths = None
    share = spec["share"]
    if share is None:
        kind = spec["ctx"][0]
        g = _rng(cid, P_CTX)
        if kind == "fixed":
            ctx = np.full(B, spec["ctx"][1], dtype=np.int64)
        elif kind == "uniform":
            ctx = g.integers(spec["ctx"][1], spec["ctx"][2], size=B, endpoint=True)
        elif kind == "loguniform":
            lo, hi = spec["ctx"][1], spec["ctx"][2]
            u = g.uniform(math.log(lo), math.log(hi), size=B)
            ctx = np.clip(np.floor(np.exp(u)), lo, hi)
        else:
            raise ValueError(kind)
        n_comp = ctx.astype(np.int32)
        n_fixed = np.zeros(B, dtype=np.int32)
    else:
        nb = share["n_branches"]
        node_len = np.array([share["prefix"]] + [share["branch"]] * nb, dtype=np.int32)
        branch = _rng(cid, P_BRANCH).integers(0, nb, size=B)
        paths = [[0, 1 + int(b)] for b in branch]
        n_fixed = np.full(B, share["prefix"] + share["branch"], dtype=np.int32)
        lo, hi = share["suffix"]
        n_comp = _rng(cid, P_CTX).integers(lo, hi, size=B, endpoint=True).astype(np.int32)

    override = None
    if spec["budget"] is not None:
        _, lo, hi, step = spec["budget"]
        k = _rng(cid, P_BUDGET).integers(0, (hi - lo) // step, size=B * Hkv, endpoint=True)
        override = (lo + step * k).astype(np.int32)

    outl = None
    oscale = 1.0
    if spec["outlier"] is not None:
        frac, oscale = spec["outlier"]
        n_out = max(1, int(round(frac * d)))
        g = _rng(cid, P_OUTLIER)
        outl = np.stack([g.choice(d, size=n_out, replace=False) for _ in range(Hkv)]).astype(np.int32)

    hi_ppm, lo_ppm = spec["ratio_ppm"]
    return Workload(
        name=name, cfg_id=cid, B=B, Hq=Hq, Hkv=Hkv, d=d,
        page_size=spec["page_size"], quant_block=spec["quant_block"],
        n_clusters=spec["n_clusters"], q_dtype=spec["q_dtype"],
        ratio_hi_ppm=int(hi_ppm), ratio_lo_ppm=int(lo_ppm), recent_ppm=int(spec["recent_ppm"]),
        head_rank=rank, n_comp=n_comp, n_fixed=n_fixed, budget_override=override,
        node_len=node_len, paths=paths, outlier_channels=outl, outlier_scale=float(oscale),
        spec=spec, old_bits=int(spec["old_bits"]),
    )


def share_arrays(w: Workload):
    """Radix paths as flat int32 arrays: (n_nodes[B], node_ids[sum], node_len[n])."""
    if w.paths is None:
        return None
    n_nodes = np.array([len(p) for p in w.paths], dtype=np.int32)
    ids = np.array([n for p in w.paths for n in p], dtype=np.int32)
    return n_nodes, ids, np.asarray(w.node_len, dtype=np.int32)
