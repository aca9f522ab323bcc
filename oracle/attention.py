"""fp64 oracle for decode attention over per-head retained rows -- TEST
INFRASTRUCTURE (see ``oracle/__init__``).

What is computed (the plain definition; no blocking or reordering):

    for request r and q-head hq, with KV-head h = hq // G (contiguous GQA
    groups), K, V = the L[r][h] rows that (r, h) retains, in logical order:

        s_t = (q[r][hq] . K[t]) * scale          scale = 1/sqrt(d) by default
        o[r][hq] = sum_t softmax(s)_t * V[t]

Sources: TTKV page, "What real problem" -- each generated token attends over
all cached KV states; Tangram page, "Three mechanisms" -- budgets and ragged
paging change which memory holds each head's retained rows, not what is
computed ("no accuracy loss"); TTKV page, "Tier Layout"/"Tier Interaction" --
slow-tier rows enter as their dequantised values (``oracle.quant``).  There is
no mask, positional term or soft-cap; rotary embedding is already inside the
cached keys.

``lse_merge`` is the blockwise-softmax identity of the online normaliser
(CAP survey page, section 2.4.3 "Distributed acceleration", the online
normaliser [88]): partial results over disjoint token sets, each kept as
(m = max score, l = sum exp(s - m), acc = sum exp(s - m) v), merge exactly to
the full softmax.

Pinned by: tests/test_oracle_attention.py -- fp64 scaled-dot-product attention
from torch on dense tensors (uniform budgets), the single-row identity, closed
forms (equal keys -> mean of V; equal values; a 3:1 two-row mix), row
permutation invariance, pure-Python brute force with math.fsum on tiny
shapes, INT8 rows equal to bf16 rows of the same value, and split
invariance of ``lse_merge``.  ``bf16_to_f64`` and ``q_f64`` are pinned by
hand-checked bit patterns, by all 65536 patterns read field by field from
the bf16 format, and end to end by the dense-SDPA pin, whose rows and
queries are decoded from those fields rather than by this module.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

from . import planner, quant


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V in fp64.  q [G][d], K/V [L][d] -> [G][d]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = (K @ q.T) * scale            # [L][G]
    m = s.max(axis=0)
    p = np.exp(s - m)
    return (p.T @ V) / p.sum(axis=0)[:, None]


def partial(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """(m [G], l [G], acc [G][d]) over the given rows, fp64."""
    q = np.asarray(q, dtype=np.float64)
    s = (np.asarray(K, np.float64) @ q.T) * scale
    m = s.max(axis=0)
    p = np.exp(s - m)
    return m, p.sum(axis=0), p.T @ np.asarray(V, np.float64)


def lse_merge(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Merge partials m [S][G], l [S][G], acc [S][G][d] -> o [G][d]."""
    m = np.asarray(m, np.float64)
    M = m.max(axis=0)
    w = np.exp(m - M)
    num = (w[:, :, None] * np.asarray(acc, np.float64)).sum(axis=0)
    return num / (w * np.asarray(l, np.float64)).sum(axis=0)[:, None]


# ------------------------------------------------------------------ workloads
def reserve_for(w) -> planner.Reservation:
    """The oracle's own reservation for a workload (integer oracle)."""
    return planner.reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters,
                           w.recent_ppm, w.quant_block, w.n_comp, w.n_fixed,
                           w.budget_override)


def q_f64(w) -> np.ndarray:
    """Queries [B][Hq][d] in fp64: fp32 queries as they are, bf16 queries
    decoded exactly."""
    q = w.q()
    return np.asarray(q, np.float64) if w.q_dtype == "f32" else bf16_to_f64(q)


def rows_f64(K16: np.ndarray, V16: np.ndarray, n_i8: int, qb: int, bits: int = 8) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 K, V a sequence attends over: its bf16 rows, with the oldest
    ``n_i8`` rows replaced by their ``bits``-bit (8 or 4) dequantised values."""
    K = bf16_to_f64(K16)
    V = bf16_to_f64(V16)
    if n_i8:
        qk, sk = quant.quantize_rows(K[:n_i8].astype(np.float32), qb, bits)
        qv, sv = quant.quantize_rows(V[:n_i8].astype(np.float32), qb, bits)
        K[:n_i8] = quant.dequantize_rows(qk, sk, qb)
        V[:n_i8] = quant.dequantize_rows(qv, sv, qb)
    return K, V


def head_rows(w, res: planner.Reservation, r: int, h: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 K, V rows of (r, h) (see ``rows_f64``)."""
    K16, V16 = w.logical_kv(r, h, res.L[r][h])
    return rows_f64(K16, V16, res.n_i8[r][h], w.quant_block, getattr(w, "old_bits", 8))


def decode_rows(q_group: np.ndarray, K16: np.ndarray, V16: np.ndarray, n_i8: int, qb: int,
                scale: float, bits: int = 8) -> np.ndarray:
    """Outputs [G][d] of one GQA group from its raw rows (bf16 bits)."""
    K, V = rows_f64(K16, V16, n_i8, qb, bits)
    return attend(q_group, K, V, scale)


def decode_pair(w, res: planner.Reservation, r: int, h: int, q: Optional[np.ndarray] = None,
                scale: Optional[float] = None) -> np.ndarray:
    """Outputs [G][d] (fp64) of the G q-heads of KV-head h in request r."""
    G = w.Hq // w.Hkv
    if q is None:
        q = q_f64(w)
    if scale is None:
        scale = 1.0 / math.sqrt(w.d)
    K16, V16 = w.logical_kv(r, h, res.L[r][h])
    return decode_rows(q[r, h * G:(h + 1) * G], K16, V16, res.n_i8[r][h], w.quant_block, scale,
                       getattr(w, "old_bits", 8))


def decode(w, res: Optional[planner.Reservation] = None,
           pairs: Optional[Iterable[Tuple[int, int]]] = None,
           scale: Optional[float] = None) -> np.ndarray:
    """o [B][Hq][d] fp64 for every (r, h) in ``pairs`` (default: all); rows
    of pairs not computed are NaN."""
    if res is None:
        res = reserve_for(w)
    G = w.Hq // w.Hkv
    q = q_f64(w)
    out = np.full((w.B, w.Hq, w.d), np.nan)
    if pairs is None:
        pairs = [(r, h) for r in range(w.B) for h in range(w.Hkv)]
    for r, h in pairs:
        out[r, h * G:(h + 1) * G] = decode_pair(w, res, r, h, q, scale)
    return out
