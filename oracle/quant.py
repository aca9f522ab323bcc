"""Oracle for the slow tier's block-wise INT8 / INT4 quantiser -- TEST INFRASTRUCTURE.

TTKV page (arXiv 2604.19769 explainer), "Tier Layout" (slow tier holds older
KV states at INT8/INT4) and "Tier Interaction" (the slow tier is quantised in
blocks).  The page does not state the quantiser; the reading taken (also in
the design notes) is symmetric absmax per (block, channel):

    s   = fp16_rne(fp32(absmax) / 127)      (fp32 division, then round to fp16;
                                             +inf saturates to 65504)
    q8  = clamp(rint_half_even(fp32(x) / fp32(s)), -127, 127)   if s > 0
    q8  = 0                                                     if s == 0
    x^  = q8 * s                            (exact in fp32 and fp64)

K and V are quantised separately, each over a block of ``Qb`` consecutive
logical rows (the oldest rows of a sequence, block k = rows [k*Qb, (k+1)*Qb)).
The INT4 variant (same page, "INT8/INT4") is the same rule with 7 in place
of 127: s = fp16_rne(absmax / 7), q4 = clamp(rint(x / s), -7, 7).

The code decision (q8) is taken from fp32 arithmetic, the same precision the
device kernel uses, so both sides must agree bit for bit.

Pinned by: tests/test_oracle_quant.py (|x - x^| <= s/2 when no clamp, the
absmax element maps to +-127, exact round trip of integer multiples of a
power-of-two scale, the all-zero block, saturation, symmetry x -> -x).
"""
from __future__ import annotations

import numpy as np

FP16_MAX = np.float16(65504.0)


def qmax_of(bits: int) -> int:
    """Largest code magnitude of a ``bits``-bit symmetric code (127 or 7)."""
    assert bits in (8, 4)
    return (1 << (bits - 1)) - 1


def block_scale(x: np.ndarray, bits: int = 8) -> np.ndarray:
    """Per-channel fp16 scale of one block ``x`` [Qb][d] (fp32 values)."""
    x = np.asarray(x, dtype=np.float32)
    absmax = np.max(np.abs(x), axis=0)
    with np.errstate(over="ignore"):
        s = (absmax / np.float32(qmax_of(bits))).astype(np.float16)
    return np.where(np.isinf(s), FP16_MAX, s).astype(np.float16)


def quantize_block(x: np.ndarray, bits: int = 8):
    """Quantise one block ``x`` [Qb][d] (fp32 values) -> (codes int8 [Qb][d], s fp16 [d])."""
    x = np.asarray(x, dtype=np.float32)
    qm = qmax_of(bits)
    s = block_scale(x, bits)
    sf = s.astype(np.float32)
    pos = sf > 0
    safe = np.where(pos, sf, np.float32(1.0))
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.rint(x / safe)
    q = np.where(pos, np.clip(y, -qm, qm), 0).astype(np.int8)
    return q, s


def quantize_rows(x: np.ndarray, qb: int, bits: int = 8):
    """Quantise rows [n][d] (n a multiple of ``qb``) block by block.

    Returns (codes [n][d] int8, scales [n/qb][d] fp16)."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    assert n % qb == 0
    qs, ss = [], []
    for k in range(n // qb):
        q, s = quantize_block(x[k * qb:(k + 1) * qb], bits)
        qs.append(q)
        ss.append(s)
    if not qs:
        return np.zeros((0, x.shape[1]), np.int8), np.zeros((0, x.shape[1]), np.float16)
    return np.concatenate(qs), np.stack(ss)


def dequantize_rows(q: np.ndarray, s: np.ndarray, qb: int) -> np.ndarray:
    """fp64 values q8 * s of rows quantised by ``quantize_rows``."""
    q = np.asarray(q, dtype=np.float64)
    sf = np.repeat(np.asarray(s, dtype=np.float64), qb, axis=0)
    return q * sf
