"""Oracle for the lossless bf16 exponent codec -- TEST INFRASTRUCTURE.

SplitZip page ("Die SplitZip-Strategie", "Warum es schnell ist"): a bf16
value is sign, 8-bit exponent and 7-bit mantissa; exponents repeat a lot,
so the 16 most frequent ones get 4-bit codes, two codes share a byte, and
the values whose exponent is not among them are listed in a sparse escape
stream (position, exponent) that the decoder writes over its first result.
The page gives no byte format; the reading taken (also in the design notes):

R-zip  codebook: the 16 exponents with the highest counts over the whole
       input, ties to the smaller exponent (exponents that never occur rank
       after every one that does, by value); code of a value = rank of its
       exponent, or 0 when the exponent is not in the codebook (escaped).
       Compressed buffer, little endian, n a multiple of 8:
         [0, 8)     n (int64)          [8, 16)   n_esc (int64)
         [16, 32)   codebook (16 uint8, rank order)        [32, 256)  zero
         [256, 256 + n)                 sign << 7 | mantissa, one byte per value
         [256 + n, 256 + 3n/2)          codes, value i in bits 4(i%2).. of byte i/2
         [256 + 3n/2, + 4 n_esc)        escape positions, uint32, ascending
         [.., + n_esc)                  escape exponents, uint8
       size = 256 + 3n/2 + 5 n_esc.

Plain numpy; pinned by tests/test_oracle_splitzip.py (hand-worked golden
buffer, round trips over random and special bit patterns, the codebook
against a brute-force count, the size formula).
"""
from __future__ import annotations

import numpy as np

HEADER = 256


def exponents(x: np.ndarray) -> np.ndarray:
    return ((np.asarray(x, dtype=np.uint16) >> 7) & 0xFF).astype(np.int64)


def codebook(x: np.ndarray) -> np.ndarray:
    """The 16 exponents in rank order (R-zip)."""
    counts = np.bincount(exponents(x), minlength=256)
    order = sorted(range(256), key=lambda e: (-counts[e], e))
    return np.array(order[:16], dtype=np.uint8)


def encode(x: np.ndarray) -> bytes:
    x = np.asarray(x, dtype=np.uint16).ravel()
    n = x.size
    if n % 8:
        raise ValueError("n must be a multiple of 8")
    book = codebook(x)
    code_of = {int(e): k for k, e in enumerate(book)}
    ex = exponents(x)
    codes = np.array([code_of.get(int(e), 0) for e in ex], dtype=np.uint8)
    sm = (((x >> 15) << 7) | (x & 0x7F)).astype(np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    esc = [i for i in range(n) if int(ex[i]) not in code_of]
    out = bytearray(HEADER)
    out[0:8] = np.int64(n).tobytes()
    out[8:16] = np.int64(len(esc)).tobytes()
    out[16:32] = book.tobytes()
    out += sm.tobytes() + packed.tobytes()
    out += np.array(esc, dtype=np.uint32).tobytes()
    out += np.array([ex[i] for i in esc], dtype=np.uint8).tobytes()
    return bytes(out)


def decode(buf: bytes) -> np.ndarray:
    b = np.frombuffer(buf, dtype=np.uint8)
    n = int(np.frombuffer(buf[0:8], np.int64)[0])
    n_esc = int(np.frombuffer(buf[8:16], np.int64)[0])
    book = b[16:32].astype(np.uint16)
    sm = b[HEADER:HEADER + n].astype(np.uint16)
    packed = b[HEADER + n:HEADER + n + n // 2]
    codes = np.empty(n, np.uint8)
    codes[0::2] = packed & 0x0F
    codes[1::2] = packed >> 4
    x = ((sm >> 7) << 15) | (book[codes] << 7) | (sm & 0x7F)
    p0 = HEADER + n + n // 2
    pos = np.frombuffer(buf[p0:p0 + 4 * n_esc], np.uint32)
    exps = b[p0 + 4 * n_esc:p0 + 5 * n_esc].astype(np.uint16)
    for i, e in zip(pos, exps):
        x[i] = (x[i] & 0x807F) | (e << 7)
    return x.astype(np.uint16)


def size(n: int, n_esc: int) -> int:
    return HEADER + n + n // 2 + 5 * n_esc
