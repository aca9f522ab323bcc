"""Pins for the lossless bf16 exponent codec oracle (oracle/splitzip.py):
a hand-worked buffer, bit-exact round trips (random, heavy-tailed and
special bit patterns), the codebook against a brute-force count, the size
formula."""
import collections
import json
import os

import numpy as np

from oracle import splitzip as Z

GOLD = os.path.join(os.path.dirname(__file__), "golden", "splitzip_hand.json")


def test_hand_worked_buffer():
    g = json.load(open(GOLD))
    x = np.array([int(v, 16) for v in g["values"]], np.uint16)
    b = Z.encode(x)
    n = x.size
    assert len(b) == g["size"] == Z.size(n, g["n_esc"])
    assert np.frombuffer(b[0:8], np.int64)[0] == n and np.frombuffer(b[8:16], np.int64)[0] == g["n_esc"]
    assert list(b[16:32]) == g["codebook"] and not any(b[32:256])
    assert list(b[256:256 + n]) == g["sm"]
    assert list(b[256 + n:256 + n + n // 2]) == g["packed"]
    p0 = 256 + n + n // 2
    assert list(np.frombuffer(b[p0:p0 + 16], np.uint32)) == g["esc_pos"]
    assert list(b[p0 + 16:p0 + 20]) == g["esc_exp"]
    assert np.array_equal(Z.decode(b), x)


def test_round_trips_bit_exact():
    g = np.random.default_rng(9)
    cases = [
        g.integers(0, 2 ** 16, size=4096, dtype=np.uint16),                     # every bit pattern
        (g.standard_normal(8192).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16),
        (g.standard_cauchy(8192).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16),
        np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x807F, 0x3F80] * 3, np.uint16),
        np.full(64, 0x4049, np.uint16),                                          # one exponent only
    ]
    for x in cases:
        assert np.array_equal(Z.decode(Z.encode(x)), x)


def test_codebook_is_the_sixteen_most_frequent():
    g = np.random.default_rng(10)
    for _ in range(20):
        e = g.integers(90, 140, size=2000)
        x = ((g.integers(0, 2, size=2000) << 15) | (e << 7) | g.integers(0, 128, size=2000)).astype(np.uint16)
        cnt = collections.Counter(int(v) for v in e)
        ranked = sorted(range(256), key=lambda k: (-cnt.get(k, 0), k))[:16]
        book = list(Z.codebook(x))
        assert book == ranked
        b = Z.encode(x)
        n_esc = int(np.frombuffer(b[8:16], np.int64)[0])
        assert n_esc == sum(c for k, c in cnt.items() if k not in ranked)
        assert len(b) == Z.size(2000, n_esc)
