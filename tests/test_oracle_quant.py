"""Pins for the INT8 / INT4 block quantiser oracle (oracle/quant.py): properties the
symmetric absmax rule fixes, checked without re-typing the rule."""
import numpy as np

from oracle import quant


def _rand_block(seed, qb=64, d=128, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((qb, d)) * scale).astype(np.float32)


def test_error_bounded_by_half_step_and_absmax_hits_127():
    x = _rand_block(1)
    q, s = quant.quantize_block(x)
    sf = s.astype(np.float64)
    xh = q.astype(np.float64) * sf
    # absmax / 127 rounded to fp16 is within 2^-11 relative of the ideal step
    absmax = np.abs(x).max(axis=0).astype(np.float64)
    assert np.all(np.abs(sf - absmax / 127) <= absmax / 127 * 2.0 ** -11 + 1e-30)
    unclamped = np.abs(q) < 127
    err = np.abs(x.astype(np.float64) - xh)
    assert np.all(err[unclamped] <= (sf / 2 * (1 + 1e-6) + 1e-30)[None, :].repeat(64, 0)[unclamped])
    # the element of largest magnitude in each channel lands on +-127 (or 126
    # when fp16 rounding of the step went up)
    idx = np.abs(x).argmax(axis=0)
    top = np.abs(q[idx, np.arange(x.shape[1])])
    assert np.all((top == 127) | (top == 126))
    assert np.all(np.abs(q) <= 127)


def test_integer_multiples_of_power_of_two_step_round_trip_exactly():
    g = np.random.default_rng(2)
    k = g.integers(-127, 128, size=(64, 32))
    k[0, :] = 127                      # pin absmax so the step is exactly 2^-5
    x = (k * 2.0 ** -5).astype(np.float32)
    q, s = quant.quantize_block(x)
    assert np.all(s == np.float16(2.0 ** -5))
    assert np.array_equal(q.astype(np.int64), k)
    assert np.array_equal(quant.dequantize_rows(q, s[None, :], 64), x.astype(np.float64))


def test_ties_round_to_even():
    x = np.zeros((64, 4), np.float32)
    x[0, :] = 127 * 2.0 ** -5
    x[1, :] = np.array([2.5, 3.5, -2.5, -0.5]) * 2.0 ** -5
    q, s = quant.quantize_block(x)
    assert list(q[1]) == [2, 4, -2, 0]


def test_zero_block_and_sign_symmetry_and_saturation():
    q, s = quant.quantize_block(np.zeros((64, 8), np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    x = _rand_block(3, d=16)
    q1, s1 = quant.quantize_block(x)
    q2, s2 = quant.quantize_block(-x)
    assert np.array_equal(s1, s2) and np.array_equal(q1, -q2)
    big = np.full((64, 2), 1e30, np.float32)
    q, s = quant.quantize_block(big)
    assert np.all(s == np.float16(65504.0)) and np.all(q == 127)


def test_rows_are_quantised_block_by_block():
    x = np.concatenate([_rand_block(4, d=8), 100 * _rand_block(5, d=8)])
    q, s = quant.quantize_rows(x, 64)
    assert s.shape == (2, 8)
    q0, s0 = quant.quantize_block(x[:64])
    q1, s1 = quant.quantize_block(x[64:])
    assert np.array_equal(q[:64], q0) and np.array_equal(q[64:], q1)
    assert np.array_equal(s[0], s0) and np.array_equal(s[1], s1)
    # the second block's larger values get a proportionally larger step
    assert np.all(s[1].astype(np.float64) > 10 * s[0].astype(np.float64))


# ---------------------------------------------------------------- INT4 (codes in [-7, 7])
def test_int4_error_bounded_and_absmax_hits_7():
    x = _rand_block(11)
    q, s = quant.quantize_block(x, 4)
    sf = s.astype(np.float64)
    absmax = np.abs(x).max(axis=0).astype(np.float64)
    assert np.all(np.abs(sf - absmax / 7) <= absmax / 7 * 2.0 ** -11 + 1e-30)
    assert np.all(np.abs(q) <= 7)
    unclamped = np.abs(q) < 7
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * sf)
    assert np.all(err[unclamped] <= (sf / 2 * (1 + 1e-6) + 1e-30)[None, :].repeat(64, 0)[unclamped])
    idx = np.abs(x).argmax(axis=0)
    top = np.abs(q[idx, np.arange(x.shape[1])])
    assert np.all((top == 7) | (top == 6))


def test_int4_exact_round_trip_and_ties():
    g = np.random.default_rng(12)
    k = g.integers(-7, 8, size=(64, 32))
    k[0, :] = 7                        # absmax 7 * 2^-3: step exactly 2^-3
    x = (k * 2.0 ** -3).astype(np.float32)
    q, s = quant.quantize_block(x, 4)
    assert np.all(s == np.float16(2.0 ** -3))
    assert np.array_equal(q.astype(np.int64), k)
    y = np.zeros((64, 4), np.float32)
    y[0, :] = 7.0
    y[1, :] = [2.5, 3.5, -2.5, -0.5]
    q, s = quant.quantize_block(y, 4)
    assert list(q[1]) == [2, 4, -2, 0]
    q, s = quant.quantize_block(np.full((64, 2), 1e30, np.float32), 4)
    assert np.all(s == np.float16(65504.0)) and np.all(q == 7)
    q, s = quant.quantize_block(np.zeros((64, 3), np.float32), 4)
    assert np.all(q == 0) and np.all(s == 0)


def test_int4_is_coarser_than_int8_on_the_same_block():
    x = _rand_block(13)
    e8 = np.abs(quant.dequantize_rows(*quant.quantize_rows(x, 64, 8), 64) - x).mean()
    e4 = np.abs(quant.dequantize_rows(*quant.quantize_rows(x, 64, 4), 64) - x).mean()
    # the step is 127/7 ~ 18x larger; mean error of a uniform rounding grows alike
    assert 10 < e4 / e8 < 30
