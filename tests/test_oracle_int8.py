"""Pins of the oracle's symmetric int8 quantiser (oracle/int8.py) against what its
definition fixes: exact round trips, ties to even, the absmax code, odd symmetry, the
error bound, zero rows."""
import numpy as np

from oracle import int8


def test_round_half_even_ties_and_neighbours():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.49999997, 0.50000006, 126.5, -126.5])
    got = int8.round_half_even(np.float32(y).astype(np.float64))
    assert got.tolist() == [0, 2, 2, -0, -2, -2, 0, 1, 126, -126]


def test_exact_multiples_round_trip():
    rng = np.random.default_rng(0)
    for _ in range(20):
        s = np.float32(2.0) ** rng.integers(-10, 10)       # power of two: x/scale exact
        k = rng.integers(-127, 128, size=64).astype(np.float32)
        k[0] = 127.0                                         # absmax hits the top code
        x = (k * s).astype(np.float32)
        codes, scale = int8.quantize_rows(x[None])
        assert scale[0] == np.float32(127.0 * s) / np.float32(127.0)
        assert np.array_equal(codes[0].astype(np.float32), k)
        assert np.array_equal(int8.dequantize(codes, scale)[0], x.astype(np.float64))


def test_absmax_maps_to_127_and_codes_are_odd():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    c, s = int8.quantize_rows(x)
    cn, sn = int8.quantize_rows(-x)
    assert np.array_equal(s, sn)
    assert np.array_equal(cn, -c)
    assert np.all(np.max(np.abs(c.astype(np.int32)), axis=1) == 127)
    assert c.min() >= -127 and c.max() <= 127


def test_error_bound_and_zero_row():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((200, 64)) * rng.uniform(1e-3, 1e3, (200, 1))).astype(np.float32)
    x[3] = 0.0
    c, s = int8.quantize_rows(x)
    assert s[3] == 0 and not c[3].any()
    err = np.abs(int8.dequantize(c, s) - x.astype(np.float64))
    # half a step, plus the float32 rounding of x / scale (relative 2^-24 of 127 steps)
    bound = s.astype(np.float64)[:, None] * (0.5 + 127 * 2.0 ** -23)
    assert np.all(err <= bound)
