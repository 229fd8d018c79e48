"""Pins of the oracle's RoPE (oracle/rope.py) against what the rotation fixes: the
identity, quarter and half turns (pairing and sign), the relative-position property,
composition of angles, and the float64 error bound of its float32 arithmetic."""
import numpy as np

import workloads as W
from oracle import rope


def _x(seed, T=5, H=3, D=16):
    return np.random.default_rng(seed).standard_normal((T, H, D)).astype(np.float32)


def _const_table(c, s, D=16, P=4):
    return np.full((P, D // 2), c, np.float32), np.full((P, D // 2), s, np.float32)


def test_zero_angle_is_identity():
    x = _x(0)
    c, s = _const_table(1.0, 0.0)
    assert np.array_equal(rope.rotate(x, np.zeros(5, np.int64), c, s), x)


def test_quarter_turn_pairs_i_with_i_plus_half():
    """cos 0, sin 1: (x_i, x_{i+D/2}) -> (-x_{i+D/2}, x_i), i.e. HF's rotate_half."""
    x = _x(1)
    c, s = _const_table(0.0, 1.0)
    r = rope.rotate(x, np.full(5, 2, np.int64), c, s)
    assert np.array_equal(r, np.concatenate([-x[..., 8:], x[..., :8]], axis=-1))


def test_half_turn_negates():
    x = _x(2)
    c, s = _const_table(-1.0, 0.0)
    assert np.array_equal(rope.rotate(x, np.ones(5, np.int64), c, s), -x)


def test_relative_position_and_composition():
    D = 64
    cos, sin = W.rope_tables(64, D, base=10000.0)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, D)).astype(np.float32)

    def dot(m, n):
        a = rope.rotate(q, np.array([m]), cos, sin).astype(np.float64)
        b = rope.rotate(k, np.array([n]), cos, sin).astype(np.float64)
        return float(np.sum(a * b))
    # <R(m) q, R(n) k> depends on m - n only
    for m, n, d in ((7, 3, 20), (40, 40, 9), (5, 30, 11)):
        assert abs(dot(m, n) - dot(m + d, n + d)) < 1e-4 * (1 + abs(dot(m, n)))
    assert abs(dot(9, 3) - dot(3, 9)) > 1e-3       # but not only on |m - n|
    # R(2) R(1) x = R(3) x
    x = _x(4, D=D)
    twice = rope.rotate(rope.rotate(x, np.ones(5, np.int64), cos, sin),
                        np.full(5, 2, np.int64), cos, sin)
    assert np.max(np.abs(twice - rope.rotate(x, np.full(5, 3, np.int64), cos, sin))) < 1e-5


def test_float32_error_bound_and_pair_norms():
    D = 128
    cos, sin = W.rope_tables(300, D)
    x = _x(5, T=40, H=4, D=D) * 30
    pos = np.random.default_rng(6).integers(0, 300, 40)
    r = rope.rotate(x, pos, cos, sin).astype(np.float64)
    a, b = x[..., :64].astype(np.float64), x[..., 64:].astype(np.float64)
    c = cos[pos][:, None, :].astype(np.float64)
    s = sin[pos][:, None, :].astype(np.float64)
    exact = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    mag = np.concatenate([np.abs(a * c) + np.abs(b * s), np.abs(b * c) + np.abs(a * s)], axis=-1)
    assert np.all(np.abs(r - exact) <= 2.0 ** -23 * mag * 1.01 + 1e-30)
    n0 = a * a + b * b
    n1 = r[..., :64] ** 2 + r[..., 64:] ** 2
    assert np.allclose(n1, n0 * (c * c + s * s), rtol=1e-5, atol=1e-6)


def test_bf16_round_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -7, -1.0 - 2 ** -8],
                 np.float32)
    assert rope.bf16_round(x).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0]
