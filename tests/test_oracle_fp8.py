"""Pins of the oracle's FP8 e4m3fn codec and quantiser (CPU only)."""
import os

import numpy as np
import pytest

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_codes.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_decode_matches_hand_worked_codes():
    tab = fp8.decode_table()
    for code, val in _golden():
        if np.isnan(val):
            assert np.isnan(tab[code]), hex(code)
        else:
            assert tab[code] == val, hex(code)
            assert np.signbit(tab[code]) == np.signbit(val), hex(code)


def test_decode_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = fp8.decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert np.array_equal(ref[~nan], tab[~nan])
    assert nan.sum() == 2


def test_table_structure():
    tab = fp8.decode_table()
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0)                 # monotone in the code
    assert np.array_equal(tab[0x80:0xFF], -tab[0:0x7F])
    assert pos.max() == 448.0 and pos[1] == 2.0 ** -9


def test_encode_roundtrip_all_finite_codes():
    tab = fp8.decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    y = tab[codes].astype(np.float32)
    assert np.array_equal(fp8.encode(y), codes)


def test_encode_midpoints_ties_to_even_and_neighbours():
    tab = fp8.decode_table()
    for c in range(0, 0x7E):
        lo, hi = tab[c], tab[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2          # exact in float32
        even = c if c % 2 == 0 else c + 1
        for sgn, sbit in ((1, 0), (-1, 0x80)):
            m = np.float32(sgn * mid)
            assert fp8.encode(np.array([m]))[0] == (even | sbit), (hex(c), sgn)
            up = np.nextafter(m, np.float32(sgn * np.inf))
            dn = np.nextafter(m, np.float32(0))
            assert fp8.encode(np.array([up]))[0] == ((c + 1) | sbit)
            assert fp8.encode(np.array([dn]))[0] == (c | sbit)


def test_encode_saturates():
    y = np.array([448, 448.0001, 464, 479, 480, 1e6, 3e38], dtype=np.float32)
    assert np.all(fp8.encode(y) == 0x7E)
    assert np.all(fp8.encode(-y) == 0xFE)


def test_encode_signed_zero_and_underflow():
    y = np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, 2.0 ** -10 * 1.0001],
                 dtype=np.float32)
    # 2^-11 is below half the smallest subnormal (2^-10) -> 0; 2^-10 is a tie -> even 0;
    # just above the tie -> smallest subnormal.
    assert list(fp8.encode(y)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x01]


def test_encode_matches_torch_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    parts = [rng.uniform(-448, 448, 200000), rng.normal(0, 1, 200000),
             rng.uniform(-2.0 ** -5, 2.0 ** -5, 200000)]
    y = np.concatenate(parts).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(y), ref)


def test_quantize_rows_definition_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, 128)).astype(np.float32)
    x[3, 1] = 0.0                              # zero row
    x[4, 2] = -0.0
    x[5, 0, :] = 0.0
    x[5, 0, 7] = -3.5                          # single non-zero
    codes, scale = fp8.quantize_rows(x)
    a = np.max(np.abs(x), axis=-1)
    assert np.array_equal(scale, (a / np.float32(448)).astype(np.float32))
    assert scale[3, 1] == 0 and np.all(codes[3, 1] == 0)
    assert scale[4, 2] == 0 and np.all(codes[4, 2] == 0)
    # the absmax element of every non-zero row maps to +-448
    nz = a > 0
    idx = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], axis=-1)[..., 0]
    assert np.all((top[nz] & 0x7F) == 0x7E)
    assert codes[5, 0, 7] == 0xFE and np.all(np.delete(codes[5, 0], 7) == 0)
    # reconstruction error: half a code step (2^-4 relative for normals, 2^-10 * scale
    # for subnormals), plus the float32 rounding of x / scale
    deq = fp8.dequantize(codes, scale)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[..., None]) * (1 + 1e-6)
    assert np.all(err <= bound + 1e-30)


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        fp8.encode(np.array([np.nan], dtype=np.float32))
