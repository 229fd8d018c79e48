"""OCP FP8 e4m3fn codec and the per-token-per-head quantiser (oracle; test infrastructure).

The pages only say that FP8/INT8 quantisation keeps per-tensor k_scale / v_scale
buffers beside the cache (PocketLLM "cpp_engine Batching Implementation (Phase 3.1)",
"current KV cache structure"). The reading used here: the OCP 8-bit e4m3fn format
(1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, the single
NaN pattern S.1111.111, largest finite value 448, subnormals m * 2^-9), one fp32 scale
per (token, KV head) row equal to absmax / 448, round-to-nearest-even with saturation
to +-448, and a zero row giving scale 0 and codes 0.

Pinned by: the decode table against the closed-form values of the format
(tests/golden/e4m3fn_codes.txt) and against torch.float8_e4m3fn; the encoder against
every midpoint between adjacent codes (ties to even), the neighbours of each midpoint,
saturation, and torch's in-range cast.
"""
import numpy as np

E4M3_MAX = 448.0


def decode_table():
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF), from the format."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = decode_table()
# Non-negative finite codes 0x00..0x7E have strictly increasing values.
_POS_VALUES = _TABLE[:0x7F].copy()


def decode(codes):
    """Exact float64 values of uint8 codes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y):
    """Nearest e4m3fn code to each float32 value y (ties to the even code, |y| > 448
    saturates to +-448, the sign of y is kept, so -0.0 and tiny negatives give 0x80).
    y must be finite. Works in float64, where y, the code values and their midpoints are
    all exact, so every comparison below is exact."""
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("encode: non-finite input")
    a = np.abs(y.astype(np.float64)).ravel()
    neg = np.signbit(y).ravel()
    # index of the first code value >= a (clipped into range)
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= _POS_VALUES[0x7E], 0x7E, code)  # saturation
    code = np.where(a <= 0.0, 0, code)
    code = code.astype(np.uint8) | (neg.astype(np.uint8) << 7)
    return code.reshape(y.shape)


def quantize_rows(x):
    """Per-row quantiser: x is float32 [..., D] (exact source values).

    For each row: a = max |x| in float32, scale = float32(a) / float32(448) (IEEE
    division, correctly rounded), y = x / scale in float32, codes = encode(y). A row
    with a == 0 gets scale 0 and codes 0x00. Returns (codes uint8 [..., D],
    scale float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    scale = (a / np.float32(E4M3_MAX)).astype(np.float32)
    zero = a == 0
    safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    codes = encode(y)
    codes[zero] = 0
    scale = np.where(zero, np.float32(0.0), scale).astype(np.float32)
    return codes, scale


def dequantize(codes, scale):
    """float64 values code * scale (exact: 4 + 24 significant bits fit in 53)."""
    return decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]
