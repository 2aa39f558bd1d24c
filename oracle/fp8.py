"""Row-scaled E4M3 state -- TEST INFRASTRUCTURE ONLY.

The FP8 state of the Systolic Linear Attention serving study (section 3.2,
"row-scaled E4M3"): row i of a (batch, value head) state -- the d_v values
of key channel i -- is stored as E4M3 codes with one fp32 scale per row.

E4M3 here is the OCP 8-bit floating-point format with 4 exponent bits (bias
7) and 3 mantissa bits in which exponent field 15 with mantissa 7 is NaN and
there is no infinity: code s.eeee.mmm is (-1)^s 2^(e-7) (1 + m/8) for
e >= 1 and (-1)^s 2^-6 (m/8) for e = 0; the largest finite value, 0x7E, is
448.  Encoding rounds to the nearest finite value, ties to the code with the
even mantissa, and saturates at +-448.

Quantising a row (this build's reading of "row-scaled"): amax = max |x|,
scale = amax / 448, codes = E4M3(x * (448 / amax)), each step in fp32 (the
division and the product correctly rounded); a zero row has scale 0 and
codes 0.  Dequantising: value(code) * scale in fp32.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """Values of E4M3 codes (uint8 array) as float64 (NaN for 0x7F, 0xFF)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: the finite non-negative values
_POS_VALUES = e4m3_value(_POS_CODES)                  # increasing


def e4m3_encode(x):
    """Nearest E4M3 code (ties to even mantissa), saturating at +-448; the sign
    of zero is kept."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_lo = np.abs(a - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - a)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0) & (hi != lo))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(x):
    """fp32 array [..., d_v] -> (codes uint8 [..., d_v], scale fp32 [...])."""
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    safe = np.where(amax > 0, amax, np.float32(1.0))
    inv = np.where(amax > 0, np.float32(E4M3_MAX) / safe, np.float32(0.0)).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    codes = e4m3_encode(y)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return codes, scale


def dequantize_rows(codes, scale):
    """(codes, scale) -> fp32 array: value(code) * scale in fp32."""
    v = e4m3_value(codes).astype(np.float32)
    return (v * np.asarray(scale, np.float32)[..., None]).astype(np.float32)
