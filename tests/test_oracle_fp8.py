"""Pins of the row-scaled E4M3 oracle (no GPU): code values from the format's
definition, round trips, ties to even, saturation, and the row scaling."""
import numpy as np

from oracle.fp8 import dequantize_rows, e4m3_encode, e4m3_value, quantize_rows


def test_code_values_from_the_definition():
    # s.eeee.mmm: 0x01 smallest subnormal 2^-9, 0x07 = 7 * 2^-9, 0x08 smallest
    # normal 2^-6, 0x38 = 1, 0x3F = 1.875, 0x40 = 2, 0x7E = 448 (1.75 * 2^8),
    # 0x80 = -0, 0xFE = -448; 0x7F and 0xFF are NaN
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3F: 1.875,
             0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for code, val in table.items():
        assert e4m3_value(np.uint8(code)) == val, hex(code)
    assert np.isnan(e4m3_value(np.uint8(0x7F))) and np.isnan(e4m3_value(np.uint8(0xFF)))
    assert np.signbit(e4m3_value(np.uint8(0x80)))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    v = e4m3_value(finite)
    assert np.array_equal(e4m3_encode(v), finite)                  # every finite code round-trips
    pos = e4m3_value(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                               # codes 0..0x7E increase


def test_rounding_ties_to_even_and_saturation():
    # halfway between 1 (0x38, mantissa 0) and 1.125 (0x39): even -> 0x38;
    # halfway between 1.125 and 1.25 (0x3A): even -> 0x3A
    assert e4m3_encode(1.0625) == 0x38 and e4m3_encode(1.1875) == 0x3A
    assert e4m3_encode(-1.1875) == 0xBA
    # subnormal ties: 0.5 * 2^-9 -> 0x00, 1.5 * 2^-9 -> 0x02
    assert e4m3_encode(0.5 * 2.0 ** -9) == 0x00 and e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    # just off the tie goes to the nearer value
    assert e4m3_encode(1.0625 + 1e-6) == 0x39
    # the top binade: 0x7C = 384, 0x7D = 416, 0x7E = 448 (2^8 times 1.5, 1.625, 1.75)
    assert e4m3_value(np.uint8(0x7D)) == 416.0
    assert e4m3_encode(440.0) == 0x7E and e4m3_encode(1e6) == 0x7E and e4m3_encode(-1e6) == 0xFE
    assert e4m3_encode(-0.0) == 0x80 and e4m3_encode(0.0) == 0x00


def test_encoding_is_nearest():
    r = np.random.default_rng(0)
    x = r.uniform(-448, 448, 20000) * 10.0 ** r.uniform(-4, 0, 20000)
    c = e4m3_encode(x)
    err = np.abs(e4m3_value(c) - x)
    finite = e4m3_value(np.array([c_ for c_ in range(256) if c_ not in (0x7F, 0xFF)], np.uint8))
    best = np.min(np.abs(x[:, None] - finite[None, :]), axis=1)
    assert np.array_equal(err, best)


def test_row_scaling():
    r = np.random.default_rng(1)
    x = (r.standard_normal((3, 5, 64)) * 10.0 ** r.uniform(-3, 2, (3, 5, 1))).astype(np.float32)
    x[1, 2] = 0.0                                                  # a zero row
    codes, scale = quantize_rows(x)
    assert scale[1, 2] == 0 and not codes[1, 2].any()
    amax = np.max(np.abs(x), axis=-1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest entry of each row lands on +-448 (code 0x7E or 0xFE)
    idx = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    nz = amax > 0
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # dequantised values are within half an E4M3 step: 2^-4 relative in the
    # normal range, 2^-10 scale in the subnormal range
    y = dequantize_rows(codes, scale)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * scale[..., None]) * 1.0001
    assert np.all(np.abs(y - x) <= bound)
