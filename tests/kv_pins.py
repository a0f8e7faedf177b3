"""Pins of the FP8 KV-cache oracle (``oracle/fp8_kv.py``): every E4M3 value round-trips through a
power-of-two scale, ties between neighbours go to the even byte, large values saturate, signed zeros
and NaN keep their sign, the calibrated scale puts the largest element on 448, and the element rule
(product with the rounded reciprocal) is re-derived in exact rational arithmetic on an input where the
division rule rounds the other way.  Each check takes the module under test."""
from fractions import Fraction

import numpy as np

from oracle import nvfp4_ref as ref

F32 = np.float32


def _e4m3_exact():
    """All finite E4M3 magnitudes as exact rationals from the field definition (bias 7, 3 mantissa bits)."""
    vals = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        vals.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


def check_round_trip(o):
    vals = _e4m3_exact()
    for s in (0.25, 1.0, 64.0):
        x = np.array([[float(v) * s for v in vals] + [-float(v) * s for v in vals[1:]]], F32)
        c, s32 = o.quantize_kv(x, "given", s)
        assert list(c[0]) == list(range(0x7F)) + [0x80 | b for b in range(1, 0x7F)], s
        assert np.array_equal(o.dequantize_kv(c, s32), x.astype(np.float64))


def check_ties_and_saturation(o):
    vals = [float(v) for v in _e4m3_exact()]
    mids = np.array([[(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]], F32)   # exact in FP32
    c, _ = o.quantize_kv(mids, "given", 1.0)
    want = [i if i % 2 == 0 else i + 1 for i in range(0x7E)]                      # the even byte of each pair
    assert list(c[0]) == want
    c, _ = o.quantize_kv(np.array([[1e30, -1e30, 464.0, 479.9, -3e38]], F32), "given", 1.0)
    assert list(c[0]) == [0x7E, 0xFE, 0x7E, 0x7E, 0xFE]


def check_signs_zero_nan(o):
    c, _ = o.quantize_kv(np.array([[0.0, -0.0, 1e-30, -1e-30, np.nan, -np.nan]], F32), "given", 1.0)
    assert list(c[0]) == [0x00, 0x80, 0x00, 0x80, 0x7F, 0xFF]


def check_calibration(o):
    rng = np.random.default_rng(51)
    x = (rng.standard_normal((8, 40)) * 3).astype(F32)
    x[5, 7] = F32(-17.25)
    c, s = o.quantize_kv(x)
    assert F32(s) == F32(F32(17.25) / F32(448.0))
    assert c[5, 7] == 0xFE and np.all((c & 0x7F) <= 0x7E)
    c0, s0 = o.quantize_kv(np.zeros((2, 3), F32))
    assert s0 == F32(1.0) and np.all(c0 == 0)
    _, tiny = o.quantize_kv(np.full((1, 4), 1e-38, F32))
    assert tiny == F32(2.0 ** -100)


def _f32(q: Fraction) -> Fraction:
    """Round an exact rational to FP32 (via the correctly rounded double, exact for these operands)."""
    return Fraction(float(np.float32(float(q))))


def _nearest_e4m3(q: Fraction) -> int:
    vals = _e4m3_exact()
    a = abs(q)
    best = min(range(0x7F), key=lambda b: (abs(vals[b] - a), b & 1))   # ties: the even byte
    return best | (0x80 if q < 0 else 0)


def check_reciprocal_rule(o):
    """x = 1377.6282958984375, s = 5.554953098297119 (both FP32): fl32(x * fl32(1/s)) is exactly 248, the
    midpoint of 240 and 256, which ties to 256 (0x78); fl32(x / s) is just below 248 and would give 0x77."""
    x, s = Fraction(1377.6282958984375), Fraction(float(F32(5.554953098297119)))
    q_mul = _f32(x * _f32(1 / s))
    q_div = _f32(x / s)
    assert q_mul == 248 and q_div < 248
    assert _nearest_e4m3(q_mul) == 0x78 and _nearest_e4m3(q_div) == 0x77
    c, _ = o.quantize_kv(np.array([[1377.6282958984375, -1377.6282958984375]], F32), "given", float(s))
    assert list(c[0]) == [0x78, 0xF8]


def check_error_bound(o):
    """Inside the range every dequantized value is within half an E4M3 step (relative 2^-4) of x, or within
    2^-10 * s below the normal range."""
    rng = np.random.default_rng(52)
    x = (rng.standard_normal((16, 64)) * np.exp(rng.uniform(-6, 4, (16, 64)))).astype(F32)
    c, s = o.quantize_kv(x)
    back = o.dequantize_kv(c, s)
    err = np.abs(back - x.astype(np.float64))
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * float(s)) * (1 + 1e-6))


ALL_CHECKS = [check_round_trip, check_ties_and_saturation, check_signs_zero_nan, check_calibration,
              check_reciprocal_rule, check_error_bound]
