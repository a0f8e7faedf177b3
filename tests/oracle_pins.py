"""Pins for the CPU oracle: facts fixed by the format definitions and the mathematics.

Each ``check_*`` takes an oracle module (``oracle.nvfp4_ref`` or a copy with a
planted mistake) and raises AssertionError when the oracle disagrees with the
pin.  The references used here are independent of the oracle's code:

* the E2M1 / E4M3 value sets are rebuilt as integer significand times a power
  of two (not from bit fields) and checked against well-known values;
* nearest-value rounding is redone by brute force in exact rational arithmetic
  (``fractions.Fraction``) over all codes;
* hand-worked examples live in ``tests/golden/`` with their derivations;
* GEMM results are checked with exact rational triple loops, closed forms and
  invariants.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32

# ---------------------------------------------------------------------------
# Independent value sets: integer significand x power of two.
# ---------------------------------------------------------------------------


def e2m1_set():
    """{code: Fraction} for codes 0..7. Subnormal: m/2 (m = 0, 1); normal: (2+m) * 2^(e-2), e = 1..3."""
    vals = {0: Fraction(0), 1: Fraction(1, 2)}
    for e in (1, 2, 3):
        for m in (0, 1):
            vals[2 * e + m] = Fraction(2 + m) * Fraction(2) ** (e - 2)
    return vals


def e4m3_set():
    """{byte: Fraction} for the 127 finite non-negative E4M3 bytes.

    Subnormal: m * 2^-9 (m = 0..7); normal: (8+m) * 2^(e-10), e = 1..15, excluding e = 15, m = 7 (NaN).
    """
    vals = {m: Fraction(m, 512) for m in range(8)}
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals[8 * e + m] = Fraction(8 + m) * Fraction(2) ** (e - 10)
    return vals


E2M1 = e2m1_set()
E4M3 = e4m3_set()


def brute_nearest(x: float, table: dict) -> int:
    """argmin_code |x - table[code]| in exact arithmetic; ties -> even code; above the max -> max code."""
    fx = Fraction(float(x))
    best, best_d = None, None
    for code in sorted(table):
        d = abs(fx - table[code])
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    top = max(table, key=lambda c: table[c])
    if fx >= table[top]:
        return top
    return best


def _f32_neighbors(v):
    v = F32(v)
    return [np.nextafter(v, F32(-np.inf)), v, np.nextafter(v, F32(np.inf))]


# ---------------------------------------------------------------------------
# Formats
# ---------------------------------------------------------------------------


def check_e2m1_values(ref):
    for c in range(16):
        want = float(E2M1[c & 7]) * (-1.0 if c & 8 else 1.0)
        got = ref.e2m1_value(c)
        assert got == want and np.signbit(got) == bool(c & 8), (c, got, want)
    assert [float(E2M1[c]) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(ref.E2M1_MAGS) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def check_e4m3_values(ref):
    for b in range(127):
        assert ref.e4m3_value(b) == float(E4M3[b]), b
        assert ref.e4m3_value(b | 0x80) == -float(E4M3[b]), b
    assert np.isnan(ref.e4m3_value(0x7F)) and np.isnan(ref.e4m3_value(0xFF))
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x48: 4.0, 0x77: 240.0, 0x7E: 448.0}
    for b, v in known.items():
        assert ref.e4m3_value(b) == v, (hex(b), ref.e4m3_value(b), v)
    assert list(ref.E4M3_VALS) == [float(E4M3[b]) for b in range(127)]
    assert np.all(np.diff(ref.E4M3_VALS) > 0)


def check_roundtrip(ref):
    for c in range(16):
        v = F32(ref.e2m1_value(c))
        if c == 8:
            v = F32(-0.0)
        assert int(ref.e2m1_encode(np.array([v], F32))[0]) == c, c
    for b in range(127):
        assert int(ref.e4m3_encode(np.array([ref.e4m3_value(b)], F32))[0]) == b, b


def check_e4m3_bruteforce(ref, n_random=3000, seed=7):
    rng = np.random.default_rng(seed)
    pts = []
    vals = sorted(E4M3.values())
    for lo, hi in zip(vals[:-1], vals[1:]):
        pts += _f32_neighbors(float((lo + hi) / 2))
        pts += _f32_neighbors(float(hi))
    pts += list(F32(2.0) ** rng.uniform(-14, 9.8, n_random).astype(F32))
    pts += [F32(0), F32(448), F32(464), F32(480), F32(1e6), F32(3e38), F32(2.0 ** -149)]
    pts = np.array(pts, dtype=F32)
    got = ref.e4m3_encode(pts)
    for x, gc in zip(pts, got):
        want = brute_nearest(float(x), E4M3)
        assert int(gc) == want, (float(x), int(gc), want)


def check_e2m1_bruteforce(ref, n_random=3000, seed=8):
    rng = np.random.default_rng(seed)
    pts = []
    vals = sorted(E2M1.values())
    for lo, hi in zip(vals[:-1], vals[1:]):
        pts += _f32_neighbors(float((lo + hi) / 2))
        pts += _f32_neighbors(float(hi))
    pts += list(rng.uniform(-8, 8, n_random).astype(F32))
    pts += [F32(0), F32(-0.0), F32(6), F32(7), F32(-100), F32(2.0 ** -149), F32(-(2.0 ** -149))]
    pts = np.array(pts, dtype=F32)
    got = ref.e2m1_encode(pts)
    for x, gc in zip(pts, got):
        want = brute_nearest(abs(float(x)), E2M1) | (8 if np.signbit(x) else 0)
        assert int(gc) == want, (float(x), int(gc), want)


def check_e2m1_thresholds(ref):
    """Threshold form of E2M1 round-to-nearest-even (ties: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4)."""
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.2500001: 1, 0.7499999: 1, 1.2500001: 3, 1.7499999: 3, 2.5000002: 5, 3.4999998: 5, 5.0000005: 7,
             6.0: 7, 6.5: 7, 1000.0: 7}
    for q, code in cases.items():
        assert int(ref.e2m1_encode(np.array([q], F32))[0]) == code, (q, code)
        assert int(ref.e2m1_encode(np.array([-q], F32))[0]) == code | 8, (-q, code)


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------


def check_global_scale(ref):
    for k in range(-20, 21):
        amax = F32(2688.0 * 2.0 ** -k)
        g = ref.global_scale(amax)
        assert g == F32(2.0 ** -k), (k, g)
        assert F32(1.0) / g == F32(2.0 ** k)
    assert ref.global_scale(F32(40.0)) == F32(40.0) / F32(2688.0)
    assert abs(float(ref.global_scale(F32(40.0))) - 40.0 / 2688.0) < 1e-9
    assert ref.global_scale(F32(0.0)) == F32(1.0)
    assert ref.global_scale(F32(1e-38)) == F32(2.0 ** -100)


def load_golden(name):
    data = {"x": [], "nibbles": [], "scales": [], "bytes0": []}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            if key == "x":
                data["x"] += [float(t) for t in val.split()]
            elif key == "g":
                data["g"] = float(val)
            elif key in ("nibbles", "scales", "bytes0"):
                data[key] += [int(t, 16) for t in val.split()]
    return data


def check_golden_given(ref):
    d = load_golden("worked_given_g.txt")
    x = np.array(d["x"], dtype=F32)[None, :]
    q = ref.quantize(x, g_mode="given", g=d["g"])
    assert list(q.scales[0]) == d["scales"], (list(q.scales[0]), d["scales"])
    nib = ref.unpack_codes(q.codes)[0]
    assert list(nib) == d["nibbles"], (list(nib), d["nibbles"])
    assert list(q.codes[0][:8]) == d["bytes0"]
    assert q.g == F32(1.0)


def check_golden_computed(ref):
    d = load_golden("worked_computed_g.txt")
    x = np.array(d["x"], dtype=F32)[None, :]
    q = ref.quantize(x)
    assert q.g == F32(d["g"]), q.g
    assert list(q.scales[0]) == d["scales"], (list(q.scales[0]), d["scales"])
    assert list(ref.unpack_codes(q.codes)[0]) == d["nibbles"]


def check_golden_op_order(ref):
    d = load_golden("worked_op_order.txt")
    x = np.array(d["x"], dtype=F32)[None, :]
    q = ref.quantize(x, g_mode="given", g=d["g"])
    assert list(q.scales[0]) == d["scales"], (list(q.scales[0]), d["scales"])
    assert list(ref.unpack_codes(q.codes)[0]) == d["nibbles"]


def check_amax_block(ref):
    """amax = 2688 * 2^-k: its block gets S = 448 (0x7E) and the amax element the code for 6."""
    rng = np.random.default_rng(3)
    for k in (-3, 0, 5, 12):
        x = rng.standard_normal((4, 64)).astype(F32)
        amax = F32(2688.0 * 2.0 ** -k)
        x *= amax / F32(np.abs(x).max()) / F32(2)
        x[2, 37] = -amax
        q = ref.quantize(x)
        assert q.g == F32(2.0 ** -k)
        assert q.scales[2, 37 // 16] == 0x7E
        assert ref.unpack_codes(q.codes)[2, 37] == 0xF


def check_outlier_locality(ref):
    """With a fixed g, changing one element changes only its own block's scale byte and 8 code bytes."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 256)).astype(F32)
    g = F32(0.05)
    base = ref.quantize(x, g_mode="given", g=g)
    for (r, c, val) in [(3, 100, 40.0), (0, 0, -40.0), (7, 255, 30 * float(x[7, 255])), (5, 17, 1e-3)]:
        y = x.copy()
        y[r, c] = val
        q = ref.quantize(y, g_mode="given", g=g)
        b = c // 16
        ds = np.argwhere(q.scales != base.scales)
        assert all((i == r and j == b) for i, j in ds), ds
        dc = np.argwhere(q.codes != base.codes)
        assert all((i == r and b * 8 <= j < b * 8 + 8) for i, j in dc), dc
    # and an outlier that raises a block's max does change that block's scale
    y = x.copy()
    y[3, 100] = 40.0
    assert ref.quantize(y, g_mode="given", g=g).scales[3, 6] != base.scales[3, 6]


def check_dynamic_g_outlier(ref):
    """With a computed g, an outlier that raises the tensor amax rescales every block (documented contrast)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 128)).astype(F32)
    base = ref.quantize(x)
    y = x.copy()
    y[0, 0] = 40.0 * float(np.abs(x).max())
    q = ref.quantize(y)
    assert q.g > base.g
    assert np.count_nonzero(q.scales != base.scales) > q.scales.size // 2


def check_pow2_equivariance(ref):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 128)).astype(F32)
    x[1, 5] = 17.0
    base = ref.quantize(x)
    for j in (-7, -1, 1, 9):
        q = ref.quantize(x * F32(2.0 ** j))
        assert q.g == base.g * F32(2.0 ** j)
        assert np.array_equal(q.codes, base.codes) and np.array_equal(q.scales, base.scales)


def check_permutation(ref):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((3, 64)).astype(F32)
    base = ref.quantize(x)
    perm = rng.permutation(16)
    y = x.reshape(3, 4, 16)[:, :, perm].reshape(3, 64)
    q = ref.quantize(y)
    assert np.array_equal(q.scales, base.scales)
    want = ref.unpack_codes(base.codes).reshape(3, 4, 16)[:, :, perm].reshape(3, 64)
    assert np.array_equal(ref.unpack_codes(q.codes), want)


def check_negation(ref):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((5, 96)).astype(F32)
    x[0, :16] = 0.0
    x[1, 3] = 1e-9
    base = ref.quantize(x, g_mode="given", g=0.01)
    q = ref.quantize(-x, g_mode="given", g=0.01)
    assert np.array_equal(q.scales, base.scales)
    assert np.array_equal(ref.unpack_codes(q.codes), ref.unpack_codes(base.codes) ^ 8)


def check_zero_block(ref):
    x = np.zeros((2, 48), F32)
    x[0, 16:32] = [0, -0.0] * 8
    x[1, 32:48] = np.float32(2.0 ** -30) * np.arange(-8, 8, dtype=F32)
    x[1, 0] = 3.0
    q = ref.quantize(x)
    nib = ref.unpack_codes(q.codes)
    assert q.scales[0, 1] == 0 and list(nib[0, 16:32]) == [0, 8] * 8
    assert q.scales[1, 2] == 0
    assert list(nib[1, 32:48]) == [8] * 8 + [0] * 8
    z = ref.quantize(np.zeros((3, 32), F32))
    assert z.g == F32(1.0) and not z.scales.any() and not z.codes.any()


def check_dequant_error_bound(ref):
    """Dequantized values lie within half an E2M1 step (times S*g) of the input where the code is not saturated."""
    rng = np.random.default_rng(16)
    x = (rng.standard_t(3, size=(32, 256)) * 3).astype(F32)
    q = ref.quantize(x)
    xh = ref.dequantize(q)
    nib = ref.unpack_codes(q.codes)
    S = np.repeat(np.array([[float(E4M3[int(b)]) for b in row] for row in q.scales]), 16, axis=1)
    mags = np.array([float(E2M1[c & 7]) for c in range(16)])[nib]
    step = np.where(mags < 2, 0.5, np.where(mags < 4, 1.0, 2.0))
    unit = S * float(q.g)
    err = np.abs(x.astype(np.float64) - xh)
    sat = np.abs(x.astype(np.float64)) > 6.0 * unit * (1 + 1e-6)
    ok = err <= 0.5 * step * unit * (1 + 1e-5) + np.abs(x) * 1e-6
    assert np.all(ok | sat), np.argwhere(~(ok | sat))[:5]
    # sign agreement and magnitude never above 6*S*g
    assert np.all(np.abs(xh) <= 6.0 * unit + 0)
    nz = xh != 0
    assert np.all(np.sign(xh[nz]) == np.sign(x[nz]))


def check_byte_counts(ref):
    q = ref.quantize(np.ones((48, 1024), F32))
    assert q.codes.shape == (48, 512) and q.scales.shape == (48, 64)
    assert (q.codes.nbytes + q.scales.nbytes) * 8 == 4.5 * 48 * 1024


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------


def _exact_dequant(codes, scales, g):
    """Fraction-valued dequantization from the independent value sets."""
    rows, half = codes.shape
    out = []
    gf = Fraction(float(g))
    for r in range(rows):
        row = []
        for j in range(half * 2):
            byte = int(codes[r, j // 2])
            c = (byte >> 4) if j % 2 else (byte & 15)
            v = E2M1[c & 7] * (-1 if c & 8 else 1)
            row.append(v * E4M3[int(scales[r, j // 16])] * gf)
        out.append(row)
    return out


def check_gemm_bruteforce(ref):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 48)).astype(F32)
    w1 = (rng.standard_normal((4, 48)) * 0.3).astype(F32)
    w2 = (rng.standard_normal((2, 48)) * 7).astype(F32)
    xq, q1, q2 = ref.quantize(x), ref.quantize(w1), ref.quantize(w2)
    y, a = ref.gemm(xq, [q1, q2])
    assert y.shape == (3, 6)
    X = _exact_dequant(xq.codes, xq.scales, xq.g)
    W = _exact_dequant(q1.codes, q1.scales, q1.g) + _exact_dequant(q2.codes, q2.scales, q2.g)
    for m in range(3):
        for n in range(6):
            exact = sum(X[m][k] * W[n][k] for k in range(48))
            absum = sum(abs(X[m][k] * W[n][k]) for k in range(48))
            assert abs(y[m, n] - float(exact)) <= 1e-13 * float(absum) + 1e-300, (m, n)
            assert abs(a[m, n] - float(absum)) <= 1e-13 * float(absum)


def check_gemm_dequantized_bruteforce(ref):
    """The product on already dequantized operands (what the full-size parity checks call) against the exact
    rational triple loop, on non-square operands with mixed signs and module scales."""
    rng = np.random.default_rng(25)
    x = (rng.standard_normal((5, 64)) * np.exp(rng.uniform(-2, 2, (5, 64)))).astype(F32)
    w = (rng.standard_normal((3, 64)) * 0.05).astype(F32)
    xq, wq = ref.quantize(x), ref.quantize(w)
    y, a = ref.gemm_dequantized(ref.dequantize(xq), ref.dequantize(wq))
    assert y.shape == (5, 3) and a.shape == (5, 3)
    X = _exact_dequant(xq.codes, xq.scales, xq.g)
    W = _exact_dequant(wq.codes, wq.scales, wq.g)
    for m in range(5):
        for n in range(3):
            exact = sum(X[m][k] * W[n][k] for k in range(64))
            absum = sum(abs(X[m][k] * W[n][k]) for k in range(64))
            assert abs(y[m, n] - float(exact)) <= 1e-13 * float(absum) + 1e-300, (m, n)
            assert abs(a[m, n] - float(absum)) <= 1e-13 * float(absum), (m, n)


def check_gemm_constant(ref):
    """Constant operands: every block is full-range (code 6, scale 448), so Y = K * x^ * w^.

    With amax = 2688 * 2^-j the global scale is exactly 2^-j and the dequantized
    constants reproduce the inputs exactly, so Y is exact; otherwise it holds to FP64 rounding.
    """
    K = 1024
    xq = ref.quantize(np.full((5, K), 168.0, F32))        # 2688 * 2^-4
    wq = ref.quantize(np.full((3, K), -5.25, F32))        # -2688 * 2^-9
    assert np.all(ref.unpack_codes(xq.codes) == 7) and np.all(xq.scales == 0x7E)
    assert np.all(ref.unpack_codes(wq.codes) == 0xF) and np.all(wq.scales == 0x7E)
    assert np.all(ref.dequantize(xq) == 168.0) and np.all(ref.dequantize(wq) == -5.25)
    y, a = ref.gemm(xq, [wq])
    assert np.all(y == -K * 168.0 * 5.25) and np.all(a == K * 168.0 * 5.25)
    xq = ref.quantize(np.full((5, K), 0.7, F32))
    wq = ref.quantize(np.full((3, K), -1.3, F32))
    xh, wh = ref.dequantize(xq), ref.dequantize(wq)
    assert len(np.unique(xh)) == 1 and len(np.unique(wh)) == 1
    y, _ = ref.gemm(xq, [wq])
    assert np.allclose(y, K * xh[0, 0] * wh[0, 0], rtol=1e-14, atol=0)
    assert abs(xh[0, 0] - 0.7) < 1e-6 and abs(wh[0, 0] + 1.3) < 1e-6


def check_gemm_onehot(ref):
    K = 256
    x = np.zeros((4, K), F32)
    w = np.zeros((3, K), F32)
    x[np.arange(4), [5, 77, 130, 255]] = [1.5, -2.0, 3.0, 0.75]
    w[np.arange(3), [5, 130, 200]] = [4.0, -0.5, 9.0]
    xq, wq = ref.quantize(x), ref.quantize(w)
    xh, wh = ref.dequantize(xq), ref.dequantize(wq)
    y, _ = ref.gemm(xq, [wq])
    want = np.zeros((4, 3))
    want[0, 0] = xh[0, 5] * wh[0, 5]
    want[2, 1] = xh[2, 130] * wh[1, 130]
    assert np.array_equal(y, want), (y, want)


def check_gemm_identity(ref):
    K = 64
    rng = np.random.default_rng(22)
    xq = ref.quantize(rng.standard_normal((7, K)).astype(F32))
    wq = ref.quantize(np.eye(K, dtype=F32))
    y, _ = ref.gemm(xq, [wq])
    c = ref.dequantize(wq)[0, 0]
    assert abs(c - 1.0) < 1e-6
    assert np.allclose(y, ref.dequantize(xq) * c, rtol=1e-15, atol=0)


def check_fused_concat(ref):
    rng = np.random.default_rng(23)
    x = rng.standard_normal((6, 128)).astype(F32)
    mods = [rng.standard_normal((r, 128)).astype(F32) * s for r, s in [(5, 0.02), (3, 0.2), (2, 0.002)]]
    xq = ref.quantize(x)
    wq = [ref.quantize(m) for m in mods]
    y, _ = ref.gemm(xq, wq)
    a = ref.gemm(xq, wq)[1]
    parts = [ref.gemm(xq, [w])[0] for w in wq]
    assert np.all(np.abs(y - np.concatenate(parts, axis=1)) <= 1e-14 * a)
    assert len({float(w.g) for w in wq}) == 3


def check_fused_pitfall(ref):
    """One shared global scale over stacked modules changes the small module's scales (the serving pitfall)."""
    rng = np.random.default_rng(24)
    big = (rng.standard_normal((16, 256)) * 0.2).astype(F32)
    small = (rng.standard_normal((4, 256)) * 0.002).astype(F32)
    own = ref.quantize(small)
    shared = ref.quantize(np.concatenate([big, small]))
    assert not np.array_equal(shared.scales[16:], own.scales)
    x = ref.quantize(rng.standard_normal((3, 256)).astype(F32))
    y_own, _ = ref.gemm(x, [ref.quantize(big), own])
    wrong = ref.Quantized(own.codes, own.scales, ref.quantize(big).g)
    y_wrong, _ = ref.gemm(x, [ref.quantize(big), wrong])
    assert np.array_equal(y_own[:, :16], y_wrong[:, :16])
    assert not np.allclose(y_own[:, 16:], y_wrong[:, 16:], rtol=1e-3)


def check_tolerance_fn(ref):
    y = np.array([[1.0, -2.0, 0.0]])
    a = np.array([[10.0, 4.0, 0.0]])
    assert ref.gemm_within_tolerance(y, y, a)[0]
    assert ref.gemm_within_tolerance(y + [[9e-5, 0, 0]], y, a)[0]
    assert not ref.gemm_within_tolerance(y + [[1.1e-4, 0, 0]], y, a)[0]
    assert not ref.gemm_within_tolerance(y + [[0, 0, 1e-30]], y, a)[0]


def check_transpose_columns(ref):
    """The encoding of x^T, column by column: output row c is the row quantizer applied to column c of x
    with the whole tensor's g (amax over every element, whatever the orientation)."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((48, 7)) * np.exp(rng.uniform(-3, 3, (48, 7)))).astype(F32)
    x[17, 3] = F32(-40.0)
    qt = ref.quantize_t(x)
    assert qt.codes.shape == (7, 24) and qt.scales.shape == (7, 3)
    assert F32(qt.g).tobytes() == ref.global_scale(F32(40.0)).tobytes()
    for c in range(7):
        col = ref.quantize(x[:, c][None, :], "given", qt.g)
        assert np.array_equal(col.codes[0], qt.codes[c]) and np.array_equal(col.scales[0], qt.scales[c])


def _grid_matrix(rng, rows, cols, scale):
    """Values on the E2M1 grid times one power of two, with a +-6 in every run of 16 along either axis
    (so every block in both orientations has amax 6 * scale and encodes exactly with g = 1)."""
    mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    v = mags[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    r, c = np.indices((rows, cols))
    v = np.where((r + c) % 16 == 0, 6.0 * np.sign(v + 0.1), v)
    return (v * scale).astype(F32)


def check_transpose_exact(ref):
    """Exactly representable input: dequantizing the x^T encoding gives x^T itself; a transposed block axis
    or a transposed layout would not."""
    rng = np.random.default_rng(32)
    x = _grid_matrix(rng, 32, 48, 0.25)
    back = ref.dequantize(ref.quantize_t(x, "given", 1.0))
    assert back.shape == (48, 32) and np.array_equal(back, x.T.astype(np.float64))
    x[3, 5] = F32(0.3)                      # off the grid: one element of column 5 changes
    q = ref.quantize_t(x, "given", 1.0)
    diff = np.argwhere(ref.dequantize(q) != x.T.astype(np.float64))
    assert len(diff) >= 1 and np.all(diff[:, 0] == 5) and np.all(diff[:, 1] < 16)


def check_backward_products(ref):
    """The backward products from quantize / quantize_t compositions on exactly representable operands:
    dX = dY . W and dW = dY^T . X are exact small dyadic results."""
    rng = np.random.default_rng(33)
    M, N, K = 32, 48, 64
    dy, w, x = _grid_matrix(rng, M, N, 1.0), _grid_matrix(rng, N, K, 0.5), _grid_matrix(rng, M, K, 2.0)
    dx, _ = ref.gemm(ref.quantize(dy, "given", 1.0), [ref.quantize_t(w, "given", 1.0)])
    assert np.array_equal(dx, dy.astype(np.float64) @ w.astype(np.float64))
    dw, _ = ref.gemm(ref.quantize_t(dy, "given", 1.0), [ref.quantize_t(x, "given", 1.0)])
    assert np.array_equal(dw, dy.T.astype(np.float64) @ x.astype(np.float64))


ALL_CHECKS = [
    check_e2m1_values, check_e4m3_values, check_roundtrip, check_e4m3_bruteforce, check_e2m1_bruteforce,
    check_e2m1_thresholds, check_global_scale, check_golden_given, check_golden_computed, check_golden_op_order, check_amax_block,
    check_outlier_locality, check_dynamic_g_outlier, check_pow2_equivariance, check_permutation,
    check_negation, check_zero_block, check_dequant_error_bound, check_byte_counts,
    check_gemm_bruteforce, check_gemm_dequantized_bruteforce, check_gemm_constant, check_gemm_onehot, check_gemm_identity,
    check_fused_concat, check_fused_pitfall, check_tolerance_fn,
    check_transpose_columns, check_transpose_exact, check_backward_products,
]
