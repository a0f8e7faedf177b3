"""Pins of the RHT oracle (``oracle/rht.py``) against what the mathematics fixes independently of it:
the Hadamard matrix built by Kronecker products, orthogonality (dot products and the inverse), a
hand-worked FP32 rounding fixture, closed-form global scale and codes of a one-hot block, and the
column-by-column definition of the transposed encoding.  Each check takes the module under test."""
import os

import numpy as np

from oracle import nvfp4_ref as ref

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rht_rounding_order.txt")


def hadamard16() -> np.ndarray:
    """H16 in natural (Sylvester) order: H2 (x) H2 (x) H2 (x) H2, entries +-1 (FP64)."""
    h2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    h = h2
    for _ in range(3):
        h = np.kron(h, h2)
    return h


def _int_matrix(seed, rows, cols, lo=-8, hi=8):
    return np.random.default_rng(seed).integers(lo, hi + 1, (rows, cols)).astype(F32)


def check_sign_vector(o):
    assert np.array_equal(o.sign_vector(0), np.ones(16, F32))
    s = o.sign_vector(0b101)
    assert list(s[:4]) == [-1.0, 1.0, -1.0, 1.0] and np.all(s[4:] == 1.0)
    assert o.sign_vector(0x8000)[15] == -1.0 and np.all(o.sign_vector(0x8000)[:15] == 1.0)
    try:
        o.sign_vector(1 << 16)
    except ValueError:
        pass
    else:
        raise AssertionError("a 17-bit mask must be rejected")


def check_matrix(o):
    """Small integers transform exactly: each block equals H16 . D . v / 4 computed in FP64."""
    h = hadamard16()
    x = _int_matrix(41, 3, 48)
    for signs in (0, 0x0001, 0xA5C3, 0xFFFF, 0x7001):
        d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
        want = np.stack([(h @ (d[:, None] * x[:, 16 * j:16 * j + 16].astype(np.float64).T)).T / 4.0
                         for j in range(3)], axis=1)
        got = o.rht_blocks(x, signs).astype(np.float64).reshape(3, 3, 16)
        assert np.array_equal(got, want), signs


def check_orthogonal(o):
    """The transform keeps dot products (so a product of transformed operands needs no change) and is
    undone by D . H16^T / 4."""
    h = hadamard16()
    x, w = _int_matrix(42, 5, 64), _int_matrix(43, 7, 64)
    for signs in (0, 0x3C5A):
        tx, tw = o.rht_blocks(x, signs).astype(np.float64), o.rht_blocks(w, signs).astype(np.float64)
        assert np.array_equal(tx @ tw.T, x.astype(np.float64) @ w.astype(np.float64).T)
        d = np.array([-1.0 if (signs >> i) & 1 else 1.0 for i in range(16)])
        back = (d[:, None] * (h.T @ tx.reshape(5, 4, 16).transpose(2, 0, 1).reshape(16, -1)) / 4.0)
        assert np.array_equal(back.reshape(16, 5, 4).transpose(1, 2, 0).reshape(5, 64), x.astype(np.float64))


def load_golden():
    cases, cur = {}, None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (t.strip() for t in line.split(":", 1))
            if key == "case":
                cur = cases.setdefault(val, {})
            elif key == "signs":
                cur["signs"] = int(val, 16)
            else:
                cur[key] = np.array([float(t) for t in val.split()], F32)
    return cases


def check_golden(o):
    """FP32 rounding order and sign placement, hand-worked in tests/golden/rht_rounding_order.txt."""
    cases = load_golden()
    assert set(cases) == {"order", "signs"}
    for name, c in cases.items():
        got = o.rht_blocks(c["x"][None, :], c["signs"])[0]
        assert np.array_equal(got, c["y"]), (name, got, c["y"])


def check_amax_and_codes(o):
    """A one-hot block of 2688 becomes sixteen entries of +-672 = 2688 / 4: the transformed amax gives
    g = 672 / 2688 = 1/4, every scale is 448 (0x7E) and every code magnitude 6 (0x7), with the sign of
    column p of H16 (times the sign of element p); an all-zero block keeps scale 0 and codes 0."""
    h = hadamard16()
    for p, signs in ((0, 0), (0, 1), (5, 0), (5, 0x0020), (11, 0x0F00)):
        x = np.zeros((2, 32), F32)
        x[0, p] = 2688.0
        q = o.quantize_rht(x, signs)
        assert F32(q.g) == F32(0.25), (p, signs, q.g)
        assert q.scales[0, 0] == 0x7E and q.scales[0, 1] == 0 and np.all(q.scales[1] == 0)
        sgn = h[:, p] * (-1.0 if (signs >> p) & 1 else 1.0)
        want = np.where(sgn > 0, 0x7, 0xF)
        nib = ref.unpack_codes(q.codes)
        assert np.array_equal(nib[0, :16], want), (p, signs)
        # zero blocks: magnitude 0 (negated zeros keep their sign through the butterflies: code 0x8)
        assert np.all(nib[0, 16:] & 7 == 0) and np.all(nib[1] & 7 == 0)


def check_transposed(o):
    """quantize_t_rht, column by column: output row c is quantize_rht of column c of x, with the whole
    (transformed) tensor's g."""
    rng = np.random.default_rng(44)
    x = rng.standard_normal((48, 5)).astype(F32)
    qt = o.quantize_t_rht(x, 0x1234)
    assert qt.codes.shape == (5, 24)
    full = o.quantize_rht(np.ascontiguousarray(x.T), 0x1234)
    assert F32(qt.g) == F32(full.g)
    for c in range(5):
        col = o.quantize_rht(np.ascontiguousarray(x[:, c][None, :]), 0x1234, "given", qt.g)
        assert np.array_equal(col.codes[0], qt.codes[c]) and np.array_equal(col.scales[0], qt.scales[c])


def check_quantized_product(o):
    """NVFP4 products of transformed operands approximate the untransformed product (the transform is
    orthogonal; only the 4-bit rounding remains)."""
    rng = np.random.default_rng(45)
    x = rng.standard_normal((64, 256)).astype(F32)
    w = rng.standard_normal((32, 256)).astype(F32)
    y, _ = ref.gemm(o.quantize_rht(x, 0xBEEF), [o.quantize_rht(w, 0xBEEF)])
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(y - exact) < 0.2 * np.linalg.norm(exact)
    y_wrong, _ = ref.gemm(o.quantize_rht(x, 0xBEEF), [o.quantize_rht(w, 0xBEEE)])   # mismatched signs
    assert np.linalg.norm(y_wrong - exact) > 0.5 * np.linalg.norm(exact)


ALL_CHECKS = [check_sign_vector, check_matrix, check_orthogonal, check_golden, check_amax_and_codes,
              check_transposed, check_quantized_product]
