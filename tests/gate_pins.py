"""Pins for the gate-epilogue oracle (``oracle.gdn_gates``): closed forms, identities
and invariants of softplus, the sigmoid and the decay, each checked against an
expression the oracle does not use.  Every ``check_*`` raises AssertionError when the
given module disagrees."""
from __future__ import annotations

import numpy as np

LN2 = 0.6931471805599453


def check_softplus(g):
    assert abs(g.softplus(0.0) - LN2) < 1e-15
    for x in (0.5, 1.0, 3.0, 7.25):                       # softplus(log(e^x - 1)) = x
        assert abs(g.softplus(np.log(np.expm1(x))) - x) < 1e-12 * max(1.0, x)
    z = np.linspace(-30, 30, 601)
    assert np.allclose(g.softplus(z) - g.softplus(-z), z, rtol=0, atol=1e-12)
    assert abs(g.softplus(40.0) - 40.0) < 1e-15 * 40
    assert abs(g.softplus(-40.0) / np.exp(-40.0) - 1.0) < 1e-12
    with np.errstate(over="raise"):
        assert g.softplus(800.0) == 800.0 and g.softplus(-800.0) == 0.0


def check_sigmoid(g):
    assert g.sigmoid(0.0) == 0.5
    assert abs(g.sigmoid(np.log(3.0)) - 0.75) < 1e-15
    z = np.linspace(-10, 10, 801)                          # (1 + tanh cancels badly further out)
    assert np.allclose(g.sigmoid(z), 0.5 * (1.0 + np.tanh(z / 2.0)), rtol=1e-10, atol=0)
    z = np.linspace(-40, 40, 801)
    assert np.allclose(g.sigmoid(z) * (1.0 + np.exp(-z)), 1.0, rtol=1e-14, atol=0)
    assert np.allclose(g.sigmoid(-z), 1.0 - g.sigmoid(z), rtol=0, atol=1e-15)
    with np.errstate(over="raise"):
        assert g.sigmoid(-800.0) == 0.0 and g.sigmoid(800.0) == 1.0


def check_decay(g):
    assert abs(g.decay(0.0, 0.0, 0.0) - 0.5) < 1e-15              # exp(-ln 2)
    assert abs(g.decay(0.0, LN2, 0.0) - 0.25) < 1e-15             # exp(-2 ln 2)
    assert abs(g.decay(-1.5, 0.0, 1.5) - 0.5) < 1e-15             # the bias adds to a
    rng = np.random.default_rng(21)
    a = rng.uniform(-20, 20, 400)
    A = rng.uniform(-3, 3, 400)
    b = rng.uniform(-5, 5, 400)
    power = (1.0 + np.exp(a + b)) ** (-np.exp(A))                # exp(-c log(1 + e^z)) = (1 + e^z)^(-c)
    assert np.allclose(g.decay(a, A, b), power, rtol=1e-11, atol=1e-300)
    d = g.decay(np.linspace(-10, 10, 201), 0.3, 0.1)
    assert np.all(d > 0) and np.all(d <= 1) and np.all(np.diff(d) < 0)   # in (0, 1], decreasing in a
    assert g.decay(1.0, 0.5, 0.0) < g.decay(1.0, 0.0, 0.0)                # decreasing in A
    assert abs(g.decay(-60.0, 0.0, 0.0) - 1.0) < 1e-20                    # a -> -inf: no decay


def check_apply_gates(g):
    rng = np.random.default_rng(22)
    y = rng.standard_normal((5, 30))
    A = rng.uniform(-1, 2, 4)
    bias = rng.uniform(-2, 1, 4)
    out = g.apply_gates(y, 20, 4, 24, 4, A, bias)
    keep = np.r_[0:20, 28:30]
    assert np.array_equal(out[:, keep], y[:, keep])                        # other columns untouched
    for h in range(4):                                                     # head h of each gate
        assert np.allclose(out[:, 20 + h], (1.0 + np.exp(y[:, 20 + h] + bias[h])) ** (-np.exp(A[h])), rtol=1e-12)
        assert np.allclose(out[:, 24 + h], 0.5 * (1.0 + np.tanh(y[:, 24 + h] / 2.0)), rtol=1e-12)
    perm = np.array([2, 0, 3, 1])                                          # heads carry their own A, bias
    y2 = y.copy()
    y2[:, 20:24] = y[:, 20:24][:, perm]
    out2 = g.apply_gates(y2, 20, 4, 24, 4, A[perm], bias[perm])
    assert np.allclose(out2[:, 20:24], out[:, 20:24][:, perm], rtol=1e-15)


def check_tolerance(g):
    rng = np.random.default_rng(23)
    y = rng.uniform(-12, 12, (64, 12))
    a_ref = np.abs(y) * 3.0 + 1.0
    A = rng.uniform(-2, 3, 4)
    bias = rng.uniform(-3, 2, 4)
    tol = g.gates_tolerance(y, a_ref, 4, 4, 8, 4, A, bias)
    assert np.all(tol > 0)
    rt = g.ref.GEMM_RTOL
    assert np.array_equal(tol[:, :4], rt * a_ref[:, :4])                   # ungated: the product's bound
    dy = rt * a_ref                                                        # the product's worst error, either side
    for sgn in (1.0, -1.0):
        moved = g.apply_gates(y + sgn * dy, 4, 4, 8, 4, A, bias) - g.apply_gates(y, 4, 4, 8, 4, A, bias)
        assert np.all(np.abs(moved[:, 4:12]) <= tol[:, 4:12])
    tight = g.gates_tolerance(y, a_ref * 0, 4, 4, 8, 4, A, bias)           # with an exact product only
    out = g.apply_gates(y, 4, 4, 8, 4, A, bias)                            # the FP32 evaluation remains
    assert np.all(tight[:, 4:12] <= 1e-5 * (1.0 + np.abs(out[:, 4:12]) * 60.0) + 1e-30)


def check_within(g):
    """The comparison the GPU gate tests call: inside the bound passes, beyond it fails, and the worst
    ratio is |diff| / tol (dyadic values, so every difference is exact)."""
    e = 2.0 ** -20
    ref_out = np.array([[0.5, 0.25, 1.0]])
    tol = np.array([[e, 2 * e, 4 * e]])
    ok, worst = g.within(ref_out + [[e, -e, 0.0]], ref_out, tol)
    assert ok and worst == 1.0
    assert not g.within(ref_out + [[0.0, 0.0, 8 * e]], ref_out, tol)[0]
    ok, worst = g.within(ref_out, ref_out, tol)
    assert ok and worst == 0.0

ALL_CHECKS = [check_softplus, check_sigmoid, check_decay, check_apply_gates, check_tolerance, check_within]
