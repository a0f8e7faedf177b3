"""CPU oracle for the Gated DeltaNet gate epilogue of the fused input projection.

TEST INFRASTRUCTURE ONLY.  Like ``nvfp4_ref``, only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module; the product path never
does, and this module imports nothing from the product package.

What it follows: the anthology-of-the-sota record theory-128 (Kozyrev and Maiboroda,
2026), section "The account", its paragraph on how the gates are parameterized: the
state decay is exp(-exp(A) * softplus(a + b)) and the write strength is a sigmoid.  The a and b of that section are the outputs of two small
projections that sit in the same fused input projection as q, k, v and z (section
"Critical Lessons for Model Serving": fused modules, each with its own global scale).

Readings (the page is terse and its extraction is garbled around the formula):

* Inside the softplus, "a + b" is the decay projection's output a plus a learned
  per-head bias (the usual dt bias of gated linear recurrences), not the write-strength
  projection's output; the write strength is sigmoid of that second projection.
* A is a learned per-head parameter entering through exp(A), so the decay lies in (0, 1].
* One gate per output column: head h of the decay projection is its column h, and the
  same for the write strength.  All other columns of the fused output pass unchanged.

Everything is computed in FP64 with the numerically stable forms of softplus and the
sigmoid; the tolerance below bounds how far a correct FP32 implementation may land.
"""
from __future__ import annotations

import numpy as np

from oracle import nvfp4_ref as ref


def softplus(z: np.ndarray) -> np.ndarray:
    """log(1 + exp(z)), evaluated without overflow: z + log1p(exp(-z)) for z > 0."""
    z = np.asarray(z, np.float64)
    return np.where(z > 0, z + np.log1p(np.exp(-np.abs(z))), np.log1p(np.exp(np.minimum(z, 0.0))))


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)), evaluated without overflow on either side."""
    z = np.asarray(z, np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def decay(a: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """exp(-exp(A) * softplus(a + bias)) per head (A = a_log, broadcast over tokens)."""
    return np.exp(-np.exp(np.asarray(a_log, np.float64)) * softplus(np.asarray(a, np.float64) + dt_bias))


def apply_gates(y: np.ndarray, a_col: int, n_a: int, b_col: int, n_b: int, a_log: np.ndarray,
                dt_bias: np.ndarray) -> np.ndarray:
    """The fused projection's output with its decay columns [a_col, a_col + n_a) turned into
    decays and its write-strength columns [b_col, b_col + n_b) into sigmoids (FP64 copy)."""
    out = np.array(y, np.float64, copy=True)
    out[:, a_col:a_col + n_a] = decay(out[:, a_col:a_col + n_a], a_log, dt_bias)
    out[:, b_col:b_col + n_b] = sigmoid(out[:, b_col:b_col + n_b])
    return out


# FP32 evaluation error allowed per gate, in units of the output: a few roundings of
# exp / log1p / the sigmoid, scaled for the decay by the size of its exponent.
EVAL_ULPS = 8.0 * 2.0 ** -24


def gates_tolerance(y_ref: np.ndarray, a_ref: np.ndarray, a_col: int, n_a: int, b_col: int, n_b: int,
                    a_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """Per-element bound for |out_gpu - out_ref|.

    Ungated columns: the product's own bound, rtol * sum|terms|.  Gated columns: that
    bound carried through the gate's derivative (twice, for its change across the
    interval), plus the FP32 evaluation of the gate itself.  For the decay
    d alpha / d a = -alpha * exp(A) * sigmoid(a + bias) and the FP32 evaluation is
    relative to the exponent X = exp(A) * softplus(a + bias); for the sigmoid
    d beta / d b = beta * (1 - beta).
    """
    y_ref = np.asarray(y_ref, np.float64)
    dy = ref.GEMM_RTOL * np.asarray(a_ref, np.float64)
    tol = dy.copy()
    ya = y_ref[:, a_col:a_col + n_a]
    c = np.exp(np.asarray(a_log, np.float64))
    alpha = decay(ya, a_log, dt_bias)
    x_exp = c * softplus(ya + dt_bias)
    tol[:, a_col:a_col + n_a] = (2.0 * alpha * c * sigmoid(ya + dt_bias) * dy[:, a_col:a_col + n_a]
                                 + EVAL_ULPS * (1.0 + x_exp) * alpha + 1e-37)
    yb = y_ref[:, b_col:b_col + n_b]
    beta = sigmoid(yb)
    tol[:, b_col:b_col + n_b] = 2.0 * beta * (1.0 - beta) * dy[:, b_col:b_col + n_b] + EVAL_ULPS * beta + 1e-37
    return tol


def within(out_gpu: np.ndarray, out_ref: np.ndarray, tol: np.ndarray) -> tuple[bool, float]:
    """(all |out_gpu - out_ref| <= tol, worst |diff| / tol)."""
    err = np.abs(np.asarray(out_gpu, np.float64) - out_ref)
    ratio = err / tol
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(worst <= 1.0), worst
