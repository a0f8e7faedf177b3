"""CPU oracle for NVFP4 quantization behind a randomized Hadamard transform (RHT).

TEST INFRASTRUCTURE ONLY.  Like ``nvfp4_ref``, only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module; the product path never
does, and this module imports nothing from the product package.

What it follows: "Normalized Architectures are Natively 4-Bit", sections "Problem" and
"Approach" and the baselines list: standard transformers trained in NVFP4 need random
Hadamard transforms (with per-tensor scaling) before quantization, which nGPT does without.
The pages give no further detail, so the following are readings:

* The transform acts on each 16-element block along the quantization axis (the same
  blocks that get one E4M3 scale): v -> H16 . D . v / 4, where D = diag(+-1) is a random
  sign vector shared by every block of the tensor and by both operands of a product, and
  H16 is the 16 x 16 Hadamard matrix in natural (Sylvester) order.  H16 . H16 = 16 I, so
  the transform is orthogonal and (T x) . (T w) = x . w: a product of two transformed
  operands needs no change.
* The random signs are an input (a 16-bit mask, bit i negating element i of every block).
* FP32 arithmetic in a fixed order, because codes are bit-exact: the signs by negation
  (exact), then the butterfly stages h = 1, 2, 4, 8, each replacing the pair (i, i + h),
  i & h == 0, by (a + b, a - b) with one rounding per operation, then the product by 1/4
  (exact except below the normal range).
* The global scale is computed from the amax of the transformed tensor (the quantizer
  sees only transformed values).
"""
from __future__ import annotations

import numpy as np

from oracle import nvfp4_ref as ref

F32 = np.float32
STAGES = (1, 2, 4, 8)


def sign_vector(signs: int) -> np.ndarray:
    """+1 / -1 per block position from the 16-bit mask (bit i set: element i negated)."""
    if not 0 <= int(signs) < 1 << 16:
        raise ValueError("signs is a 16-bit mask")
    return np.array([-1.0 if (int(signs) >> i) & 1 else 1.0 for i in range(16)], F32)


def rht_blocks(x: np.ndarray, signs: int) -> np.ndarray:
    """The transform of every 16-element block along the last axis of a 2-D FP32 array."""
    v = np.asarray(x, F32)
    rows, K = v.shape
    if K % 16:
        raise ValueError("the transformed axis must be a multiple of 16")
    b = (v.reshape(rows, K // 16, 16) * sign_vector(signs)).astype(F32)   # negation: exact
    for h in STAGES:
        out = b.copy()
        for i in range(16):
            if i & h:
                continue
            a, c = b[:, :, i], b[:, :, i + h]
            out[:, :, i] = (a + c).astype(F32)
            out[:, :, i + h] = (a - c).astype(F32)
        b = out
    return (b * F32(0.25)).astype(F32).reshape(rows, K)


def quantize_rht(x: np.ndarray, signs: int, g_mode: str = "compute", g: float | None = None) -> ref.Quantized:
    """NVFP4 quantization (blocks along the last axis) of the transformed tensor."""
    return ref.quantize(rht_blocks(x, signs), g_mode, g)


def quantize_t_rht(x: np.ndarray, signs: int, g_mode: str = "compute", g: float | None = None) -> ref.Quantized:
    """The same for x^T (blocks of 16 consecutive rows of x), as the backward products use it."""
    return quantize_rht(np.ascontiguousarray(np.asarray(x, F32).T), signs, g_mode, g)
