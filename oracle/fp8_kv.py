"""CPU oracle for the FP8 (E4M3) KV-cache quantizer with a calibrated per-tensor scale.

TEST INFRASTRUCTURE ONLY.  Like ``nvfp4_ref``, only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module; the product path never
does, and this module imports nothing from the product package.

What it follows: "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent
Half of a Hybrid 27B LLM", summary: calibrated FP8 scales applied to the KV cache recover most
of the long-context loss.  The page names nothing finer, so these are readings:

* FP8 is E4M3 "FN" (bias 7, largest value 448, no infinities), the same byte format as the
  NVFP4 block scales; one FP32 scale s per tensor (a layer's K or V cache).
* A calibrated scale is given by the caller; the computed mode calibrates on the tensor itself,
  s = fl32(amax / 448) (1 for an all-zero tensor, floored at 2^-100), so the largest element
  lands on 448.
* Per element, as in the NVFP4 element step: r = fl32(1 / s), q = fl32(x * r), byte = sign of q
  in bit 7 and the E4M3 magnitude nearest to |q| (ties to even, saturating at 448); the sign is
  kept when the magnitude rounds to 0; a NaN input gives 0x7F with its sign.
* Dequantized value: e4m3(byte) * s.
"""
from __future__ import annotations

import numpy as np

from oracle import nvfp4_ref as ref

F32 = np.float32
KV_RANGE = 448.0
S_FLOOR = F32(2.0 ** -100)


def kv_scale(amax: float) -> np.float32:
    """Calibrated scale from a largest magnitude: fl32(amax / 448), 1 for 0, floored at 2^-100."""
    amax = F32(amax)
    if amax == F32(0.0):
        return F32(1.0)
    return max(F32(amax / F32(KV_RANGE)), S_FLOOR)


def quantize_kv(x: np.ndarray, s_mode: str = "compute", s: float | None = None) -> tuple[np.ndarray, np.float32]:
    """FP8 bytes [rows, cols] (uint8) and the scale used."""
    v = np.asarray(x, dtype=F32)
    if s_mode == "compute":
        s32 = kv_scale(F32(np.max(np.abs(v))) if v.size else F32(0.0))
    elif s_mode == "given":
        s32 = F32(s)
        if not (np.isfinite(s32) and s32 > 0):
            raise ValueError("a given scale must be finite and positive")
    else:
        raise ValueError(s_mode)
    r = F32(1.0) / s32
    q = (v * r).astype(F32)
    mag = np.abs(q)
    nan = np.isnan(q)
    code = ref.e4m3_encode(np.where(nan, F32(0.0), mag).astype(F32)).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    sign = (np.signbit(q).astype(np.uint8) << 7).astype(np.uint8)
    return (code | sign).astype(np.uint8), s32


_E4M3_SIGNED = np.array([(-1.0 if b & 0x80 else 1.0) * (ref.E4M3_VALS[b & 0x7F] if (b & 0x7F) < 0x7F else np.nan)
                         for b in range(256)], dtype=np.float64)


def dequantize_kv(codes: np.ndarray, s: float) -> np.ndarray:
    """FP64 values e4m3(byte) * s."""
    return _E4M3_SIGNED[np.asarray(codes, np.uint8)] * np.float64(F32(s))
