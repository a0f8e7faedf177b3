"""CPU oracle for the NVFP4 W4A4 linear layer (quantize activations + block-scaled GEMM).

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the C-ABI
library and its Python binding) never imports, calls or links anything here, and
this module imports nothing from the product package.

What it follows (the pages are cited by title and section):

* "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent
  Half of a Hybrid 27B LLM", section "Why the 'Fragile' Recurrence is Actually
  Robust": NVFP4 scales small groups of 16 elements, which keeps an outlier's
  error inside its own group.  Section "Performance and Efficiency Gains": every
  linear layer runs with weights *and* activations in NVFP4 (W4A4).  Section
  "Critical Lessons for Model Serving": each module carries its own global
  scale; fusing modules into one kernel must not mix those scales.
* "Normalized Architectures are Natively 4-Bit" (summary page, sections
  "Problem" and "Approach"; abstract of arXiv 2605.06067): NVFP4 dot products,
  and per-tensor scaling as an optional step (``g_mode='given'`` with g = 1).

The NVFP4 number format itself (E2M1 element codes, E4M3 block scales, an FP32
per-tensor scale) is not spelled out on the pages; the encodings below are the
format's public definitions (E2M1: 1 sign, 2 exponent bits with bias 1, 1
mantissa bit; E4M3 "FN": 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
no infinities, max 448).  Every point the pages leave open is a stated reading,
marked "Reading:" where it is used.

Precision: every step that *decides* a code or a scale is carried out in IEEE
FP32 with round-to-nearest-even, one rounding per operation, in the order
written (numpy float32 ufuncs round each operation once and never fuse).  The
dequantized values and the GEMM are computed in FP64.  Codes and scales are
chosen by nearest-value search over explicit value tables, not by bit tricks.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# The two small formats, written out from their field definitions.
# ---------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.

    Exponent field 0 is the subnormal range (mantissa * 0.5); otherwise the value
    is 2**(e-1) * (1 + m/2).
    """
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e4m3_value(byte: int) -> float:
    """Value of an E4M3 ("FN" variant) byte: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.

    Exponent field 0 is subnormal (m/8 * 2**-6).  The two all-ones patterns
    (0x7F, 0xFF) are NaN; there are no infinities, so the largest finite value is
    0x7E = 1.75 * 2**8 = 448.
    """
    s = (byte >> 7) & 1
    e = (byte >> 3) & 15
    m = byte & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


#: magnitudes of E2M1 codes 0..7, ascending with the code
E2M1_MAGS = np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)
#: values of the 127 finite non-negative E4M3 bytes 0x00..0x7E, ascending with the byte
E4M3_VALS = np.array([e4m3_value(b) for b in range(127)], dtype=np.float64)

E2M1_MAX = 6.0      # largest E2M1 magnitude
E4M3_MAX = 448.0    # largest finite E4M3 value
#: Reading: the per-tensor scale maps the tensor amax onto the largest value an
#: element can reach, largest element code times largest block scale.
GLOBAL_RANGE = E2M1_MAX * E4M3_MAX  # 2688
#: Reading: floor on the computed global scale so that 1/g stays finite.
G_FLOOR = F32(2.0 ** -100)


def _nearest_code(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of the ascending ``table`` for each x >= 0.

    Ties pick the even index, which is the even code (round half to even).
    Values above the last entry return the last index (saturation).
    Distances are taken in FP64, where they are exact for the inputs used
    (FP32 values against short table entries).
    """
    xd = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(table, xd, side="left")          # table[hi-1] < x <= table[hi]
    hi = np.clip(hi, 1, len(table) - 1)
    lo = hi - 1
    d_lo = xd - table[lo]
    d_hi = table[hi] - xd
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(xd >= table[-1], len(table) - 1, idx)  # saturate
    idx = np.where(xd <= table[0], 0, idx)
    return idx.astype(np.uint8)


def e4m3_encode(u: np.ndarray) -> np.ndarray:
    """Non-negative FP32 value -> E4M3 byte: nearest finite value, ties to even, saturating at 448.

    Reading: round-to-nearest-even with saturation (no NaN is ever produced);
    values below half the smallest subnormal (2**-10) round to 0, and 2**-10
    itself ties to the even byte 0x00.
    """
    return _nearest_code(np.asarray(u, dtype=F32), E4M3_VALS)


def e2m1_encode(q: np.ndarray) -> np.ndarray:
    """FP32 value -> 4-bit E2M1 code: sign from the sign bit, magnitude by nearest-even, saturating at 6.

    Reading: the sign bit is kept even when the magnitude rounds to 0, so a
    negative value that rounds to zero, or -0.0, is code 0x8.
    """
    q = np.asarray(q, dtype=F32)
    sign = np.signbit(q).astype(np.uint8) << 3
    return sign | _nearest_code(np.abs(q), E2M1_MAGS)


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------


def global_scale(amax: float) -> np.float32:
    """FP32 per-tensor scale g from the tensor's largest magnitude.

    Reading: g = fl32(amax / 2688), so the block holding the tensor amax gets
    the largest block scale (448) and its largest element the largest code (6).
    An all-zero tensor gets g = 1, and g is floored at 2**-100.
    """
    amax = F32(amax)
    if amax == F32(0.0):
        return F32(1.0)
    g = amax / F32(GLOBAL_RANGE)
    return max(g, G_FLOOR)


class Quantized:
    """An NVFP4 tensor in the canonical layout.

    codes  : uint8 [rows, K/2], byte j holds element 2j in its low nibble and 2j+1 in its high nibble
    scales : uint8 [rows, K/16], E4M3 scale of each 16-element block along K, row-major
    g      : FP32 per-tensor scale (dequantized value = e2m1(code) * e4m3(scale) * g)
    """

    def __init__(self, codes, scales, g, nibbles=None):
        self.codes = codes
        self.scales = scales
        self.g = F32(g)
        self.nibbles = nibbles  # uint8 [rows, K], one code per element (unpacked view)

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def encode_block_scale(bamax: np.ndarray, s_enc: np.float32) -> np.ndarray:
    """E4M3 block scale from the block's largest magnitude: S = e4m3(fl32(fl32(bamax * s_enc) / 6)).

    The block's largest element should land on the largest E2M1 magnitude (6)
    once divided by the decoded scale.
    """
    t = (np.asarray(bamax, F32) * F32(s_enc)).astype(F32)
    u = (t / F32(E2M1_MAX)).astype(F32)
    return e4m3_encode(u)


def block_reciprocal(S: np.ndarray, s_enc: np.float32) -> np.ndarray:
    """Per-block multiplier r = fl32(s_enc / e4m3(S)); 0 for a zero scale.

    Reading: elements are multiplied by this one reciprocal per block rather than
    divided one by one; a zero scale sends the whole block to signed zero.
    """
    S = np.asarray(S, np.uint8)
    S_val = E4M3_VALS[np.minimum(S, 126)].astype(F32)     # exact: E4M3 values fit FP32
    safe = np.where(S == 0, F32(1.0), S_val).astype(F32)
    r = (F32(s_enc) / safe).astype(F32)
    return np.where(S == 0, F32(0.0), r).astype(F32)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """uint8 [rows, K] codes -> uint8 [rows, K/2]: element 2j in the low nibble of byte j, 2j+1 in the high one."""
    nib = np.asarray(nib, np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def quantize(x: np.ndarray, g_mode: str = "compute", g: float | None = None) -> Quantized:
    """NVFP4-quantize a 2-D tensor [rows, K] along K (the contraction axis).

    Steps, in order:
      1. v = fp32(x)                         (bf16 inputs widen exactly)
      2. per tensor: amax = max|v|, g = global_scale(amax)   (g_mode='compute')
         or g = caller's value                              (g_mode='given')
      3. s_enc = fl32(1 / g)
      4. per 16-element block along K: bamax = max|v|, S = encode_block_scale(bamax, s_enc)
      5. r = block_reciprocal(S, s_enc)
      6. per element: q = fl32(v * r), code = e2m1_encode(q)
      7. pack two codes per byte, even element in the low nibble

    Reading: the block axis is K, the only axis along which a block scale factors
    out of a dot product; step 3 takes the reciprocal of the stored g so that both
    g modes share one definition.
    """
    v = np.ascontiguousarray(np.asarray(x, dtype=F32))
    if v.ndim != 2 or v.shape[1] % 16 != 0:
        raise ValueError("quantize expects a 2-D array whose second dimension is a multiple of 16")
    rows, K = v.shape
    if g_mode == "compute":
        amax = F32(np.max(np.abs(v))) if v.size else F32(0.0)
        g32 = global_scale(amax)
    elif g_mode == "given":
        g32 = F32(g)
        if not (np.isfinite(g32) and g32 > 0):
            raise ValueError("given g must be finite and positive")
    else:
        raise ValueError(g_mode)
    s_enc = F32(1.0) / g32

    blocks = v.reshape(rows, K // 16, 16)
    bamax = np.max(np.abs(blocks), axis=2) if v.size else np.zeros((rows, K // 16), F32)
    S = encode_block_scale(bamax, s_enc)
    r = block_reciprocal(S, s_enc)
    q = (blocks * r[:, :, None]).astype(F32)
    nib = e2m1_encode(q).reshape(rows, K)
    return Quantized(pack_nibbles(nib), S.astype(np.uint8), g32, nibbles=nib)


def quantize_t(x: np.ndarray, g_mode: str = "compute", g: float | None = None) -> Quantized:
    """NVFP4 encoding of x^T for x [rows, cols]: blocks of 16 consecutive rows of x.

    The backward products of end-to-end NVFP4 training ("Normalized Architectures are
    Natively 4-Bit", abstract and section "Approach") contract over the other axis of
    their operands (dX = dY . W over W's rows, dW = dY^T . X over the tokens), so each
    of those operands is quantized as its transpose.  Definition: ``quantize`` applied
    to x^T (the amax, hence g, does not depend on the orientation).
    """
    return quantize(np.ascontiguousarray(np.asarray(x, dtype=F32).T), g_mode, g)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [rows, K/2] -> one code per element [rows, K] (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


_E2M1_ALL = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3_ALL = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)


def dequantize(qt: Quantized) -> np.ndarray:
    """FP64 values e2m1(code) * e4m3(scale) * g (exact: each factor has a short mantissa)."""
    nib = unpack_codes(qt.codes)
    rows, K = nib.shape
    vals = _E2M1_ALL[nib].reshape(rows, K // 16, 16)
    sc = _E4M3_ALL[qt.scales][:, :, None]
    return (vals * sc).reshape(rows, K) * np.float64(qt.g)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------


def gemm(xq: Quantized, w_modules: list[Quantized]) -> tuple[np.ndarray, np.ndarray]:
    """Y = X^ . W^T in FP64 for one activation tensor and a stack of weight modules.

    ``w_modules`` are the sub-modules of one (possibly fused) projection, each
    quantized with its own global scale (section "Critical Lessons for Model
    Serving": modules calibrated individually keep their own scale when fused).
    Their output columns are concatenated in the given order.

    Reading: all sub-modules read one quantization of X (one g_x), since they
    share the same input.

    Returns (Y, A) where A[m, n] = sum_k |x^[m,k] * w^[n,k]|, the scale of the
    FP32 accumulation-order error used by the tolerance check.
    """
    xh = dequantize(xq)
    wh = np.concatenate([dequantize(w) for w in w_modules], axis=0)
    y = xh @ wh.T
    a = np.abs(xh) @ np.abs(wh).T
    return y, a


def gemm_dequantized(xh: np.ndarray, wh: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Same as ``gemm`` on already dequantized FP64 operands [M,K] and [N,K]."""
    return xh @ wh.T, np.abs(xh) @ np.abs(wh).T


#: Tolerance of a GEMM output against the FP64 oracle, relative to the sum of
#: |terms| of its dot product (FP32 accumulation-order error scale).
GEMM_RTOL = 1e-5


def gemm_within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray,
                          rtol: float = GEMM_RTOL) -> tuple[bool, float]:
    """|y_gpu - y_ref| <= rtol * A elementwise; returns (ok, worst ratio |dy| / A)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    denom = np.where(a_ref > 0, a_ref, 1.0)
    ratio = np.where(a_ref > 0, err / denom, np.where(err > 0, np.inf, 0.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(worst <= rtol), worst
