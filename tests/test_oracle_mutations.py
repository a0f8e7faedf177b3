"""Plants plausible mistakes in a private copy of the oracle (on the CPU) and checks
that at least one pin in ``oracle_pins`` fails for each of them.  This is the
evidence that the pins constrain every step of the oracle."""
import importlib.util
import os

import numpy as np
import pytest

import oracle_pins as pins

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "nvfp4_ref.py")
F32 = np.float32


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("nvfp4_ref_mutant", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _nearest_tie_mutant(tie_pick_hi):
    def nearest(x, table):
        xd = np.asarray(x, dtype=np.float64)
        hi = np.clip(np.searchsorted(table, xd, side="left"), 1, len(table) - 1)
        lo = hi - 1
        d_lo, d_hi = xd - table[lo], table[hi] - xd
        pick = (d_hi < d_lo) | ((d_hi == d_lo) & tie_pick_hi)
        idx = np.where(pick, hi, lo)
        idx = np.where(xd >= table[-1], len(table) - 1, idx)
        return np.where(xd <= table[0], 0, idx).astype(np.uint8)
    return nearest


def m_ties_away(o):
    o._nearest_code = _nearest_tie_mutant(True)


def m_ties_down(o):
    o._nearest_code = _nearest_tie_mutant(False)


def m_e2m1_truncate(o):
    def enc(q):
        q = np.asarray(q, F32)
        idx = np.searchsorted(o.E2M1_MAGS, np.abs(q).astype(np.float64), side="right") - 1
        return (np.signbit(q).astype(np.uint8) << 3) | idx.astype(np.uint8)
    o.e2m1_encode = enc


def m_no_sign(o):
    orig = o.e2m1_encode
    o.e2m1_encode = lambda q: orig(np.abs(np.asarray(q, F32)))


def m_zero_drops_sign(o):
    orig = o.e2m1_encode
    def enc(q):
        c = orig(q)
        return np.where((c & 7) == 0, 0, c).astype(np.uint8)
    o.e2m1_encode = enc


def m_no_sat(o):
    orig = o._nearest_code
    def nearest(x, table):
        idx = orig(x, table)
        return np.where(np.asarray(x, np.float64) > table[-1] * 1.0001, len(table) - 2, idx).astype(np.uint8)
    o._nearest_code = nearest


def m_no_div6(o):
    o.encode_block_scale = lambda bamax, s_enc: o.e4m3_encode((np.asarray(bamax, F32) * F32(s_enc)).astype(F32))


def m_div6_before_mul(o):
    o.encode_block_scale = lambda bamax, s_enc: o.e4m3_encode(
        ((np.asarray(bamax, F32) / F32(6)).astype(F32) * F32(s_enc)).astype(F32))


def m_recip_inverted(o):
    def rec(S, s_enc):
        S_val = o.E4M3_VALS[np.minimum(np.asarray(S), 126)].astype(F32)
        return np.where(np.asarray(S) == 0, F32(0), (S_val / F32(s_enc)).astype(F32)).astype(F32)
    o.block_reciprocal = rec


def m_recip_no_zero_rule(o):
    def rec(S, s_enc):
        S_val = o.E4M3_VALS[np.minimum(np.asarray(S), 126)].astype(F32)
        with np.errstate(divide="ignore"):
            return (F32(s_enc) / S_val).astype(F32)
    o.block_reciprocal = rec


def m_nibble_swap(o):
    o.pack_nibbles = lambda nib: ((np.asarray(nib)[:, 1::2] | (np.asarray(nib)[:, 0::2] << 4))).astype(np.uint8)


def m_range_448(o):
    o.GLOBAL_RANGE = 448.0


def m_range_6(o):
    o.GLOBAL_RANGE = 6.0


def m_no_zero_tensor_rule(o):
    orig = o.global_scale
    o.global_scale = lambda amax: F32(0.0) if F32(amax) == 0 else orig(amax)


def m_dequant_no_g(o):
    orig = o.dequantize
    o.dequantize = lambda qt: orig(qt) / np.float64(qt.g)


def m_dequant_scale_shift(o):
    def deq(qt):
        nib = o.unpack_codes(qt.codes)
        rows, K = nib.shape
        vals = o._E2M1_ALL[nib].reshape(rows, K // 16, 16)
        sc = o._E4M3_ALL[np.roll(qt.scales, 1, axis=1)][:, :, None]
        return (vals * sc).reshape(rows, K) * np.float64(qt.g)
    o.dequantize = deq


def m_gemm_modules_reversed(o):
    orig = o.gemm
    o.gemm = lambda xq, mods: orig(xq, list(reversed(mods)))


def m_gemm_shared_scale(o):
    orig = o.gemm
    o.gemm = lambda xq, mods: orig(xq, [o.Quantized(m.codes, m.scales, mods[0].g) for m in mods])


def m_gemm_transposed(o):
    def gemm(xq, mods):
        xh = o.dequantize(xq)
        wh = np.concatenate([o.dequantize(w) for w in mods], axis=0)
        n = min(xh.shape[0], wh.shape[0])
        return (wh[:n] @ xh[:n].T)[: xh.shape[0]], np.abs(wh[:n]) @ np.abs(xh[:n]).T
    o.gemm = gemm


def m_gemm_dequantized_no_abs(o):
    o.gemm_dequantized = lambda xh, wh: (xh @ wh.T, np.abs(xh @ wh.T))


def m_gemm_dequantized_transposed(o):
    o.gemm_dequantized = lambda xh, wh: ((wh @ xh.T).T[:, ::-1].copy(), (np.abs(wh) @ np.abs(xh).T).T[:, ::-1].copy())


def m_block_32(o):
    orig_q = o.quantize
    def quantize(x, g_mode="compute", g=None):
        base = orig_q(x, g_mode, g)
        v = np.asarray(x, F32)
        rows, K = v.shape
        s_enc = F32(1.0) / base.g
        bam = np.repeat(np.max(np.abs(v.reshape(rows, K // 32, 32)), axis=2), 2, axis=1) if K % 32 == 0 else \
            np.max(np.abs(v.reshape(rows, K // 16, 16)), axis=2)
        S = o.encode_block_scale(bam, s_enc)
        r = o.block_reciprocal(S, s_enc)
        nib = o.e2m1_encode((v.reshape(rows, K // 16, 16) * r[:, :, None]).astype(F32)).reshape(rows, K)
        return o.Quantized(o.pack_nibbles(nib), S, base.g, nibbles=nib)
    o.quantize = quantize


def m_amax_per_row(o):
    orig_q = o.quantize
    def quantize(x, g_mode="compute", g=None):
        if g_mode != "compute":
            return orig_q(x, g_mode, g)
        v = np.asarray(x, F32)
        rows = [orig_q(v[i:i + 1]) for i in range(v.shape[0])]
        return o.Quantized(np.concatenate([r.codes for r in rows]), np.concatenate([r.scales for r in rows]),
                           rows[0].g, nibbles=np.concatenate([r.nibbles for r in rows]))
    o.quantize = quantize


def m_e4m3_bias8(o):
    o.E4M3_VALS = o.E4M3_VALS / 2.0
    o._E4M3_ALL = o._E4M3_ALL / 2.0


def m_tolerance_loose(o):
    o.GEMM_RTOL = 1e-3
    orig = o.gemm_within_tolerance
    o.gemm_within_tolerance = lambda y, r, a, rtol=1e-3: orig(y, r, a, rtol)


def m_t_blocks_along_columns(o):
    """x^T encoding that blocks along x's rows' own axis and lays the result out transposed."""
    def quantize_t(x, g_mode="compute", g=None):
        v = np.asarray(x, F32)
        if v.shape[1] % 16:
            v = np.pad(v, ((0, 0), (0, 16 - v.shape[1] % 16)))
        q = o.quantize(v, g_mode, g)
        nib = q.nibbles[:, :x.shape[1]].T.copy()
        sc = np.repeat(q.scales, 16, axis=1)[:, :x.shape[1]].T[:, ::16].copy()
        return o.Quantized(o.pack_nibbles(nib), sc, q.g, nibbles=nib)
    o.quantize_t = quantize_t


def m_t_g_first_column(o):
    orig = o.quantize_t
    o.quantize_t = lambda x, g_mode="compute", g=None: orig(
        x, "given", o.global_scale(F32(np.max(np.abs(np.asarray(x, F32)[:, 0]))))) if g_mode == "compute" \
        else orig(x, g_mode, g)


def m_t_no_transpose_layout(o):
    orig = o.quantize_t
    def quantize_t(x, g_mode="compute", g=None):
        q = orig(x, g_mode, g)
        rows = np.asarray(x).shape[0]
        nib = q.nibbles.reshape(-1, rows)[::-1].copy()       # output rows in reverse column order
        return o.Quantized(o.pack_nibbles(nib), q.scales[::-1].copy(), q.g, nibbles=nib)
    o.quantize_t = quantize_t


MUTANTS = [m_ties_away, m_ties_down, m_e2m1_truncate, m_no_sign, m_zero_drops_sign, m_no_sat, m_no_div6,
           m_div6_before_mul, m_recip_inverted, m_recip_no_zero_rule, m_nibble_swap, m_range_448, m_range_6,
           m_no_zero_tensor_rule, m_dequant_no_g, m_dequant_scale_shift, m_gemm_modules_reversed,
           m_gemm_shared_scale, m_gemm_transposed, m_gemm_dequantized_no_abs,
           m_gemm_dequantized_transposed, m_block_32, m_amax_per_row, m_e4m3_bias8, m_tolerance_loose,
           m_t_blocks_along_columns, m_t_g_first_column, m_t_no_transpose_layout]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutate):
    o = fresh_oracle()
    mutate(o)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(o)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mutate.__name__}"
