"""The FP8 KV-cache oracle against its pins, and planted mistakes in a private copy of it (on the CPU)
that the pins must catch."""
import importlib.util
import os

import numpy as np
import pytest

import kv_pins as pins
from oracle import fp8_kv

KV_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fp8_kv.py")
F32 = np.float32


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(fp8_kv)


def fresh():
    spec = importlib.util.spec_from_file_location("fp8_kv_mutant", KV_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_divide(o):
    def q(x, s_mode="compute", s=None):
        v = np.asarray(x, F32)
        s32 = o.kv_scale(F32(np.max(np.abs(v)))) if s_mode == "compute" else F32(s)
        qq = (v / s32).astype(F32)
        code = o.ref.e4m3_encode(np.abs(np.nan_to_num(qq)).astype(F32)).astype(np.uint8)
        code = np.where(np.isnan(qq), np.uint8(0x7F), code)
        return (code | (np.signbit(qq).astype(np.uint8) << 7)).astype(np.uint8), s32
    o.quantize_kv = q


def m_range_6(o):
    o.KV_RANGE = 6.0


def m_no_sign(o):
    orig = o.quantize_kv
    o.quantize_kv = lambda x, s_mode="compute", s=None: (lambda c, s32: ((c & 0x7F).astype(np.uint8), s32))(
        *orig(x, s_mode, s))


def m_zero_drops_sign(o):
    orig = o.quantize_kv
    def q(x, s_mode="compute", s=None):
        c, s32 = orig(x, s_mode, s)
        return np.where((c & 0x7F) == 0, np.uint8(0), c).astype(np.uint8), s32
    o.quantize_kv = q


def m_ties_up(o):
    orig_enc = o.ref.e4m3_encode
    vals = o.ref.E4M3_VALS.astype(np.float64)
    def enc(u):
        u = np.asarray(u, np.float64)
        hi = np.clip(np.searchsorted(vals, u, side="left"), 1, len(vals) - 1)
        lo = hi - 1
        pick = (vals[hi] - u) <= (u - vals[lo])
        idx = np.where(pick, hi, lo)
        return np.where(u >= vals[-1], len(vals) - 1, np.where(u <= 0, 0, idx)).astype(np.uint8)
    class R:   # a private stand-in for the shared module, so the mutation stays in this copy
        pass
    r = R()
    r.__dict__.update(o.ref.__dict__)
    r.e4m3_encode = enc
    o.ref = r


def m_no_zero_rule(o):
    orig = o.kv_scale
    o.kv_scale = lambda amax: F32(0.0) if F32(amax) == 0 else orig(amax)


def m_dequant_no_scale(o):
    o.dequantize_kv = lambda codes, s: o._E4M3_SIGNED[np.asarray(codes, np.uint8)]


MUTANTS = [m_divide, m_range_6, m_no_sign, m_zero_drops_sign, m_ties_up, m_no_zero_rule, m_dequant_no_scale]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutate):
    o = fresh()
    mutate(o)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(o)
        except Exception as e:  # noqa: BLE001 - any failing pin counts
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught {mutate.__name__}"
