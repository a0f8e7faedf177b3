"""The RHT oracle against its pins, and planted mistakes in a private copy of it (on the CPU)
that the pins must catch."""
import importlib.util
import os

import numpy as np
import pytest

import rht_pins as pins
from oracle import rht

RHT_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "rht.py")
F32 = np.float32


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(rht)


def fresh():
    spec = importlib.util.spec_from_file_location("rht_mutant", RHT_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_reverse_stages(o):
    o.STAGES = (8, 4, 2, 1)


def m_no_quarter(o):
    orig = o.rht_blocks
    o.rht_blocks = lambda x, s: (orig(x, s) * F32(4.0)).astype(F32)


def m_half_instead_of_quarter(o):
    orig = o.rht_blocks
    o.rht_blocks = lambda x, s: (orig(x, s) * F32(2.0)).astype(F32)


def m_signs_after(o):
    orig = o.rht_blocks
    def rht_blocks(x, s):
        y = orig(x, 0)
        rows, K = y.shape
        return (y.reshape(rows, K // 16, 16) * o.sign_vector(s)).astype(F32).reshape(rows, K)
    o.rht_blocks = rht_blocks


def m_signs_bit_reversed(o):
    orig = o.sign_vector
    o.sign_vector = lambda s: orig(s)[::-1].copy()


def m_g_untransformed(o):
    def quantize_rht(x, s, g_mode="compute", g=None):
        if g_mode == "compute":
            g = o.ref.global_scale(F32(np.max(np.abs(np.asarray(x, F32)))))
        return o.ref.quantize(o.rht_blocks(x, s), "given", g)
    o.quantize_rht = quantize_rht


def m_t_not_transposed(o):
    o.quantize_t_rht = lambda x, s, g_mode="compute", g=None: o.quantize_rht(
        np.asarray(x, F32)[: (np.asarray(x).shape[0] // 16) * 16].reshape(-1, 16), s, g_mode, g)


MUTANTS = [m_reverse_stages, m_no_quarter, m_half_instead_of_quarter, m_signs_after, m_signs_bit_reversed,
           m_g_untransformed, m_t_not_transposed]


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
