"""The gate-epilogue oracle against its pins, and planted mistakes in a private copy of it
(on the CPU) that the pins must catch."""
import importlib.util
import os

import numpy as np
import pytest

import gate_pins as pins
from oracle import gdn_gates

GATES_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "gdn_gates.py")


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(gdn_gates)


def fresh():
    spec = importlib.util.spec_from_file_location("gdn_gates_mutant", GATES_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_softplus_no_log(o):
    o.softplus = lambda z: np.exp(np.asarray(z, np.float64))


def m_softplus_unshifted(o):
    o.softplus = lambda z: np.log1p(np.exp(np.asarray(z, np.float64)) + 1.0)


def m_sigmoid_sign(o):
    o.sigmoid = lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, np.float64)))


def m_decay_no_exp_A(o):
    o.decay = lambda a, A, b: np.exp(-np.asarray(A, np.float64) * o.softplus(np.asarray(a, np.float64) + b))


def m_decay_no_bias(o):
    o.decay = lambda a, A, b: np.exp(-np.exp(np.asarray(A, np.float64)) * o.softplus(np.asarray(a, np.float64)))


def m_decay_sign(o):
    o.decay = lambda a, A, b: np.exp(np.exp(np.asarray(A, np.float64)) * o.softplus(np.asarray(a, np.float64) + b))


def m_gates_off_by_one(o):
    orig = o.apply_gates
    o.apply_gates = lambda y, ac, na, bc, nb, A, b: orig(y, ac + 1, na, bc, nb, A, b)


def m_gates_swapped(o):
    orig = o.apply_gates
    o.apply_gates = lambda y, ac, na, bc, nb, A, b: orig(y, bc, nb, ac, na, A, b)


def m_tolerance_no_derivative(o):
    orig = o.gates_tolerance

    def tol(y, a_ref, ac, na, bc, nb, A, b):
        t = orig(y, a_ref * 0, ac, na, bc, nb, A, b)
        keep = np.ones(t.shape[1], bool)
        keep[ac:ac + na] = False
        keep[bc:bc + nb] = False
        t[:, keep] = o.ref.GEMM_RTOL * np.asarray(a_ref)[:, keep]
        return t
    o.gates_tolerance = tol


def m_within_relative(o):
    def within(out_gpu, out_ref, tol):
        err = np.abs(np.asarray(out_gpu, np.float64) - out_ref) / np.maximum(np.abs(out_ref), 1e-300)
        worst = float(err.max()) if err.size else 0.0
        return bool(worst <= 1e-5), worst
    o.within = within


MUTANTS = [m_softplus_no_log, m_softplus_unshifted, m_sigmoid_sign, m_decay_no_exp_A, m_decay_no_bias, m_decay_sign,
           m_gates_off_by_one, m_gates_swapped, m_tolerance_no_derivative, m_within_relative]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutate):
    o = fresh()
    mutate(o)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(o)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mutate.__name__}"
