"""Pins of the oracle's output stage (per-head RMSNorm times a sigmoid gate) against what the
definition fixes: unit RMS, scale invariance, hand-computed rows, exact sigmoid values, row
independence and the eps guard.  A planted mistake in any part of the formula fails a pin."""
import numpy as np
import pytest


def pin_unit_rms(og):
    """With eps = 0, no gain and an open gate (sigmoid(60) = 1 in float64), every row has RMS 1."""
    rng = np.random.default_rng(0)
    o = rng.standard_normal((7, 3, 32)) * rng.uniform(0.1, 10, (7, 3, 1))
    y = og(o, np.full_like(o, 60.0), None, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-14)


def pin_scale_invariance(og):
    rng = np.random.default_rng(1)
    o = rng.standard_normal((5, 2, 16))
    z = rng.standard_normal((5, 2, 16))
    w = rng.uniform(0.5, 2.0, 16)
    assert np.allclose(og(3.5 * o, z, w, 0.0), og(o, z, w, 0.0), rtol=1e-14, atol=1e-15)


def pin_hand_rows(og):
    """o = (3, 4, 0, 0): mean square 25/4, so the normed row is (1.2, 1.6, 0, 0); sigmoid(0) = 1/2
    and sigmoid(ln 3) = 3/4 exactly; the gain multiplies channel by channel."""
    o = np.array([[3.0, 4.0, 0.0, 0.0], [3.0, 4.0, 0.0, 0.0]])
    z = np.array([[0.0, 0.0, 0.0, 0.0], [np.log(3.0)] * 4])
    w = np.array([1.0, 2.0, 3.0, 4.0])
    y = og(o, z, w, 0.0)
    assert np.allclose(y[0], [0.6, 1.6, 0.0, 0.0], rtol=0, atol=1e-15)
    assert np.allclose(y[1], [0.9, 2.4, 0.0, 0.0], rtol=0, atol=1e-15)
    # a closed gate passes (almost) nothing
    assert np.abs(og(o, np.full_like(o, -60.0), w, 0.0)).max() < 1e-25


def pin_rows_independent(og):
    """The norm runs over each (token, head) row's dv values only."""
    rng = np.random.default_rng(2)
    o = rng.standard_normal((4, 3, 8))
    z = rng.standard_normal((4, 3, 8))
    y = og(o, z, None, 1e-6)
    o2 = o.copy()
    o2[1, 2] *= 100.0
    o2[3, 0] = 0.0
    y2 = og(o2, z, None, 1e-6)
    keep = np.ones((4, 3), bool)
    keep[1, 2] = keep[3, 0] = False
    assert np.array_equal(y[keep], y2[keep])


def pin_eps(og):
    """eps sits inside the square root: a zero row stays zero, and a row of ones with eps = 3 is
    scaled by 1/2."""
    o = np.zeros((1, 1, 16))
    assert np.array_equal(og(o, np.zeros_like(o), None, 1e-6), o)
    ones = np.ones((1, 1, 16))
    y = og(ones, np.full_like(ones, 60.0), None, 3.0)
    assert np.allclose(y, 0.5, rtol=0, atol=1e-15)


PINS = [pin_unit_rms, pin_scale_invariance, pin_hand_rows, pin_rows_independent, pin_eps]


def _wrap(oracle_mod):
    return lambda o, z, w, eps: oracle_mod.output_gate(o, z, w, eps)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_output_gate_pin(oracle_mod, pin):
    pin(_wrap(oracle_mod))


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


MUTANTS = {
    "mean_abs_not_square": lambda o, z, w, eps: o / (np.mean(np.abs(o), -1, keepdims=True) + eps)
    * (1 if w is None else w) * _sig(z),
    "sum_not_mean": lambda o, z, w, eps: o / np.sqrt(np.sum(o * o, -1, keepdims=True) + eps)
    * (1 if w is None else w) * _sig(z),
    "gate_sign": lambda o, z, w, eps: o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps)
    * (1 if w is None else w) * _sig(-z),
    "norm_over_heads": lambda o, z, w, eps: o / np.sqrt(np.mean(o * o, (-2, -1), keepdims=True)
                                                        + eps) * (1 if w is None else w) * _sig(z),
    "eps_outside_root": lambda o, z, w, eps: o / (np.sqrt(np.mean(o * o, -1, keepdims=True)) + eps)
    * (1 if w is None else w) * _sig(z),
    "gain_dropped": lambda o, z, w, eps: o / np.sqrt(np.mean(o * o, -1, keepdims=True) + eps)
    * _sig(z),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(MUTANTS[name])
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
