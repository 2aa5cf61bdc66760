"""Pins of the oracle's fusable input preprocessing (CPU): q/k L2 normalisation and the
beta activation, against closed forms, a scalar brute force, and planted mistakes."""
import math

import numpy as np
import pytest

from oracle.preprocess import L2NORM_EPS, beta_sigmoid, l2norm


def pin_unit_norm(norm, sig):
    """Rows of clearly non-zero vectors come out with norm 1 (to the eps term)."""
    x = np.random.default_rng(1).normal(0, 3, (2, 7, 3, 16))
    y = norm(x)
    n = np.sqrt((y * y).sum(-1))
    return np.allclose(n, 1.0, atol=1e-6) and np.allclose(y * np.sqrt((x * x).sum(-1, keepdims=True) + L2NORM_EPS), x, rtol=1e-12)


def pin_direction_and_axis(norm, sig):
    """Only the last axis is normalised, direction kept: scaling one row by c > 0 leaves
    every row of the output unchanged (to the eps term), scaling an element changes only
    its own row."""
    x = np.random.default_rng(2).normal(0, 1, (1, 4, 2, 8))
    y = norm(x)
    x2 = x.copy()
    x2[0, 1, 0] *= 7.0
    y2 = norm(x2)
    x3 = x.copy()
    x3[0, 2, 1, 3] += 0.5
    moved = np.abs(norm(x3) - y) > 1e-15
    return (np.allclose(y2, y, atol=1e-9) and moved[0, 2, 1].all() and moved.sum() == moved[0, 2, 1].size)


def pin_zero_row(norm, sig):
    """A zero row stays zero (the eps keeps it finite)."""
    x = np.zeros((1, 2, 1, 8))
    x[0, 1, 0, 0] = 3.0
    y = norm(x)
    return np.all(np.isfinite(y)) and np.all(y[0, 0] == 0) and abs(y[0, 1, 0, 0] - 3 / math.sqrt(9 + L2NORM_EPS)) < 1e-15


def pin_sigmoid_values(norm, sig):
    """sigmoid(0) = 1/2; sigmoid(ln 3) = 3/4; large |b| limits; the scale 2 option."""
    b = np.array([0.0, math.log(3.0), -40.0, 40.0])
    s1, s2 = sig(b, False), sig(b, True)
    return (np.allclose(s1, [0.5, 0.75, math.exp(-40.0), 1.0], rtol=1e-14, atol=0)
            and np.allclose(s2, 2 * s1, rtol=1e-15, atol=0))


def pin_brute_force(norm, sig):
    """Scalar loops with math.sqrt / math.exp."""
    rng = np.random.default_rng(3)
    x = rng.normal(0, 2, (1, 3, 2, 5))
    y = norm(x)
    b = rng.normal(0, 3, (1, 3, 2))
    sb = sig(b, True)
    worst = 0.0
    for t in range(3):
        for h in range(2):
            ss = sum(x[0, t, h, d] ** 2 for d in range(5))
            for d in range(5):
                worst = max(worst, abs(y[0, t, h, d] - x[0, t, h, d] / math.sqrt(ss + L2NORM_EPS)))
            worst = max(worst, abs(sb[0, t, h] - 2.0 / (1.0 + math.exp(-b[0, t, h]))))
    return worst < 1e-14


PINS = [pin_unit_norm, pin_direction_and_axis, pin_zero_row, pin_sigmoid_values, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_preprocess_pin(pin):
    assert pin(l2norm, beta_sigmoid)


def _mut(kind):
    def norm(x, eps=L2NORM_EPS):
        x = np.asarray(x, np.float64)
        if kind == "l1":
            return x / (np.abs(x).sum(-1, keepdims=True) + eps)
        if kind == "wrong_axis":
            return x / np.sqrt((x * x).sum(-2, keepdims=True) + eps)
        if kind == "no_sqrt":
            return x / ((x * x).sum(-1, keepdims=True) + eps)
        if kind == "eps_outside":
            return x / (np.sqrt((x * x).sum(-1, keepdims=True)) + 1e-3)
        return l2norm(x, eps)

    def sig(b, allow_neg_eigval=False):
        b = np.asarray(b, np.float64)
        if kind == "tanh":
            return (2.0 if allow_neg_eigval else 1.0) * np.tanh(b)
        if kind == "scale_ignored":
            return 1.0 / (1.0 + np.exp(-b))
        if kind == "sign":
            return (2.0 if allow_neg_eigval else 1.0) / (1.0 + np.exp(b))
        return beta_sigmoid(b, allow_neg_eigval)
    return norm, sig


@pytest.mark.parametrize("kind", ["l1", "wrong_axis", "no_sqrt", "eps_outside", "tanh", "scale_ignored", "sign"])
def test_preprocess_pins_catch_mistake(kind):
    norm, sig = _mut(kind)
    assert [p.__name__ for p in PINS if not p(norm, sig)], kind


def test_mutant_harness_identity():
    norm, sig = _mut("none")
    assert all(p(norm, sig) for p in PINS)
