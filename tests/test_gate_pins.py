"""Pins of the oracle's fused gate activation (CPU): closed forms, limits, the clamp,
a pure-Python scalar brute force, and planted mistakes that must each fail a pin.

Activation (oracle/gate.py): gate = -exp(A_log[hv]) * softplus(g + dt_bias[hv, d]) / ln 2,
optionally with the natural-log activation clamped from below at lower_bound.
"""
import math

import numpy as np
import pytest

from oracle import gate as gate_mod
from oracle.gate import gate_activation

LN2 = math.log(2.0)


def _rand(seed, B=1, T=5, HV=3, K=4):
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, 3.0, (B, T, HV, K))
    A_log = rng.normal(0.0, 0.7, HV)
    dt = rng.normal(0.0, 1.0, HV * K)
    return g, A_log, dt


# ---- the pins, each a function of an activation implementation `act` ----
def pin_softplus_zero(act):
    """x = 0: softplus = ln 2, so with A_log = 0 the log2 gate is exactly -1, and with
    A_log = ln 3 it is -3."""
    HV, K = 2, 3
    dt = np.linspace(-1.0, 1.0, HV * K)
    g = -dt.reshape(1, 1, HV, K).copy()
    out = act(g, np.array([0.0, math.log(3.0)]), dt, None)
    want = np.array([-1.0, -3.0])[None, None, :, None] * np.ones((1, 1, HV, K))
    return np.abs(out - want).max() < 1e-14


def pin_limits(act):
    """x -> -inf: softplus ~ e^x; x -> +inf: softplus ~ x (closed forms to fp64)."""
    A = np.array([0.3])
    g = np.array([-40.0, -30.0, 30.0, 45.0]).reshape(1, 4, 1, 1)
    out = act(g, A, None, None)[0, :, 0, 0]
    x = g[0, :, 0, 0]
    sp = np.where(x < 0, np.exp(x), x)
    want = -math.exp(0.3) * sp / LN2
    return np.allclose(out, want, rtol=1e-12, atol=0.0)


def pin_brute_force(act):
    """Against a pure-Python scalar loop: log1p(exp(x)) (x <= 30) or x + log1p(exp(-x))."""
    g, A, dt = _rand(7)
    lb = -2.5
    out = act(g, A, dt, lb)
    B, T, HV, K = g.shape
    worst = 0.0
    for t in range(T):
        for h in range(HV):
            for d in range(K):
                x = g[0, t, h, d] + dt[h * K + d]
                sp = math.log1p(math.exp(x)) if x <= 30 else x + math.log1p(math.exp(-x))
                gn = max(-math.exp(A[h]) * sp, lb)
                worst = max(worst, abs(out[0, t, h, d] - gn / LN2))
    return worst < 1e-13


def pin_lower_bound(act):
    """The clamp: activations below lower_bound become lower_bound / ln 2, the others are
    unchanged; without a bound nothing is clamped."""
    g, A, dt = _rand(3)
    free = act(g, A, dt, None)
    lb = -1.75
    clamped = act(g, A, dt, lb)
    below = free * LN2 < lb
    return (below.any() and (~below).any()
            and np.allclose(clamped[below], lb / LN2, rtol=0, atol=1e-15)
            and np.array_equal(clamped[~below], free[~below]))


def pin_per_head_channel_map(act):
    """dt_bias is indexed [hv, d] (hv-major) and A_log by hv: shifting one (hv, d) entry
    of dt_bias moves only that channel of that head."""
    g, A, dt = _rand(11)
    base = act(g, A, dt, None)
    dt2 = dt.copy()
    HV, K = g.shape[2], g.shape[3]
    dt2[1 * K + 2] += 1.0
    moved = act(g, A, dt2, None) != base
    return moved[:, :, 1, 2].all() and moved.sum() == moved[:, :, 1, 2].size


PINS = [pin_softplus_zero, pin_limits, pin_brute_force, pin_lower_bound, pin_per_head_channel_map]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_gate_pin(pin):
    assert pin(gate_activation)


# ---- planted mistakes: each must fail at least one pin ----
def _mutant(kind):
    def act(g_raw, A_log, dt_bias=None, lower_bound=None):
        g = np.asarray(g_raw, np.float64)
        B, T, HV, K = g.shape
        a = np.asarray(A_log, np.float64).reshape(HV)
        dt = 0.0 if dt_bias is None else np.asarray(dt_bias, np.float64).reshape(HV, K)
        if kind == "dt_transposed" and dt_bias is not None:
            dt = np.asarray(dt_bias, np.float64).reshape(K, HV).T
        x = g + dt
        sp = gate_mod.softplus(x)
        if kind == "exp_not_softplus":
            sp = np.exp(x)
        if kind == "relu_not_softplus":
            sp = np.maximum(x, 0.0)
        scale_a = np.exp(a) if kind != "A_log_not_exponentiated" else a
        gn = -scale_a[:, None] * sp
        if kind == "positive_sign":
            gn = -gn
        if lower_bound is not None and kind != "bound_ignored":
            gn = np.maximum(gn, float(lower_bound)) if kind != "bound_as_upper" else np.minimum(gn, float(lower_bound))
        if kind == "natural_log_units":
            return gn
        if kind == "log10_units":
            return gn / math.log(10.0)
        return gn / LN2
    return act


MUTANTS = ["dt_transposed", "exp_not_softplus", "relu_not_softplus", "A_log_not_exponentiated",
           "positive_sign", "bound_ignored", "bound_as_upper", "natural_log_units", "log10_units"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_gate_pins_catch_mistake(kind):
    act = _mutant(kind)
    failed = [p.__name__ for p in PINS if not p(act)]
    assert failed, f"no pin catches the planted mistake {kind!r}"


def test_mutant_harness_identity():
    """The mutant builder with no mistake passes every pin (the harness itself is sound)."""
    act = _mutant("none")
    assert all(p(act) for p in PINS)
