"""Pins of the oracle's gradients of the fused preprocessing (CPU): the gate activation
(raw gate, A_log, dt_bias, with and without the lower bound), the q/k L2 normalisation
and the beta sigmoid, each against central finite differences of the forward oracle
function, with planted mistakes that must fail."""
import numpy as np
import pytest

from oracle.gate import gate_activation, gate_activation_bwd
from oracle.preprocess import beta_sigmoid, beta_sigmoid_bwd, l2norm, l2norm_bwd

EPS = 1e-6


def _fd(f, x, w, eps=EPS):
    """Central differences of sum(w * f(x)) in every element of x."""
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy()
        xp[idx] += eps
        xm = x.copy()
        xm[idx] -= eps
        g[idx] = (np.sum(w * f(xp)) - np.sum(w * f(xm))) / (2 * eps)
    return g


def _gate_case(seed):
    rng = np.random.default_rng(seed)
    g = rng.normal(0, 2, (1, 5, 2, 3))
    A = np.log(rng.uniform(1, 2, 2))
    dt = rng.normal(0, 0.5, (2, 3))
    w = rng.normal(size=(1, 5, 2, 3))
    return g, A, dt, w


def pin_gate(bwd, lower_bound):
    g, A, dt, w = _gate_case(3)
    dx, dA, ddt = bwd(g, A, dt, lower_bound, w)
    worst = np.max(np.abs(dx - _fd(lambda x: gate_activation(x, A, dt, lower_bound), g, w)))
    worst = max(worst, np.max(np.abs(dA - _fd(lambda a: gate_activation(g, a, dt, lower_bound), A, w))))
    worst = max(worst, np.max(np.abs(ddt - _fd(lambda t: gate_activation(g, A, t, lower_bound), dt, w))))
    return worst


def pin_l2norm(bwd):
    """Rows at scales 1e-3 (near the eps floor), 1 and 30; the difference step follows
    each row's scale."""
    rng = np.random.default_rng(4)
    worst = 0.0
    for sc in (1e-3, 1.0, 30.0):
        x = rng.normal(0, 1, (2, 8)) * sc
        w = rng.normal(size=x.shape)
        an = bwd(x, w)
        worst = max(worst, np.max(np.abs(an - _fd(l2norm, x, w, eps=1e-5 * sc)) / (1 + np.abs(an))))
    return worst


def pin_sigmoid(bwd):
    rng = np.random.default_rng(5)
    b = rng.normal(0, 3, (4, 5))
    w = rng.normal(size=b.shape)
    worst = 0.0
    for neg in (False, True):
        worst = max(worst, np.max(np.abs(bwd(b, w, neg) - _fd(lambda x: beta_sigmoid(x, neg), b, w))))
    return worst


@pytest.mark.parametrize("bound", [None, -1.5])
def test_gate_bwd_matches_finite_differences(bound):
    assert pin_gate(gate_activation_bwd, bound) < 1e-7


def test_gate_bwd_bound_clamps_something():
    g, A, dt, _ = _gate_case(3)
    gn = gate_activation(g, A, dt, None) * np.log(2.0)
    assert (gn < -1.5).any() and (gn > -1.5).any(), "the bounded pin must exercise both sides"


def test_l2norm_bwd_matches_finite_differences():
    assert pin_l2norm(l2norm_bwd) < 1e-7


def test_beta_sigmoid_bwd_matches_finite_differences():
    assert pin_sigmoid(beta_sigmoid_bwd) < 1e-7


def _gate_mut(kind):
    def bwd(g, A, dt, lb, dgate):
        dx, dA, ddt = gate_activation_bwd(g, A, dt, lb, dgate)
        if kind == "no_ln2":
            return dx * np.log(2.0), dA * np.log(2.0), None if ddt is None else ddt * np.log(2.0)
        if kind == "clamp_ignored":
            return gate_activation_bwd(g, A, dt, None, dgate)
        if kind == "dA_sign":
            return dx, -dA, ddt
        if kind == "ddt_over_heads":
            return dx, dA, None if ddt is None else np.broadcast_to(ddt.sum(0, keepdims=True), ddt.shape)
        return dx, dA, ddt
    return bwd


@pytest.mark.parametrize("kind", ["no_ln2", "clamp_ignored", "dA_sign", "ddt_over_heads"])
def test_gate_bwd_pin_catches_mistake(kind):
    bound = -1.5 if kind == "clamp_ignored" else None
    assert pin_gate(_gate_mut(kind), bound) > 1e-4


@pytest.mark.parametrize("kind", ["no_projection", "rstd_squared"])
def test_l2norm_bwd_pin_catches_mistake(kind):
    def bwd(x, dy):
        r = 1.0 / np.sqrt(np.sum(x * x, -1, keepdims=True) + 1e-6)
        if kind == "no_projection":
            return r * dy
        return r * r * (dy - x * r * np.sum(x * r * dy, -1, keepdims=True))
    assert pin_l2norm(bwd) > 1e-4


def test_sigmoid_bwd_pin_catches_mistake():
    def bwd(b, w, neg):
        s = 1.0 / (1.0 + np.exp(-b))
        return s * (1 - s) * w          # the factor 2 of allow_neg_eigval dropped
    assert pin_sigmoid(bwd) > 1e-4
