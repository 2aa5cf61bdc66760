"""Fused gate activation, fp64 -- TEST INFRASTRUCTURE ONLY (part of the oracle package).

The gate input w_g(x) [B, T, HV, K] is turned into the per-token log2 decay the
recurrence consumes:

    gate[b, t, hv, d] = -exp(A_log[hv]) * softplus(g[b, t, hv, d] + dt_bias[hv, d]) / ln 2

softplus(x) = log(1 + e^x). The activation itself is stated on the "kernel-fun 0.2.0.dev1
sdist" page (the chain module's gate_cumsum helper and its docstring, the op's
use_gate_in_kernel path: A_log [HV], dt_bias [HV*K]); ALGORITHM.md, Forward, places it in
stage 1's cumsum, and the cumsum's scale 1/ln 2 turns the natural-log activation into
the base-2 gate of the chunk algebra. The pages name an optional ``lower_bound`` but
give no formula for it; the reading taken here is the plain one: the natural-log
activation is clamped from below at lower_bound (< 0).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def softplus(x):
    """log(1 + e^x) without overflow."""
    return np.logaddexp(0.0, x)


def gate_activation(g_raw, A_log, dt_bias=None, lower_bound=None):
    """Per-token log2 decay [B, T, HV, K] from the raw gate input (see the module doc)."""
    g = _f64(g_raw)
    B, T, HV, K = g.shape
    a = _f64(A_log).reshape(HV)
    x = g if dt_bias is None else g + _f64(dt_bias).reshape(HV, K)
    gn = -np.exp(a)[:, None] * softplus(x)
    if lower_bound is not None:
        gn = np.maximum(gn, float(lower_bound))
    return gn / np.log(2.0)


def gate_activation_bwd(g_raw, A_log, dt_bias, lower_bound, dgate):
    """Gradients of ``gate_activation`` given dgate (the gradient of its log2 output):
    returns (d g_raw, d A_log [HV], d dt_bias [HV, K] or None). With x = g + dt_bias and
    gn = -e^A softplus(x) the natural-log value, where the lower bound does not clamp:
    d gn = dgate / ln 2, d x = d gn (-e^A sigmoid(x)), d A_log = sum of d gn gn over
    (b, t, d) per head, d dt_bias = sum of d x over (b, t) per (head, channel); where the
    bound clamps, nothing flows back. The gate backward of the "kernel-fun 0.2.0.dev1
    sdist" page (the chain module's gate_backward: dg with respect to the raw input,
    dA_log, ddt_bias)."""
    g = _f64(g_raw)
    B, T, HV, K = g.shape
    a = _f64(A_log).reshape(HV)
    x = g if dt_bias is None else g + _f64(dt_bias).reshape(HV, K)
    gn = -np.exp(a)[:, None] * softplus(x)
    dgn = _f64(dgate) / np.log(2.0)
    if lower_bound is not None:
        dgn = np.where(gn < float(lower_bound), 0.0, dgn)
    sig = 1.0 / (1.0 + np.exp(-x))
    dx = dgn * (-np.exp(a)[:, None]) * sig
    dA = np.sum(dgn * gn, axis=(0, 1, 3))
    ddt = None if dt_bias is None else np.sum(dx, axis=(0, 1))
    return dx, dA, ddt
