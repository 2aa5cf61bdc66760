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
