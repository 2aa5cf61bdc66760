"""Input preprocessing that the chunked op can fuse, fp64 -- TEST INFRASTRUCTURE ONLY
(part of the oracle package).

  * q, k L2 normalisation over K per (token, head): x / sqrt(sum_d x_d^2 + eps). The
    "kernel-fun 0.2.0.dev1 sdist" page applies fla's l2norm to q and k when
    use_qk_l2norm_in_kernel is set (the autograd Function's forward, which keeps the
    reciprocal norms for the backward); the pages give no epsilon, and the reading taken
    is eps = 1e-6, which only matters for (near-)zero rows.
  * beta from its pre-activation: sigmoid(b) times 2 when negative eigenvalues are
    allowed (beta in (0, 2)), else times 1 (the same page: use_beta_sigmoid_in_kernel,
    fused_beta_sigmoid with scale 2.0 if allow_neg_eigval else 1.0).
  * their backward (the same page: the autograd Function's backward applies fla's
    l2norm_bwd to dq and dk): with y = x r and r = (sum x^2 + eps)^-1/2,
    dx = r (dy - y (y . dy)); for the sigmoid, db = dbeta c s (1 - s) with s = sigmoid(b).
"""
from __future__ import annotations

import numpy as np

L2NORM_EPS = 1e-6


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def l2norm(x, eps=L2NORM_EPS):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def beta_sigmoid(b, allow_neg_eigval=False):
    """sigmoid(b) * (2 if allow_neg_eigval else 1)."""
    b = _f64(b)
    return (2.0 if allow_neg_eigval else 1.0) / (1.0 + np.exp(-b))


def l2norm_bwd(x, dy, eps=L2NORM_EPS):
    """Gradient of ``l2norm`` with respect to x, given dy (the gradient of its output):
    r (dy - y (y . dy)) over the last axis, y = x r, r = (sum x^2 + eps)^-1/2."""
    x, dy = _f64(x), _f64(dy)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * np.sum(y * dy, axis=-1, keepdims=True))


def beta_sigmoid_bwd(b, dbeta, allow_neg_eigval=False):
    """Gradient of ``beta_sigmoid`` with respect to b, given dbeta: c s (1 - s) dbeta."""
    b, dbeta = _f64(b), _f64(dbeta)
    s = 1.0 / (1.0 + np.exp(-b))
    return (2.0 if allow_neg_eigval else 1.0) * s * (1.0 - s) * dbeta
