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
