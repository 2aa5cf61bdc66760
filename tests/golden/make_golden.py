"""Write tests/golden/oracle_regression.npz from the fp64 oracle (only oracle/ is called).

Inputs: seed 0 draws via numpy (B=2, T=37, H=1, HV=2, K=8, V=6, gates in [-4, 0],
beta in [0.05, 0.95], unit-norm q and k, h0 ~ 0.3 N(0, 1)) plus a packed case with an
empty slot. Run from the repository root: ``python tests/golden/make_golden.py``.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def cases():
    r = np.random.default_rng(0)

    def unit(x):
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    B, T, H, HV, K, V = 2, 37, 1, 2, 8, 6
    d = dict(q=unit(r.standard_normal((B, T, H, K))), k=unit(r.standard_normal((B, T, H, K))),
             v=r.standard_normal((B, T, HV, V)), g=r.uniform(-4, 0, (B, T, HV, K)),
             beta=r.uniform(0.05, 0.95, (B, T, HV)), h0=0.3 * r.standard_normal((B, HV, K, V)))
    cu = np.array([0, 20, 20, 50, 71], np.int32)
    Tp = 80
    p = dict(q=unit(r.standard_normal((1, Tp, H, K))), k=unit(r.standard_normal((1, Tp, H, K))),
             v=r.standard_normal((1, Tp, HV, V)), g=r.uniform(-4, 0, (1, Tp, HV, K)),
             beta=r.uniform(0.05, 0.95, (1, Tp, HV)), h0=0.3 * r.standard_normal((4, HV, K, V)),
             cu=cu)
    return d, p


def compute():
    d, p = cases()
    o1, s1 = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, None)
    o2, s2 = oracle.recurrent(p["q"], p["k"], p["v"], p["g"], p["beta"], p["h0"], p["cu"], None)
    return dict(dense_o=o1, dense_ht=s1, packed_o=o2, packed_ht=s2)


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.npz")
    np.savez(out, **compute())
    print("wrote", out)
