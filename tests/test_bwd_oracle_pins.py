"""Pins of the backward oracle (CPU): every gradient it returns must match central
finite differences of the forward oracle, element by element, on small cases that
cover packed sequences (an empty one, lengths crossing the 64-token checkpoint
boundary), dense batches, GVA, an initial state and a final-state gradient. Copies of
the backward source with one planted mistake each must fail that pin."""
import os
import subprocess

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle_bwd.c")


def _case(kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "packed":
        lens = [70, 0, 80]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B, T, H, HV, K, V = 1, int(cu[-1]) + 5, 1, 2, 4, 3
        N = len(lens)
    else:
        cu = None
        B, T, H, HV, K, V = 2, 70, 2, 4, 4, 3
        N = B
    q = rng.normal(size=(B, T, H, K))
    k = rng.normal(size=(B, T, H, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, HV, V))
    g = -rng.uniform(0.0, 0.7, size=(B, T, HV, K))
    beta = rng.uniform(0.1, 1.2, size=(B, T, HV))
    h0 = rng.normal(size=(N, HV, K, V)) * 0.3 if kind == "packed" else None
    do = rng.normal(size=(B, T, HV, V))
    dht = rng.normal(size=(N, HV, K, V)) if kind == "packed" else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, cu=cu, do=do, dht=dht)


def _loss(c, **over):
    a = dict(c)
    a.update(over)
    o, ht = oracle.recurrent(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], nthreads=1)
    o = np.nan_to_num(o)   # rows outside every sequence
    L = float(np.sum(o * c["do"]))
    if c["dht"] is not None:
        L += float(np.sum(ht * c["dht"]))
    return L


def _fd(c, name, eps=1e-5, sample=None):
    """Central differences of the loss in every element of input ``name`` (or in
    ``sample`` seeded random elements; the others are left at zero)."""
    x = c[name]
    grad = np.zeros_like(x)
    idxs = list(np.ndindex(*x.shape))
    if sample is not None and sample < len(idxs):
        pick = np.random.default_rng(7).choice(len(idxs), size=sample, replace=False)
        idxs = [idxs[i] for i in pick]
    for idx in idxs:
        xp = x.copy()
        xp[idx] += eps
        xm = x.copy()
        xm[idx] -= eps
        grad[idx] = (_loss(c, **{name: xp}) - _loss(c, **{name: xm})) / (2 * eps)
    return grad


def pin_finite_differences(bwd, c, sample=None):
    """Largest |analytic - finite difference| / (1 + |analytic|) over every element of
    every gradient (or over ``sample`` elements of each)."""
    dq, dk, dv, dg, dbeta, dh0 = bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"],
                                     c["h0"], c["cu"], c["dht"], nthreads=1)
    pairs = [("q", dq), ("k", dk), ("v", dv), ("g", dg), ("beta", dbeta)]
    if c["h0"] is not None:
        pairs.append(("h0", dh0))
    worst = 0.0
    for name, an in pairs:
        fd = _fd(c, name, sample=sample)
        if sample is not None:
            idxs = list(np.ndindex(*an.shape))
            if sample < len(idxs):
                pick = np.random.default_rng(7).choice(len(idxs), size=sample, replace=False)
                mask = np.zeros(an.shape, bool)
                for i in pick:
                    mask[idxs[i]] = True
                an, fd = an[mask], fd[mask]
        worst = max(worst, float(np.max(np.abs(an - fd) / (1.0 + np.abs(an)))))
    return worst


@pytest.fixture(scope="module")
def cases():
    return {"packed": _case("packed", 1), "dense_gva": _case("dense", 2)}


@pytest.mark.parametrize("kind", ["packed", "dense_gva"])
def test_bwd_oracle_matches_finite_differences(cases, kind):
    worst = pin_finite_differences(oracle.recurrent_bwd, cases[kind])
    assert worst < 1e-7, worst


def test_bwd_oracle_null_initial_state_equals_zeros(cases):
    """With no initial state the forward reads zeros, and dh0 is still the gradient with
    respect to that (zero) state: checked against the packed case with h0 = 0 given."""
    c = dict(cases["packed"])
    z = np.zeros_like(c["h0"])
    a = oracle.recurrent_bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], None, c["cu"], c["dht"])
    b = oracle.recurrent_bwd(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], z, c["cu"], c["dht"])
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_oracle_empty_slot_and_tail(cases):
    """The empty slot passes dht to dh0 unchanged; rows past the last offset get zero
    gradients."""
    c = cases["packed"]
    dq, dk, dv, dg, dbeta, dh0 = oracle.recurrent_bwd(c["q"], c["k"], c["v"], c["g"], c["beta"],
                                                      c["do"], c["h0"], c["cu"], c["dht"])
    assert np.array_equal(dh0[1], c["dht"][1])
    end = int(c["cu"][-1])
    for x in (dq, dk, dv, dg, dbeta):
        assert not np.any(x[:, end:])


MUTANTS = {
    "dg_natural_units": ("dgt[d] = LN2 * acc;", "dgt[d] = acc;"),
    "dp_sign": ("dp[c] = -bt * ddel[c];", "dp[c] = bt * ddel[c];"),
    "dk_misses_prediction_path": ("                dkt[d] += acc;\n", ""),
    "no_state_decay_in_adjoint": ("A[(size_t)d * V + c] = a * dSd[(size_t)d * V + c];",
                                  "A[(size_t)d * V + c] = dSd[(size_t)d * V + c];"),
    "read_scale_dropped": ("dqt[d] = J->scale * acc;", "dqt[d] = acc;"),
    "dbeta_uses_v_only": ("acc += ddel[c] * (vt[c] - p[c]);", "acc += ddel[c] * vt[c];"),
    "dht_ignored": ("memcpy(A, J->dht + sofs, sizeof(double) * KV);", "memset(A, 0, sizeof(double) * KV);"),
    "gva_first_head_only": ("for (int j = 0; j < G; ++j) {", "for (int j = 0; j < 1; ++j) {"),
    "checkpoint_off_by_one": ("memcpy(S, W->ckpt + (size_t)sgi * KV, sizeof(double) * KV);",
                              "memcpy(S, W->ckpt + (size_t)(sgi > 0 ? sgi - 1 : 0) * KV, sizeof(double) * KV);"),
    "read_adjoint_before_update": ("A[(size_t)d * V + c] += J->scale * qt[d] * dot[c];",
                                   "A[(size_t)d * V + c] += 0.0 * qt[d] * dot[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pin_catches_planted_mistake(tmp_path, cases, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    c_file = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c_file.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", str(c_file),
                    "-o", str(so), "-lm"], check=True)
    lib = oracle.load_bwd_library(str(so))

    def bwd(*a, **kw):
        return oracle.recurrent_bwd(*a, lib=lib, **kw)
    worst = max(pin_finite_differences(bwd, cases[k], sample=40) for k in ("packed", "dense_gva"))
    assert worst > 1e-4, f"{name} survived the pin (worst {worst:.2e})"
