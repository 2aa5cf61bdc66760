"""Checks that pin a KDA implementation to what the mathematics fixes.

Each ``pin_*`` takes ``impl(q, k, v, g, beta, h0, cu_seqlens, scale) -> (o, ht)``
(numpy float64 in, float64 out; h0/cu_seqlens may be None) and raises AssertionError
when the implementation breaks the property. ``tests/test_oracle_pins.py`` runs them all
on the fp64 oracle; ``tests/test_pin_sensitivity.py`` runs them on copies of the oracle
with planted mistakes and requires each copy to fail at least one of them.

None of these re-types the recurrence the oracle runs: the exact check builds the
explicit K x K transition matrices (I - beta k k^T) Diag(2^g) in rational arithmetic;
the others are closed forms, identities or reductions that hold at any size.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, B=1, T=9, H=1, HV=1, K=8, V=8, h0=True, gate_lo=-3.0):
    r = _rng(seed)
    q = _unit(r.standard_normal((B, T, H, K)))
    k = _unit(r.standard_normal((B, T, H, K)))
    v = r.standard_normal((B, T, HV, V))
    g = r.uniform(gate_lo, 0.0, (B, T, HV, K))
    beta = r.uniform(0.05, 0.95, (B, T, HV))
    s0 = 0.3 * r.standard_normal((B, HV, K, V)) if h0 else None
    return q, k, v, g, beta, s0


# --------------------------------------------------------------------------------------
# P1: exact rational brute force on tiny inputs
# --------------------------------------------------------------------------------------

def _dyadic(r, shape, denom=8, lo=-8, hi=8):
    vals = r.integers(lo, hi + 1, size=shape)
    return vals, denom


def exact_case(seed, B, T, H, HV, K, V, gate_choices=(0, -1, -2, -3)):
    """Inputs that are exact binary fractions, plus integer log2 gates."""
    r = _rng(seed)
    qi, _ = _dyadic(r, (B, T, H, K))
    ki, _ = _dyadic(r, (B, T, H, K))
    vi, _ = _dyadic(r, (B, T, HV, V))
    gi = r.choice(np.array(gate_choices), size=(B, T, HV, K))
    bi = r.integers(0, 5, size=(B, T, HV))          # beta in {0, 1/4, ..., 1}
    hi, _ = _dyadic(r, (B, HV, K, V))
    F = Fraction
    qf = np.vectorize(lambda x: F(int(x), 8), otypes=[object])(qi)
    kf = np.vectorize(lambda x: F(int(x), 8), otypes=[object])(ki)
    vf = np.vectorize(lambda x: F(int(x), 8), otypes=[object])(vi)
    bf = np.vectorize(lambda x: F(int(x), 4), otypes=[object])(bi)
    hf = np.vectorize(lambda x: F(int(x), 16), otypes=[object])(hi)
    gf = gi.astype(np.int64)
    return dict(q=qf, k=kf, v=vf, g=gf, beta=bf, h0=hf)


def exact_reference(case, scale):
    """S_t = M_t S_{t-1} + beta_t k_t v_t^T with M_t = (I - beta_t k_t k_t^T) Diag(2^g_t),
    o_t = scale S_t^T q_t, all in Fractions with explicit K x K matrices."""
    q, k, v, g, beta, h0 = (case[x] for x in ("q", "k", "v", "g", "beta", "h0"))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    grp = HV // H
    F = Fraction
    o = np.empty((B, T, HV, V), dtype=object)
    ht = np.empty((B, HV, K, V), dtype=object)
    for b in range(B):
        for hv in range(HV):
            h = hv // grp
            S = [[h0[b, hv, i, j] for j in range(V)] for i in range(K)]
            for t in range(T):
                kk = [k[b, t, h, i] for i in range(K)]
                bt = beta[b, t, hv]
                dec = [F(2) ** int(g[b, t, hv, i]) for i in range(K)]
                M = [[(F(1) if i == j else F(0)) * dec[j] - bt * kk[i] * kk[j] * dec[j]
                      for j in range(K)] for i in range(K)]
                S = [[sum(M[i][m] * S[m][c] for m in range(K)) + bt * kk[i] * v[b, t, hv, c]
                      for c in range(V)] for i in range(K)]
                for c in range(V):
                    o[b, t, hv, c] = scale * sum(S[i][c] * q[b, t, h, i] for i in range(K))
            for i in range(K):
                for c in range(V):
                    ht[b, hv, i, c] = S[i][c]
    return o, ht


def pin_exact(impl, seed=0, B=2, T=7, H=1, HV=2, K=4, V=3, gates=(0, -1, -2, -3)):
    case = exact_case(seed, B, T, H, HV, K, V, gates)
    scale = Fraction(1, int(round(K ** 0.5)))
    assert scale * scale * K == 1, "K must be a perfect square for an exact scale"
    o_ex, ht_ex = exact_reference(case, scale)
    f = np.vectorize(float, otypes=[np.float64])
    o, ht = impl(f(case["q"]), f(case["k"]), f(case["v"]), case["g"].astype(np.float64),
                 f(case["beta"]), f(case["h0"]), None, float(scale))
    o_ex, ht_ex = f(o_ex), f(ht_ex)
    tol = 1e-13 * max(1.0, np.abs(o_ex).max(), np.abs(ht_ex).max())
    assert np.abs(o - o_ex).max() <= tol, np.abs(o - o_ex).max()
    assert np.abs(ht - ht_ex).max() <= tol, np.abs(ht - ht_ex).max()


# --------------------------------------------------------------------------------------
# P2: retrieval identity.  For a unit key, S_t^T k_t = (1-b) (D_t S_{t-1})^T k_t + b v_t
# --------------------------------------------------------------------------------------

def pin_retrieval(impl, seed=1):
    """beta = 1 and q = k: each output is exactly scale * v_t, whatever the history."""
    q, k, v, g, beta, h0 = random_case(seed, B=2, T=12, H=2, HV=4, K=8, V=6)
    beta = np.ones_like(beta)
    scale = 0.37
    o, _ = impl(k, k, v, g, beta, h0, None, scale)
    assert np.allclose(o, scale * v, rtol=0, atol=1e-12), np.abs(o - scale * v).max()


def pin_retrieval_step(impl, seed=2):
    """General beta, q = k: o_t = scale ((1-b_t) (2^g_t * S_{t-1})^T k_t + b_t v_t),
    with S_{t-1} the final state of the prefix run (decay acts on key rows)."""
    q, k, v, g, beta, h0 = random_case(seed, B=1, T=6, H=1, HV=1, K=7, V=5)
    scale = 0.5
    o, _ = impl(k, k, v, g, beta, h0, None, scale)
    S = h0
    for t in range(6):
        if t > 0:
            _, S = impl(k[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], h0, None, scale)
        D = np.exp2(g[0, t, 0])[:, None] * S[0, 0]
        want = scale * ((1 - beta[0, t, 0]) * (D.T @ k[0, t, 0]) + beta[0, t, 0] * v[0, t, 0])
        assert np.allclose(o[0, t, 0], want, rtol=0, atol=1e-12), (t, np.abs(o[0, t, 0] - want).max())


# --------------------------------------------------------------------------------------
# P3: one-hot keys -- a per-slot exponential moving average in closed form
# --------------------------------------------------------------------------------------

def pin_one_hot(impl, seed=3):
    r = _rng(seed)
    B, T, H, HV, K, V = 1, 15, 1, 1, 5, 4
    idx = r.integers(0, K, size=T)
    k = np.zeros((B, T, H, K))
    k[0, np.arange(T), 0, idx] = 1.0
    q = _unit(r.standard_normal((B, T, H, K)))
    v = r.standard_normal((B, T, HV, V))
    g = r.uniform(-2, 0, (B, T, HV, K))
    beta = r.uniform(0, 1, (B, T, HV))
    h0 = r.standard_normal((B, HV, K, V))
    scale = 0.25
    o, ht = impl(q, k, v, g, beta, h0, None, scale)
    S = h0[0, 0].copy()
    for t in range(T):
        i = idx[t]
        a = np.exp2(g[0, t, 0])
        b = beta[0, t, 0]
        for row in range(K):
            if row == i:
                S[row] = (1 - b) * a[row] * S[row] + b * v[0, t, 0]
            else:
                S[row] = a[row] * S[row]
        want = scale * (q[0, t, 0] @ S)
        assert np.allclose(o[0, t, 0], want, rtol=0, atol=1e-12), t
    assert np.allclose(ht[0, 0], S, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# P4: special cases that reduce to textbook rules
# --------------------------------------------------------------------------------------

def pin_beta_zero(impl, seed=4):
    """beta = 0: nothing is written; the state only decays (a pure gated read of h0)."""
    q, k, v, g, beta, h0 = random_case(seed, B=2, T=10, H=1, HV=2, K=6, V=5)
    beta = np.zeros_like(beta)
    scale = 0.3
    o, ht = impl(q, k, v, g, beta, h0, None, scale)
    cum = np.cumsum(g, axis=1)                                   # full-sequence decay
    for b in range(2):
        for hv in range(2):
            for t in range(10):
                want = scale * ((q[b, t, 0] * np.exp2(cum[b, t, hv])) @ h0[b, hv])
                assert np.allclose(o[b, t, hv], want, rtol=1e-12, atol=1e-13)
            assert np.allclose(ht[b, hv], np.exp2(cum[b, -1, hv])[:, None] * h0[b, hv],
                               rtol=1e-12, atol=1e-14)


def pin_small_beta_gla(impl, seed=5, eps=1e-7):
    """beta = eps * b -> 0 with h0 = 0: o / eps tends to the gated-linear-attention form
    scale * sum_{s <= t} b_s (sum_d q_t k_s 2^(G_t - G_s)) v_s (G the full cumsum)."""
    q, k, v, g, beta, _ = random_case(seed, B=1, T=9, H=1, HV=1, K=6, V=4)
    scale = 0.4
    o, _ = impl(q, k, v, g, eps * beta, None, None, scale)
    cum = np.cumsum(g[0, :, 0], axis=0)
    for t in range(9):
        want = np.zeros(4)
        for s in range(t + 1):
            a = np.sum(q[0, t, 0] * k[0, s, 0] * np.exp2(cum[t] - cum[s]))
            want += beta[0, s, 0] * a * v[0, s, 0]
        want *= scale
        assert np.allclose(o[0, t, 0] / eps, want, rtol=1e-5, atol=1e-6), t


def pin_deltanet(impl, seed=6):
    """g = 0: the DeltaNet rule S_t = S_{t-1} + b_t k_t (v_t - S_{t-1}^T k_t)^T, o_t = scale S_t^T q_t."""
    q, k, v, g, beta, h0 = random_case(seed, B=1, T=11, H=1, HV=1, K=5, V=7)
    g = np.zeros_like(g)
    scale = 0.6
    o, ht = impl(q, k, v, g, beta, h0, None, scale)
    S = h0[0, 0].copy()
    for t in range(11):
        kt = k[0, t, 0]
        S = S + beta[0, t, 0] * np.outer(kt, v[0, t, 0] - S.T @ kt)
        assert np.allclose(o[0, t, 0], scale * S.T @ q[0, t, 0], rtol=0, atol=1e-12)
    assert np.allclose(ht[0, 0], S, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------------------
# P6 .. P10: structural identities
# --------------------------------------------------------------------------------------

def pin_gva(impl, seed=7):
    """HV = G*H value heads reading q/k head h = hv // G  ==  H' = HV heads with q/k
    repeated G times along the head axis (bitwise: the same arithmetic)."""
    q, k, v, g, beta, h0 = random_case(seed, B=1, T=8, H=2, HV=6, K=4, V=3)
    o1, s1 = impl(q, k, v, g, beta, h0, None, 0.5)
    qr = np.repeat(q, 3, axis=2)
    kr = np.repeat(k, 3, axis=2)
    o2, s2 = impl(qr, kr, v, g, beta, h0, None, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    # and a different head->value-head assignment must change the result
    q_alt = np.concatenate([q[:, :, 1:], q[:, :, :1]], axis=2)
    o3, _ = impl(q_alt, k, v, g, beta, h0, None, 0.5)
    assert not np.allclose(o1, o3)


def pin_split_resume(impl, seed=8):
    """run(0..T) == run(0..T1) then run(T1..T) from the first run's final state."""
    q, k, v, g, beta, h0 = random_case(seed, B=2, T=13, H=1, HV=2, K=5, V=4)
    o, ht = impl(q, k, v, g, beta, h0, None, 0.45)
    t1 = 6
    oa, sa = impl(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], h0, None, 0.45)
    ob, sb = impl(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], sa, None, 0.45)
    assert np.allclose(np.concatenate([oa, ob], axis=1), o, rtol=0, atol=1e-13)
    assert np.allclose(sb, ht, rtol=0, atol=1e-13)


def pin_packed(impl, seed=9):
    """Packed sequences == separate dense runs; empty slots pass their state through
    bitwise; rows past the last offset are not written (NaN sentinel stays)."""
    r = _rng(seed)
    lens = [3, 0, 5, 1, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tphys = int(cu[-1]) + 3
    q, k, v, g, beta, _ = random_case(seed, B=1, T=Tphys, H=1, HV=2, K=4, V=3)
    h0 = r.standard_normal((len(lens), 2, 4, 3))
    o, ht = impl(q, k, v, g, beta, h0, cu, 0.5)
    for n, L in enumerate(lens):
        a, b = int(cu[n]), int(cu[n + 1])
        if L == 0:
            assert np.array_equal(ht[n], h0[n])
            continue
        od, sd = impl(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                      h0[n:n + 1], None, 0.5)
        assert np.allclose(o[:, a:b], od, rtol=0, atol=1e-13)
        assert np.allclose(ht[n], sd[0], rtol=0, atol=1e-13)
    assert np.all(np.isnan(o[:, int(cu[-1]):]))


def pin_null_state(impl, seed=10):
    """No initial state == explicit zeros, bitwise."""
    q, k, v, g, beta, _ = random_case(seed, B=2, T=5, H=1, HV=1, K=4, V=4)
    o1, s1 = impl(q, k, v, g, beta, None, None, 0.5)
    o2, s2 = impl(q, k, v, g, beta, np.zeros((2, 1, 4, 4)), None, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def pin_linearity(impl, seed=11):
    """o and the final state are linear in (v, h0) jointly; o is proportional to scale;
    o is linear in q."""
    q, k, v, g, beta, h0 = random_case(seed, B=1, T=7, H=1, HV=1, K=5, V=4)
    o, s = impl(q, k, v, g, beta, h0, None, 0.5)
    o2, s2 = impl(q, k, 4 * v, g, beta, 4 * h0, None, 0.5)
    assert np.allclose(o2, 4 * o, rtol=1e-14, atol=0) and np.allclose(s2, 4 * s, rtol=1e-14, atol=0)
    o3, _ = impl(q, k, v, g, beta, h0, None, 0.125)
    assert np.allclose(o3, o * 0.25, rtol=1e-14, atol=0)
    q2 = _unit(_rng(seed + 100).standard_normal(q.shape))
    oa, _ = impl(q2, k, v, g, beta, h0, None, 0.5)
    ob, _ = impl(q + q2, k, v, g, beta, h0, None, 0.5)
    assert np.allclose(ob, o + oa, rtol=0, atol=1e-12)


def pin_extreme_decay(impl, seed=12):
    """Integer gates down to -40 per step, still exact against rationals."""
    pin_exact(impl, seed=seed, B=1, T=6, H=1, HV=1, K=4, V=2, gates=(0, -15, -40, -1))


ALL_PINS = [
    pin_exact, pin_retrieval, pin_retrieval_step, pin_one_hot, pin_beta_zero,
    pin_small_beta_gla, pin_deltanet, pin_gva, pin_split_resume, pin_packed,
    pin_null_state, pin_linearity, pin_extreme_decay,
]
