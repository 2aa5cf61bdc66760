"""Chunked form of KDA in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

The chunk decomposition stated in "kernel-fun 0.2.0.dev1 sdist, ALGORITHM.md",
section Forward, written out plainly with a free chunk size ``BT`` and no blocking,
fusion or sub-chunking: every gate factor is the one-sided ``2**(g2[i]-g2[j])`` with
i >= j computed directly, which fp64 represents at any gate magnitude that matters.

Per (sequence, value head hv), with q/k head h = hv // (HV // H):

  Stage 1 (cumsum):   g2[t, d] = sum of g[s, d] over s <= t in t's chunk (base 2
                      already, so the 1/ln2 factor of a natural-log gate is 1);
                      G[d] = g2 at the chunk's last row.
  Stage 2 (intra/WY): Aqk[i, j] = scale * sum_d q[i,d] k[j,d] 2^(g2[i,d]-g2[j,d]), i >= j
                      L[i, j]   = beta[i] * sum_d k[i,d] k[j,d] 2^(g2[i,d]-g2[j,d]), i > j
                      Akk       = (I + L)^-1          (the solved WY inverse, beta in L)
                      w = Akk @ (beta * 2^g2 * k),  u = Akk @ (beta * v)
                      kg = k * 2^(G - g2),          qg = q * 2^g2
  Stage 3+4 (scan):   v' = u - w @ h
                      o  = scale * qg @ h + Aqk @ v'
                      h  = 2^G[:, None] * h + kg^T @ v'
                      after the last chunk the final state is h.

Chunks restart at every sequence start; a sequence's last chunk may be short.
The matrix inverse is a library call (numpy.linalg.solve on the identity).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def gate_cumsum(g_chunk: np.ndarray) -> np.ndarray:
    """Stage 1: inclusive cumsum down the rows of one chunk's [C, K] log2 gates."""
    return np.cumsum(g_chunk, axis=0)


def intra(q, k, v, g2, beta, scale):
    """Stage 2 for one chunk: returns dict(Aqk, L, Akk, w, u, kg, qg, G)."""
    C = q.shape[0]
    # one-sided factor 2^(g2[i]-g2[j]) for every (i, j, d); only i >= j is used
    diff = g2[:, None, :] - g2[None, :, :]                 # [C, C, K]
    lower_incl = np.tril(np.ones((C, C), dtype=bool))
    lower_strict = np.tril(np.ones((C, C), dtype=bool), -1)
    m = lower_incl[:, :, None]
    fac = np.where(m, np.exp2(np.where(m, diff, 0.0)), 0.0)
    Aqk = scale * np.einsum("id,jd,ijd->ij", q, k, fac)
    Aqk = np.where(lower_incl, Aqk, 0.0)
    L = beta[:, None] * np.einsum("id,jd,ijd->ij", k, k, fac)
    L = np.where(lower_strict, L, 0.0)
    Akk = np.linalg.solve(np.eye(C) + L, np.eye(C))
    e = np.exp2(g2)
    G = g2[-1]
    w = Akk @ (beta[:, None] * e * k)
    u = Akk @ (beta[:, None] * v)
    kg = k * np.exp2(G[None, :] - g2)
    qg = q * e
    return dict(Aqk=Aqk, L=L, Akk=Akk, w=w, u=u, kg=kg, qg=qg, G=G)


def scan_step(h, st, scale):
    """Stage 3+4 for one chunk: returns (o_chunk, new_h, v_new)."""
    v_new = st["u"] - st["w"] @ h
    o = scale * (st["qg"] @ h) + st["Aqk"] @ v_new
    h = np.exp2(st["G"])[:, None] * h + st["kg"].T @ v_new
    return o, h, v_new


def chunked(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None,
            chunk_size=64, return_stages=False):
    """KDA via the chunk algebra. Returns ``(o, final_state)`` (float64 numpy), plus a
    list of per-chunk stage dicts when ``return_stages`` (keys n, hv, start, length and
    the Stage 2 tensors). Rows of ``o`` outside every sequence are NaN.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    h0 = _f64(initial_state)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    grp = HV // H
    if scale is None:
        scale = float(K) ** -0.5
    if cu_seqlens is not None:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]
    N = len(seqs)
    o = np.full((B, T, HV, V), np.nan)
    ht = np.zeros((N, HV, K, V))
    stages = []
    for n, (b, bos, eos) in enumerate(seqs):
        for hv in range(HV):
            h = hv // grp
            S = h0[n, hv].copy() if h0 is not None else np.zeros((K, V))
            for s in range(bos, eos, chunk_size):
                e = min(s + chunk_size, eos)
                g2 = gate_cumsum(g[b, s:e, hv])
                st = intra(q[b, s:e, h], k[b, s:e, h], v[b, s:e, hv], g2, beta[b, s:e, hv], scale)
                oc, S, v_new = scan_step(S, st, scale)
                o[b, s:e, hv] = oc
                if return_stages:
                    st = dict(st, n=n, hv=hv, start=s, length=e - s, g2=g2, v_new=v_new)
                    stages.append(st)
            ht[n, hv] = S
    if return_stages:
        return o, ht, stages
    return o, ht
