"""fp64 CPU oracle for KDA -- TEST INFRASTRUCTURE ONLY.

This package is the reference the HIP library is checked against. It shares no code
with that library and never imports it. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from here; the product path must
never route through it.

Contents
  * ``recurrent``  -- the token-by-token recurrence (plain C, fp64, ``kda_oracle.c``).
  * ``recurrent_bwd`` -- its gradients, the adjoint written out token by token (plain C,
                      fp64, ``kda_oracle_bwd.c``).
  * ``chunked``    -- the chunk decomposition of the same recurrence, written in numpy
                      fp64 with a free chunk size (``chunked.py``); used for stage-level
                      checks and pinned against ``recurrent``.
  * ``gate_activation`` -- the fused gate activation (raw gate input -> per-token log2
                      decay), numpy fp64 (``gate.py``).
  * ``l2norm``, ``beta_sigmoid`` -- the q/k normalisation and beta activation the op can
                      fuse (``preprocess.py``); ``gate_activation_bwd``, ``l2norm_bwd``,
                      ``beta_sigmoid_bwd`` -- their gradients.

All inputs are converted to float64 exactly (bf16 and fp32 values are exactly
representable), so the oracle sees the very values the GPU sees.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_BWD_SRC = os.path.join(_HERE, "kda_oracle_bwd.c")
_BWD_LIB_PATH = os.path.join(_HERE, "libkda_oracle_bwd.so")
_lock = threading.Lock()
_lib = None
_bwd_lib = None


def _gcc(src, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(force: bool = True) -> str:
    """Compile the C oracles with gcc (plain -O2, no fast-math: exact IEEE fp64)."""
    if force or not os.path.exists(_LIB_PATH):
        _gcc(_SRC, _LIB_PATH)
    if force or not os.path.exists(_BWD_LIB_PATH):
        _gcc(_BWD_SRC, _BWD_LIB_PATH)
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load (building first if absent) a compiled oracle; ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    f = lib.kda_oracle_recurrent
    f.restype = ctypes.c_int
    f.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, dp, dp,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    return lib


def _f64(x):
    """Exact conversion of an array-like (numpy or torch, any float dtype) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


def recurrent(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None,
              nthreads=None, lib=None):
    """Token-by-token KDA in fp64. Returns ``(o, final_state)`` as float64 numpy arrays.

    Shapes: q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K] (per-token log2 decay);
    beta [B,T,HV]; initial_state [N,HV,K,V] or None (zeros); cu_seqlens int32 [N+1] or
    None (then N = B). ``scale`` defaults to K**-0.5. Rows of ``o`` outside every
    sequence are left as NaN. Raises ValueError on a malformed ``cu_seqlens``.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    h0 = _f64(initial_state)
    cu = _i32(cu_seqlens)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, HV, K) \
            or beta.shape != (B, T, HV):
        raise ValueError("inconsistent shapes")
    if HV % H != 0:
        raise ValueError("HV must be a multiple of H")
    if cu is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        N = cu.shape[0] - 1
    else:
        N = B
    if h0 is not None and h0.shape != (N, HV, K, V):
        raise ValueError("initial_state must be [N, HV, K, V]")
    if scale is None:
        scale = float(K) ** -0.5
    o = np.full((B, T, HV, V), np.nan, dtype=np.float64)
    ht = np.zeros((N, HV, K, V), dtype=np.float64)
    if lib is None:
        lib = load_library()
    dp = ctypes.POINTER(ctypes.c_double)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = lib.kda_oracle_recurrent(
        ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(h0),
        None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        int(N), ptr(o), ptr(ht), B, T, H, HV, K, V, float(scale),
        int(nthreads or default_threads()))
    if rc == -2:
        raise ValueError("invalid cu_seqlens")
    if rc != 0:
        raise RuntimeError("kda_oracle_recurrent failed with code %d" % rc)
    return o, ht


def load_bwd_library(path: str | None = None):
    """Load (building first if absent) the compiled backward oracle."""
    global _bwd_lib
    if path is not None:
        return _bind_bwd(ctypes.CDLL(path))
    with _lock:
        if _bwd_lib is None:
            if not os.path.exists(_BWD_LIB_PATH):
                _gcc(_BWD_SRC, _BWD_LIB_PATH)
            _bwd_lib = _bind_bwd(ctypes.CDLL(_BWD_LIB_PATH))
    return _bwd_lib


def _bind_bwd(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    f = lib.kda_oracle_recurrent_bwd
    f.restype = ctypes.c_int
    f.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp,
                  dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    return lib


def recurrent_bwd(q, k, v, g, beta, do, initial_state=None, cu_seqlens=None, dht=None,
                  scale=None, nthreads=None, lib=None):
    """Gradients of ``recurrent``'s outputs, in fp64: given ``do`` [B,T,HV,V] (the
    gradient of a loss with respect to o) and ``dht`` [N,HV,K,V] or None (with respect
    to the final state), returns ``(dq, dk, dv, dg, dbeta, dh0)`` as float64 numpy arrays
    with the shapes of q, k, v, g, beta and the initial state; ``dg`` is with respect to
    the per-token log2 decay. Rows outside every sequence get zeros."""
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    h0 = _f64(initial_state)
    dht = _f64(dht)
    cu = _i32(cu_seqlens)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, HV, K) \
            or beta.shape != (B, T, HV) or do.shape != v.shape:
        raise ValueError("inconsistent shapes")
    if HV % H != 0:
        raise ValueError("HV must be a multiple of H")
    if cu is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        N = cu.shape[0] - 1
    else:
        N = B
    for name, a in (("initial_state", h0), ("dht", dht)):
        if a is not None and a.shape != (N, HV, K, V):
            raise ValueError(f"{name} must be [N, HV, K, V]")
    if scale is None:
        scale = float(K) ** -0.5
    dq = np.zeros((B, T, H, K))
    dk = np.zeros((B, T, H, K))
    dq_hv = np.zeros((B, T, HV, K))
    dk_hv = np.zeros((B, T, HV, K))
    dv = np.zeros((B, T, HV, V))
    dg = np.zeros((B, T, HV, K))
    dbeta = np.zeros((B, T, HV))
    dh0 = np.zeros((N, HV, K, V))
    if lib is None:
        lib = load_bwd_library()
    dp = ctypes.POINTER(ctypes.c_double)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(dp)

    rc = lib.kda_oracle_recurrent_bwd(
        ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(h0),
        None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        int(N), ptr(do), ptr(dht), ptr(dq), ptr(dk), ptr(dv), ptr(dg), ptr(dbeta), ptr(dh0),
        ptr(dq_hv), ptr(dk_hv), B, T, H, HV, K, V, float(scale),
        int(nthreads or default_threads()))
    if rc == -2:
        raise ValueError("invalid cu_seqlens")
    if rc != 0:
        raise RuntimeError("kda_oracle_recurrent_bwd failed with code %d" % rc)
    return dq, dk, dv, dg, dbeta, dh0


from . import chunked  # noqa: E402  (numpy only; no dependency on the library above)
from .gate import gate_activation, gate_activation_bwd  # noqa: E402,F401  (numpy only)
from .preprocess import beta_sigmoid, beta_sigmoid_bwd, l2norm, l2norm_bwd  # noqa: E402,F401  (numpy only)
