"""ctypes binding of libkda.so (see ``include/kda.h`` for the contract)."""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
KDA_DEV_BAD_CU_SEQLENS = 1
KDA_GATE_LOG2 = 0
KDA_GATE_RAW_F32 = 1
KDA_GATE_RAW_BF16 = 2
KDA_PRE_L2NORM_Q = 1
KDA_PRE_L2NORM_K = 2
KDA_PRE_BETA_SIGMOID = 4
KDA_PRE_NEG_EIGVAL = 8
KDA_STATE_KV = 0
KDA_STATE_VK = 1

_lock = threading.Lock()
_lib = None


class KdaError(RuntimeError):
    """A non-zero status from the library, with its reason string."""

    def __init__(self, code: int, reason: str):
        super().__init__(f"kda error {code}: {reason}")
        self.code = code
        self.reason = reason


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the built library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m gated_delta_rule_64_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.kda_chunk_fwd.restype = i32
        lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                      i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                      vp, sz, vp, vp]
        lib.kda_chunk_fwd_gated.restype = i32
        lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, ctypes.c_float, vp, vp,
                                            vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            i32, ctypes.c_float, i32, vp, sz, vp, vp]
        lib.kda_chunk_fwd_ex.restype = i32
        lib.kda_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, f32, vp, i32, vp, vp,
                                         i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                         f32, i32, vp, sz, vp, vp, vp]
        lib.kda_recurrent_fwd_ex.restype = i32
        lib.kda_recurrent_fwd_ex.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, f32, vp, i32, i32,
                                             vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32, i32, f32, vp, vp]
        lib.kda_chunk_bwd.restype = i32
        lib.kda_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                      vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp,
                                      sz, vp, vp]
        lib.kda_chunk_bwd_ex.restype = i32
        lib.kda_chunk_bwd_ex.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, f32, vp, i32, vp, vp, i32,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                         i32, i32, i32, i32, f32, i32, vp, sz, vp, vp]
        lib.kda_chunk_bwd_ex_workspace_bytes.restype = sz
        lib.kda_chunk_bwd_ex_workspace_bytes.argtypes = [i32] * 9
        lib.kda_chunk_bwd_workspace_bytes.restype = sz
        lib.kda_chunk_bwd_workspace_bytes.argtypes = [i32] * 9
        lib.kda_recurrent_fwd.restype = i32
        lib.kda_recurrent_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                          i32, i32, i32, i32, i32, i32, i32, i32, f32, vp, vp]
        lib.kda_chunk_fwd_workspace_bytes.restype = sz
        lib.kda_chunk_fwd_workspace_bytes.argtypes = [i32] * 9
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_abi_version.restype = i32
        lib.kda_abi_version.argtypes = []
        _lib = lib
        return lib


def kda_last_error() -> str:
    return load_library().kda_last_error().decode()


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"{what} must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_device(tensors):
    dev = None
    for name, t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def _common(q, k, v, g, beta, initial_state, cu_seqlens, raw_gate=False):
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B, T, H, K] and v [B, T, HV, V]")
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if tuple(k.shape) != tuple(q.shape):
        raise ValueError(f"q and k must match, got {tuple(q.shape)} vs {tuple(k.shape)}")
    if tuple(v.shape[:2]) != (B, T):
        raise ValueError("v must share B and T with q")
    if tuple(g.shape) != (B, T, HV, K):
        raise ValueError(f"g must be {[B, T, HV, K]}, got {list(g.shape)}")
    if tuple(beta.shape) != (B, T, HV):
        raise ValueError(f"beta must be {[B, T, HV]}, got {list(beta.shape)}")
    if not raw_gate and g.dtype != torch.float32:
        raise TypeError("g must be float32 (per-token log2 decay)")
    if raw_gate and g.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("the raw gate input must be float32 or bfloat16")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    qkv = _dtype_code(q, "q")
    bdt = _dtype_code(beta, "beta")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        if initial_state.dtype != torch.float32:
            raise TypeError("initial_state must be float32")
        if tuple(initial_state.shape) != (N, HV, K, V):
            raise ValueError(f"initial_state must be {[N, HV, K, V]}, got {list(initial_state.shape)}")
    dev = _check_device([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                         ("initial_state", initial_state), ("cu_seqlens", cu_seqlens)])
    return B, T, H, HV, K, V, N, qkv, bdt, dev


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, packed, dtype=KDA_BF16) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, int(bool(packed)), int(dtype)))


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                  output_final_state=False, scale=None, *, out=None, final_state=None,
                  workspace=None, dev_status=None):
    """Chunked KDA forward. Returns ``(o, final_state or None)``.

    ``out`` / ``final_state`` / ``workspace`` may be given to reuse buffers;
    ``dev_status`` (int32 [1] GPU tensor) receives device-side check flags.
    ``final_state`` may be ``initial_state`` itself (in place).
    """
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    if out is None:
        out = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state), B, T, H, HV, K, V,
                           qkv, bdt, float(scale or 0.0), 64, _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _ptr(dev_status),
                           _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return out, final_state


def kda_chunk_fwd_gated(q, k, v, g_raw, beta, A_log, dt_bias=None, lower_bound=None,
                        initial_state=None, cu_seqlens=None, output_final_state=False, scale=None,
                        *, out=None, final_state=None, workspace=None, dev_status=None):
    """Chunked KDA forward with the gate activation fused into Stage 1.

    ``g_raw`` is the raw gate input [B, T, HV, K] (bfloat16 or float32); the library forms
    the per-token log2 decay -exp(A_log[hv]) * softplus(g_raw + dt_bias[hv, d]) / ln 2,
    the natural-log activation clamped from below at ``lower_bound`` (a negative float)
    when one is given. ``A_log``: float32 [HV]; ``dt_bias``: float32 [HV * K] or [HV, K],
    or None for zeros. Returns ``(o, final_state or None)`` like ``kda_chunk_fwd``.
    """
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g_raw, beta, initial_state, cu_seqlens,
                                                  raw_gate=True)
    if A_log.dtype != torch.float32 or A_log.numel() != HV:
        raise ValueError(f"A_log must be float32 with {HV} elements")
    if dt_bias is not None and (dt_bias.dtype != torch.float32 or dt_bias.numel() != HV * K):
        raise ValueError(f"dt_bias must be float32 with {HV * K} elements")
    _check_device([("g_raw", g_raw), ("A_log", A_log), ("dt_bias", dt_bias)])
    if out is None:
        out = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _dtype_code(g_raw, "g_raw"),
                                 _ptr(A_log), _ptr(dt_bias), int(lower_bound is not None),
                                 float(lower_bound if lower_bound is not None else 0.0), _ptr(beta),
                                 _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out),
                                 _ptr(final_state), B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0),
                                 64, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return out, final_state


def kda_recurrent_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                      output_final_state=False, scale=None, *, out=None, final_state=None,
                      dev_status=None):
    """Per-token recurrent KDA forward. Returns ``(o, final_state or None)``."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    if out is None:
        out = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    rc = lib.kda_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                               _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state), B, T, H, HV, K, V,
                               qkv, bdt, float(scale or 0.0), _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return out, final_state


def _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound, use_qk_l2norm_in_kernel,
             l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel, allow_neg_eigval):
    """The gate code and preprocessing flags of the _ex entry points, with checks."""
    if use_gate_in_kernel:
        gate = KDA_GATE_RAW_BF16 if g.dtype == torch.bfloat16 else KDA_GATE_RAW_F32
        if A_log is None:
            raise ValueError("A_log is required with use_gate_in_kernel")
        if A_log.dtype != torch.float32 or A_log.numel() != HV:
            raise ValueError(f"A_log must be float32 with {HV} elements")
        if dt_bias is not None and (dt_bias.dtype != torch.float32 or dt_bias.numel() != HV * K):
            raise ValueError(f"dt_bias must be float32 with {HV * K} elements")
        _check_device([("g", g), ("A_log", A_log), ("dt_bias", dt_bias)])
    else:
        if A_log is not None or dt_bias is not None or lower_bound is not None:
            raise ValueError("A_log, dt_bias and lower_bound need use_gate_in_kernel")
        gate = KDA_GATE_LOG2
    lq = use_qk_l2norm_in_kernel if l2norm_q is None else l2norm_q
    lk = use_qk_l2norm_in_kernel if l2norm_k is None else l2norm_k
    if allow_neg_eigval and not use_beta_sigmoid_in_kernel:
        raise ValueError("allow_neg_eigval needs use_beta_sigmoid_in_kernel")
    pre = ((KDA_PRE_L2NORM_Q if lq else 0) | (KDA_PRE_L2NORM_K if lk else 0)
           | (KDA_PRE_BETA_SIGMOID if use_beta_sigmoid_in_kernel else 0)
           | (KDA_PRE_NEG_EIGVAL if allow_neg_eigval else 0))
    return gate, pre


def kda_chunk_fwd_ex(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                     output_final_state=False, scale=None, *, use_gate_in_kernel=False,
                     A_log=None, dt_bias=None, lower_bound=None, use_qk_l2norm_in_kernel=False,
                     l2norm_q=None, l2norm_k=None, use_beta_sigmoid_in_kernel=False,
                     allow_neg_eigval=False, out=None, final_state=None, workspace=None,
                     dev_status=None, events=None):
    """Chunked KDA forward with every option. Returns ``(o, final_state or None)``.

    ``g`` is the float32 per-token log2 decay, or with ``use_gate_in_kernel`` the raw gate
    input (bfloat16 or float32) with ``A_log`` / ``dt_bias`` / ``lower_bound`` as in
    ``kda_chunk_fwd_gated``. ``use_qk_l2norm_in_kernel`` normalises q and k rows in the
    loads (``l2norm_q`` / ``l2norm_k`` set each one separately); ``beta`` goes through a
    sigmoid with ``use_beta_sigmoid_in_kernel``, doubled with ``allow_neg_eigval``.
    ``events``: optional sequence of four HIP event handles (ints), as in the timed entry.
    """
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel)
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    if out is None:
        out = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * 4)(*[int(e) for e in events])
    rc = lib.kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log), _ptr(dt_bias),
                              int(lower_bound is not None),
                              float(lower_bound if lower_bound is not None else 0.0), _ptr(beta),
                              pre, _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out),
                              _ptr(final_state), B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0),
                              64, _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _ptr(dev_status), _stream(dev), ev)
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return out, final_state


def kda_recurrent_fwd_ex(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                         output_final_state=False, scale=None, *, use_gate_in_kernel=False,
                         A_log=None, dt_bias=None, lower_bound=None,
                         use_qk_l2norm_in_kernel=False, l2norm_q=None, l2norm_k=None,
                         use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                         state_layout="kv", output_intermediate_states=False, out=None,
                         final_state=None, intermediate_states=None, dev_status=None):
    """Per-token recurrent KDA forward with every decode option: those of
    ``kda_chunk_fwd_ex``, ``state_layout`` ("kv": states [N, HV, K, V]; "vk": [N, HV, V, K])
    and ``output_intermediate_states`` (the state after every token, float32
    [B*T, HV, K, V] or [B*T, HV, V, K] in the states' layout). Returns
    ``(o, final_state or None)``, plus the intermediate states when requested."""
    lib = load_library()
    if state_layout not in ("kv", "vk"):
        raise ValueError("state_layout must be 'kv' or 'vk'")
    vk = state_layout == "vk"
    h0 = initial_state
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, None if vk else h0, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel)
    sshape = (N, HV, V, K) if vk else (N, HV, K, V)
    if vk and h0 is not None:
        if h0.dtype != torch.float32 or tuple(h0.shape) != sshape:
            raise ValueError(f"initial_state must be float32 {list(sshape)}")
        _check_device([("initial_state", h0)])
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    if out is None:
        out = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty(*sshape, dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    if output_intermediate_states and intermediate_states is None:
        intermediate_states = torch.empty(B * T, HV, *sshape[2:], dtype=torch.float32, device=dev)
    if not output_intermediate_states:
        intermediate_states = None
    rc = lib.kda_recurrent_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log),
                                  _ptr(dt_bias), int(lower_bound is not None),
                                  float(lower_bound if lower_bound is not None else 0.0),
                                  _ptr(beta), pre, KDA_STATE_VK if vk else KDA_STATE_KV, _ptr(h0),
                                  _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state),
                                  _ptr(intermediate_states), B, T, H, HV, K, V, qkv, bdt,
                                  float(scale or 0.0), _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    if output_intermediate_states:
        return out, final_state, intermediate_states
    return out, final_state


def kda_chunk_bwd(q, k, v, g, beta, do, initial_state=None, cu_seqlens=None, dht=None,
                  scale=None, *, want_dh0=True, workspace=None, dev_status=None):
    """Gradients of the chunked forward. ``do`` [B, T, HV, V] in q's dtype is the gradient
    with respect to o, ``dht`` (float32 [N, HV, K, V] or None) with respect to the final
    state. Returns ``(dq, dk, dv, dg, dbeta, dh0)``: dq, dk, dv in q's dtype, dg float32
    (with respect to the per-token log2 decay g), dbeta in beta's dtype, dh0 float32
    [N, HV, K, V] (None unless ``want_dh0``). Rows outside every sequence are zero."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    if tuple(do.shape) != tuple(v.shape) or do.dtype != q.dtype:
        raise ValueError("do must match v's shape and q's dtype")
    if dht is not None and (dht.dtype != torch.float32 or tuple(dht.shape) != (N, HV, K, V)):
        raise ValueError(f"dht must be float32 {[N, HV, K, V]}")
    _check_device([("do", do), ("dht", dht)])
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    dg = torch.zeros(B, T, HV, K, dtype=torch.float32, device=dev)
    dbeta = torch.zeros_like(beta)
    dh0 = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev) if want_dh0 else None
    need = lib.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), N, _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(dg), _ptr(dbeta), _ptr(dh0), B, T, H, HV, K, V, qkv, bdt,
                           float(scale or 0.0), 64, _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _ptr(dev_status),
                           _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return dq, dk, dv, dg, dbeta, dh0


def kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, packed, dtype=KDA_BF16) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, int(bool(packed)), int(dtype)))


def kda_chunk_bwd_ex(q, k, v, g, beta, do, initial_state=None, cu_seqlens=None, dht=None,
                     scale=None, *, use_gate_in_kernel=False, A_log=None, dt_bias=None,
                     lower_bound=None, use_qk_l2norm_in_kernel=False, l2norm_q=None,
                     l2norm_k=None, use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                     want_dh0=True, workspace=None, dev_status=None):
    """Gradients of ``kda_chunk_fwd_ex`` with the same options, with respect to the raw
    inputs. Returns ``(dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias)``; the last two are
    None unless the gate is raw (``ddt_bias`` also needs ``dt_bias``)."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel)
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    if tuple(do.shape) != tuple(v.shape) or do.dtype != q.dtype:
        raise ValueError("do must match v's shape and q's dtype")
    if dht is not None and (dht.dtype != torch.float32 or tuple(dht.shape) != (N, HV, K, V)):
        raise ValueError(f"dht must be float32 {[N, HV, K, V]}")
    _check_device([("do", do), ("dht", dht)])
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    dg = torch.zeros(B, T, HV, K, dtype=torch.float32, device=dev)
    dbeta = torch.zeros_like(beta)
    dh0 = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev) if want_dh0 else None
    dA = torch.empty(HV, dtype=torch.float32, device=dev) if use_gate_in_kernel else None
    ddt = torch.empty(HV * K, dtype=torch.float32, device=dev) if (use_gate_in_kernel and dt_bias is not None) else None
    need = lib.kda_chunk_bwd_ex_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    rc = lib.kda_chunk_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log), _ptr(dt_bias),
                              int(lower_bound is not None),
                              float(lower_bound if lower_bound is not None else 0.0), _ptr(beta), pre,
                              _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(do), _ptr(dht), _ptr(dq),
                              _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(dA), _ptr(ddt),
                              B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0), 64, _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(dev_status),
                              _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return dq, dk, dv, dg, dbeta, dh0, dA, ddt
