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
        lib.kda_chunk_bwd_saved.restype = i32
        lib.kda_chunk_bwd_saved.argtypes = lib.kda_chunk_bwd.argtypes
        lib.kda_chunk_fwd_train.restype = i32
        lib.kda_chunk_fwd_train.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                            i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                            vp, sz, vp, vp]
        lib.kda_chunk_bwd_ex.restype = i32
        lib.kda_chunk_bwd_ex.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, f32, vp, i32, vp, vp, i32,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                         i32, i32, i32, i32, f32, i32, vp, sz, vp, vp]
        lib.kda_chunk_bwd_ex_saved.restype = i32
        lib.kda_chunk_bwd_ex_saved.argtypes = lib.kda_chunk_bwd_ex.argtypes
        lib.kda_chunk_fwd_ex_train.restype = i32
        lib.kda_chunk_fwd_ex_train.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, f32, vp, i32, vp, vp, i32,
                                               vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                               vp, sz, vp, vp]
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
        lib.kda_chunk_fwd_noalloc.restype = i32
        lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                              i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                              vp, vp]
        lib.kda_noalloc_scratch_bytes.restype = sz
        lib.kda_noalloc_scratch_bytes.argtypes = []
        _lib = lib
        return lib


def kda_last_error() -> str:
    return load_library().kda_last_error().decode()


_F32 = (torch.float32,)
_FLOAT = (torch.bfloat16, torch.float32)


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"{what} has dtype {t.dtype}; the library takes bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_table(rows):
    """Every row is (name, tensor or None, expected shape or None, accepted dtypes or None).
    Absent tensors are skipped; a wrong shape raises ValueError, a wrong dtype TypeError.
    Nothing here looks at devices, so CPU tensors reach these checks too."""
    for name, t, shape, dtypes in rows:
        if t is None:
            continue
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: got shape {tuple(t.shape)}, this problem needs {tuple(shape)}")
        if dtypes is not None and t.dtype not in dtypes:
            names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
            raise TypeError(f"{name}: got dtype {str(t.dtype).replace('torch.', '')}, expected {names}")


def _check_device(tensors):
    """All given tensors contiguous GPU tensors on one device; returns that device."""
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


def _common(q, k, v, g, beta, initial_state, cu_seqlens, raw_gate=False, state_shape=None):
    """Sizes and dtype codes of a forward or backward call, after checking every input
    against the layouts of the C ABI. ``state_shape`` overrides the expected
    initial_state shape (the transposed decode layout)."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and k take [B, T, H, K] and v [B, T, HV, V]")
    B, T, H, K = (int(x) for x in q.shape)
    HV, V = int(v.shape[2]), int(v.shape[3])
    qkv = _dtype_code(q, "q")
    if cu_seqlens is not None:
        _check_table([("cu_seqlens", cu_seqlens, None, (torch.int32,))])
        if cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens: expected a 1-D tensor of N + 1 offsets")
        if B != 1:
            raise ValueError("cu_seqlens packs sequences into one row: B must be 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    bdt = _dtype_code(beta, "beta")
    _check_table([
        ("k", k, (B, T, H, K), (q.dtype,)),
        ("v", v, (B, T, HV, V), (q.dtype,)),
        ("g", g, (B, T, HV, K), _FLOAT if raw_gate else _F32),
        ("beta", beta, (B, T, HV), _FLOAT),
        ("initial_state", initial_state, state_shape or (N, HV, K, V), _F32),
    ])
    dev = _check_device([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                         ("initial_state", initial_state), ("cu_seqlens", cu_seqlens)])
    return B, T, H, HV, K, V, N, qkv, bdt, dev


def _check_buffers(dev, rows, workspace=None, dev_status=None):
    """Caller-supplied output buffers: each (name, tensor, shape, dtype) must match exactly
    and sit contiguous on ``dev`` (the C ABI cannot see tensor sizes, so a wrong buffer
    would be written past its end). The workspace is checked for device and contiguity
    (its size and alignment by the library); dev_status must be an int32 word on dev."""
    _check_table([(n, t, s, (dt,)) for n, t, s, dt in rows])
    if dev_status is not None:
        if dev_status.dtype != torch.int32 or dev_status.numel() < 1:
            raise TypeError("dev_status: expected an int32 tensor with at least one element")
    tensors = [(n, t) for n, t, _, _ in rows] + [("workspace", workspace), ("dev_status", dev_status)]
    for name, t in tensors:
        if t is not None and (not t.is_cuda or t.device != dev):
            raise ValueError(f"{name} must be on {dev}, found {t.device}")
    _check_device(tensors)


class KdaDeviceCheckError(KdaError):
    """Raised in debug mode when a device-side check set a bit of the status word."""

    def __init__(self, status: int):
        reasons = []
        if status & KDA_DEV_BAD_CU_SEQLENS:
            reasons.append("KDA_DEV_BAD_CU_SEQLENS: some packed slot's offsets broke "
                           "0 = cu[0] <= cu[n] <= cu[n+1] <= T (its outputs were left untouched)")
        rest = status & ~KDA_DEV_BAD_CU_SEQLENS
        if rest:
            reasons.append(f"unknown status bits 0x{rest:x}")
        super().__init__(0, "device-side check failed: " + "; ".join(reasons))
        self.status = status


def _debug_status(debug, dev_status, dev):
    """The status word a call writes: in debug mode a fresh zeroed word unless the caller
    gave one."""
    if debug and dev_status is None:
        return torch.zeros(1, dtype=torch.int32, device=dev)
    return dev_status


def _debug_raise(debug, dev_status, dev):
    """Debug mode: wait for the call on the current stream, then raise when any status
    bit is set. Without debug nothing is synchronised."""
    if not debug or dev_status is None:
        return
    torch.cuda.current_stream(dev).synchronize()
    status = int(dev_status.view(-1)[0].item())
    if status:
        raise KdaDeviceCheckError(status)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, packed, dtype=KDA_BF16) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, int(bool(packed)), int(dtype)))


def _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state, state_shape=None):
    """Check the caller's o / final-state buffers (or allocate them)."""
    sshape = state_shape or (N, HV, K, V)
    if not output_final_state:
        final_state = None
    _check_buffers(dev, [("out", out, tuple(v.shape), q.dtype),
                         ("final_state", final_state, sshape, torch.float32)])
    if out is None:
        out = torch.empty_like(v)
    if output_final_state and final_state is None:
        final_state = torch.empty(*sshape, dtype=torch.float32, device=dev)
    return out, final_state


def _chunk_workspace(lib, workspace, dev, B, T, H, HV, K, V, N, packed, qkv):
    _check_buffers(dev, [], workspace=workspace)
    if workspace is None:
        need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, N, int(packed), qkv)
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    return workspace


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                  output_final_state=False, scale=None, *, out=None, final_state=None,
                  workspace=None, dev_status=None, debug=False):
    """Chunked KDA forward. Returns ``(o, final_state or None)``.

    ``out`` / ``final_state`` / ``workspace`` may be given to reuse buffers (each is
    checked against the problem's shape and dtype); ``dev_status`` (int32 [1] GPU tensor)
    receives device-side check flags. ``final_state`` may be ``initial_state`` itself
    (in place). ``debug=True`` waits for the call and raises ``KdaDeviceCheckError``
    when a device-side check flagged the inputs (using a fresh status word unless
    ``dev_status`` is given); without it nothing is synchronised.
    """
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    workspace = _chunk_workspace(lib, workspace, dev, B, T, H, HV, K, V, N, cu_seqlens is not None, qkv)
    _check_buffers(dev, [], dev_status=dev_status)
    dev_status = _debug_status(debug, dev_status, dev)
    rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state), B, T, H, HV, K, V,
                           qkv, bdt, float(scale or 0.0), 64, _ptr(workspace), _nbytes(workspace),
                           _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return out, final_state


def kda_chunk_fwd_noalloc(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                          output_final_state=False, scale=None, *, out, final_state=None,
                          dev_status=None):
    """``kda_chunk_fwd`` through the library's entry point that allocates nothing: the
    caller passes ``out`` (and ``final_state`` when requested); the per-chunk
    intermediates live in the library's per-device scratch array, so problems needing
    more than ``kda_noalloc_scratch_bytes()`` bytes are rejected, and calls that
    overlap on one GPU race on it."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    if out is None or (output_final_state and final_state is None):
        raise ValueError("kda_chunk_fwd_noalloc allocates nothing: pass out (and final_state)")
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    _check_buffers(dev, [], dev_status=dev_status)
    rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out),
                                   _ptr(final_state), B, T, H, HV, K, V, qkv, bdt,
                                   float(scale or 0.0), 64, _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    return out, final_state


def kda_noalloc_scratch_bytes() -> int:
    """Bytes of the per-device scratch array behind ``kda_chunk_fwd_noalloc``."""
    return int(load_library().kda_noalloc_scratch_bytes())


def kda_chunk_fwd_gated(q, k, v, g_raw, beta, A_log, dt_bias=None, lower_bound=None,
                        initial_state=None, cu_seqlens=None, output_final_state=False, scale=None,
                        *, out=None, final_state=None, workspace=None, dev_status=None,
                        debug=False):
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
        raise ValueError(f"A_log: expected {HV} float32 values (one per value head)")
    if dt_bias is not None and (dt_bias.dtype != torch.float32 or dt_bias.numel() != HV * K):
        raise ValueError(f"dt_bias: expected {HV * K} float32 values (one per value head and channel)")
    _check_device([("g_raw", g_raw), ("A_log", A_log), ("dt_bias", dt_bias)])
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    workspace = _chunk_workspace(lib, workspace, dev, B, T, H, HV, K, V, N, cu_seqlens is not None, qkv)
    _check_buffers(dev, [], dev_status=dev_status)
    dev_status = _debug_status(debug, dev_status, dev)
    rc = lib.kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _dtype_code(g_raw, "g_raw"),
                                 _ptr(A_log), _ptr(dt_bias), int(lower_bound is not None),
                                 float(lower_bound if lower_bound is not None else 0.0), _ptr(beta),
                                 _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out),
                                 _ptr(final_state), B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0),
                                 64, _ptr(workspace), _nbytes(workspace), _ptr(dev_status),
                                 _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return out, final_state


def kda_recurrent_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                      output_final_state=False, scale=None, *, out=None, final_state=None,
                      dev_status=None, debug=False):
    """Per-token recurrent KDA forward. Returns ``(o, final_state or None)``; ``out``,
    ``final_state``, ``dev_status`` and ``debug`` as in ``kda_chunk_fwd``."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    _check_buffers(dev, [], dev_status=dev_status)
    dev_status = _debug_status(debug, dev_status, dev)
    rc = lib.kda_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                               _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state), B, T, H, HV, K, V,
                               qkv, bdt, float(scale or 0.0), _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return out, final_state


def _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound, use_qk_l2norm_in_kernel,
             l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel, allow_neg_eigval):
    """The gate code and preprocessing flags of the _ex entry points, with checks."""
    if use_gate_in_kernel:
        gate = KDA_GATE_RAW_BF16 if g.dtype == torch.bfloat16 else KDA_GATE_RAW_F32
        if A_log is None:
            raise ValueError("use_gate_in_kernel needs A_log")
        if A_log.dtype != torch.float32 or A_log.numel() != HV:
            raise ValueError(f"A_log: expected {HV} float32 values (one per value head)")
        if dt_bias is not None and (dt_bias.dtype != torch.float32 or dt_bias.numel() != HV * K):
            raise ValueError(f"dt_bias: expected {HV * K} float32 values (one per value head and channel)")
        _check_device([("g", g), ("A_log", A_log), ("dt_bias", dt_bias)])
    else:
        if A_log is not None or dt_bias is not None or lower_bound is not None:
            raise ValueError("A_log, dt_bias and lower_bound only apply with use_gate_in_kernel")
        gate = KDA_GATE_LOG2
    lq = use_qk_l2norm_in_kernel if l2norm_q is None else l2norm_q
    lk = use_qk_l2norm_in_kernel if l2norm_k is None else l2norm_k
    if allow_neg_eigval and not use_beta_sigmoid_in_kernel:
        raise ValueError("allow_neg_eigval applies to the in-kernel beta sigmoid only")
    pre = ((KDA_PRE_L2NORM_Q if lq else 0) | (KDA_PRE_L2NORM_K if lk else 0)
           | (KDA_PRE_BETA_SIGMOID if use_beta_sigmoid_in_kernel else 0)
           | (KDA_PRE_NEG_EIGVAL if allow_neg_eigval else 0))
    return gate, pre


def kda_chunk_fwd_ex(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                     output_final_state=False, scale=None, *, use_gate_in_kernel=False,
                     A_log=None, dt_bias=None, lower_bound=None, use_qk_l2norm_in_kernel=False,
                     l2norm_q=None, l2norm_k=None, use_beta_sigmoid_in_kernel=False,
                     allow_neg_eigval=False, out=None, final_state=None, workspace=None,
                     dev_status=None, events=None, debug=False):
    """Chunked KDA forward with every option. Returns ``(o, final_state or None)``.

    ``g`` is the float32 per-token log2 decay, or with ``use_gate_in_kernel`` the raw gate
    input (bfloat16 or float32) with ``A_log`` / ``dt_bias`` / ``lower_bound`` as in
    ``kda_chunk_fwd_gated``. ``use_qk_l2norm_in_kernel`` normalises q and k rows in the
    loads (``l2norm_q`` / ``l2norm_k`` set each one separately); ``beta`` goes through a
    sigmoid with ``use_beta_sigmoid_in_kernel``, doubled with ``allow_neg_eigval``.
    ``events``: optional sequence of four HIP event handles (ints), as in the timed entry.
    ``debug`` as in ``kda_chunk_fwd``.
    """
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel)
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    workspace = _chunk_workspace(lib, workspace, dev, B, T, H, HV, K, V, N, cu_seqlens is not None, qkv)
    _check_buffers(dev, [], dev_status=dev_status)
    dev_status = _debug_status(debug, dev_status, dev)
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * 4)(*[int(e) for e in events])
    rc = lib.kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log), _ptr(dt_bias),
                              int(lower_bound is not None),
                              float(lower_bound if lower_bound is not None else 0.0), _ptr(beta),
                              pre, _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out),
                              _ptr(final_state), B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0),
                              64, _ptr(workspace), _nbytes(workspace), _ptr(dev_status),
                              _stream(dev), ev)
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return out, final_state


def kda_recurrent_fwd_ex(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                         output_final_state=False, scale=None, *, use_gate_in_kernel=False,
                         A_log=None, dt_bias=None, lower_bound=None,
                         use_qk_l2norm_in_kernel=False, l2norm_q=None, l2norm_k=None,
                         use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                         state_layout="kv", output_intermediate_states=False, out=None,
                         final_state=None, intermediate_states=None, dev_status=None,
                         debug=False):
    """Per-token recurrent KDA forward with every decode option: those of
    ``kda_chunk_fwd_ex``, ``state_layout`` ("kv": states [N, HV, K, V]; "vk": [N, HV, V, K])
    and ``output_intermediate_states`` (the state after every token, float32
    [B*T, HV, K, V] or [B*T, HV, V, K] in the states' layout). Returns
    ``(o, final_state or None)``, plus the intermediate states when requested."""
    lib = load_library()
    if state_layout not in ("kv", "vk"):
        raise ValueError("state_layout must be 'kv' or 'vk'")
    vk = state_layout == "vk"
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and k take [B, T, H, K] and v [B, T, HV, V]")
    Kq, HVv, Vv = int(q.shape[3]), int(v.shape[2]), int(v.shape[3])
    Nq = (cu_seqlens.numel() - 1) if cu_seqlens is not None else int(q.shape[0])
    sshape = (Nq, HVv, Vv, Kq) if vk else (Nq, HVv, Kq, Vv)
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel, state_shape=sshape)
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state,
                                    state_shape=sshape)
    if not output_intermediate_states:
        intermediate_states = None
    ishape = (B * T, HV, *sshape[2:])
    _check_buffers(dev, [("intermediate_states", intermediate_states, ishape, torch.float32)],
                   dev_status=dev_status)
    if output_intermediate_states and intermediate_states is None:
        intermediate_states = torch.empty(*ishape, dtype=torch.float32, device=dev)
    dev_status = _debug_status(debug, dev_status, dev)
    rc = lib.kda_recurrent_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log),
                                  _ptr(dt_bias), int(lower_bound is not None),
                                  float(lower_bound if lower_bound is not None else 0.0),
                                  _ptr(beta), pre, KDA_STATE_VK if vk else KDA_STATE_KV,
                                  _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out),
                                  _ptr(final_state), _ptr(intermediate_states), B, T, H, HV, K, V,
                                  qkv, bdt, float(scale or 0.0), _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    if output_intermediate_states:
        return out, final_state, intermediate_states
    return out, final_state


def _bwd_inputs(q, v, do, dht, N, HV, K, V, dev):
    _check_table([("do", do, tuple(v.shape), (q.dtype,)),
                  ("dht", dht, (N, HV, K, V), _F32)])
    _check_device([("do", do), ("dht", dht)])


def kda_chunk_bwd(q, k, v, g, beta, do, initial_state=None, cu_seqlens=None, dht=None,
                  scale=None, *, want_dh0=True, workspace=None, dev_status=None, debug=False):
    """Gradients of the chunked forward. ``do`` [B, T, HV, V] in q's dtype is the gradient
    with respect to o, ``dht`` (float32 [N, HV, K, V] or None) with respect to the final
    state. Returns ``(dq, dk, dv, dg, dbeta, dh0)``: dq, dk, dv in q's dtype, dg float32
    (with respect to the per-token log2 decay g), dbeta in beta's dtype, dh0 float32
    [N, HV, K, V] (None unless ``want_dh0``). Rows outside every sequence are zero.
    ``debug`` as in ``kda_chunk_fwd``."""
    return _chunk_bwd(False, q, k, v, g, beta, do, initial_state, cu_seqlens, dht, scale,
                      want_dh0, workspace, dev_status, debug)


def _chunk_bwd(saved, q, k, v, g, beta, do, initial_state, cu_seqlens, dht, scale, want_dh0,
               workspace, dev_status, debug):
    if saved and workspace is None:
        raise ValueError("the backward from saved checkpoints needs the training forward's workspace")
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    _bwd_inputs(q, v, do, dht, N, HV, K, V, dev)
    _check_buffers(dev, [], workspace=workspace, dev_status=dev_status)
    dq = torch.zeros_like(q)
    dk = torch.zeros_like(k)
    dv = torch.zeros_like(v)
    dg = torch.zeros(B, T, HV, K, dtype=torch.float32, device=dev)
    dbeta = torch.zeros_like(beta)
    dh0 = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev) if want_dh0 else None
    if workspace is None:
        need = lib.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    dev_status = _debug_status(debug, dev_status, dev)
    fn = lib.kda_chunk_bwd_saved if saved else lib.kda_chunk_bwd
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
            _ptr(cu_seqlens), N, _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(dg), _ptr(dbeta), _ptr(dh0), B, T, H, HV, K, V, qkv, bdt,
            float(scale or 0.0), 64, _ptr(workspace), _nbytes(workspace),
            _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return dq, dk, dv, dg, dbeta, dh0


def kda_chunk_fwd_train(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                        output_final_state=False, scale=None, *, out=None, final_state=None,
                        workspace=None, dev_status=None, debug=False):
    """Training forward: ``kda_chunk_fwd``'s outputs, with the forward's checkpoints
    for the backward kept in a workspace. Returns ``(o, final_state or None, workspace)``;
    pass the workspace to ``kda_chunk_bwd_saved`` with the same inputs. ``workspace``
    (uint8, at least ``kda_chunk_bwd_workspace_bytes`` bytes) may be given to reuse one."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens)
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    need = int(lib.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_buffers(dev, [], workspace=workspace, dev_status=dev_status)
    dev_status = _debug_status(debug, dev_status, dev)
    rc = lib.kda_chunk_fwd_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                 _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state), B, T, H, HV, K, V,
                                 qkv, bdt, float(scale or 0.0), 64, _ptr(workspace), _nbytes(workspace),
                                 _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return out, final_state, workspace


def kda_chunk_bwd_saved(q, k, v, g, beta, do, workspace, initial_state=None, cu_seqlens=None,
                        dht=None, scale=None, *, want_dh0=True, dev_status=None, debug=False):
    """``kda_chunk_bwd`` from the workspace a ``kda_chunk_fwd_train`` call with the same
    inputs left: the same results, without the forward recompute."""
    return _chunk_bwd(True, q, k, v, g, beta, do, initial_state, cu_seqlens, dht, scale,
                      want_dh0, workspace, dev_status, debug)


def kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, packed, dtype=KDA_BF16) -> int:
    if isinstance(dtype, torch.dtype):
        dtype = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, N, int(bool(packed)), int(dtype)))


def kda_chunk_bwd_ex(q, k, v, g, beta, do, initial_state=None, cu_seqlens=None, dht=None,
                     scale=None, *, use_gate_in_kernel=False, A_log=None, dt_bias=None,
                     lower_bound=None, use_qk_l2norm_in_kernel=False, l2norm_q=None,
                     l2norm_k=None, use_beta_sigmoid_in_kernel=False, allow_neg_eigval=False,
                     want_dh0=True, workspace=None, dev_status=None, debug=False):
    """Gradients of ``kda_chunk_fwd_ex`` with the same options, with respect to the raw
    inputs. Returns ``(dq, dk, dv, dg, dbeta, dh0, dA_log, ddt_bias)``; the last two are
    None unless the gate is raw (``ddt_bias`` also needs ``dt_bias``)."""
    return _chunk_bwd_ex(False, q, k, v, g, beta, do, initial_state, cu_seqlens, dht, scale,
                         use_gate_in_kernel, A_log, dt_bias, lower_bound, use_qk_l2norm_in_kernel,
                         l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel, allow_neg_eigval, want_dh0,
                         workspace, dev_status, debug)


def kda_chunk_bwd_ex_saved(q, k, v, g, beta, do, workspace, initial_state=None, cu_seqlens=None,
                           dht=None, scale=None, *, use_gate_in_kernel=False, A_log=None,
                           dt_bias=None, lower_bound=None, use_qk_l2norm_in_kernel=False,
                           l2norm_q=None, l2norm_k=None, use_beta_sigmoid_in_kernel=False,
                           allow_neg_eigval=False, want_dh0=True, dev_status=None, debug=False):
    """``kda_chunk_bwd_ex`` from the workspace a ``kda_chunk_fwd_ex_train`` call with the
    same inputs and options left: the same results, without the forward recompute."""
    return _chunk_bwd_ex(True, q, k, v, g, beta, do, initial_state, cu_seqlens, dht, scale,
                         use_gate_in_kernel, A_log, dt_bias, lower_bound, use_qk_l2norm_in_kernel,
                         l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel, allow_neg_eigval, want_dh0,
                         workspace, dev_status, debug)


def kda_chunk_fwd_ex_train(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
                           output_final_state=False, scale=None, *, use_gate_in_kernel=False,
                           A_log=None, dt_bias=None, lower_bound=None, use_qk_l2norm_in_kernel=False,
                           l2norm_q=None, l2norm_k=None, use_beta_sigmoid_in_kernel=False,
                           allow_neg_eigval=False, out=None, final_state=None, workspace=None,
                           dev_status=None, debug=False):
    """``kda_chunk_fwd_train`` with the options of ``kda_chunk_fwd_ex``. Returns
    ``(o, final_state or None, workspace)`` for ``kda_chunk_bwd_ex_saved``."""
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel)
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    out, final_state = _fwd_outputs(q, v, N, HV, K, V, dev, out, final_state, output_final_state)
    if workspace is None:
        need = lib.kda_chunk_bwd_ex_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    _check_buffers(dev, [], workspace=workspace, dev_status=dev_status)
    dev_status = _debug_status(debug, dev_status, dev)
    rc = lib.kda_chunk_fwd_ex_train(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log), _ptr(dt_bias),
                                    int(lower_bound is not None),
                                    float(lower_bound if lower_bound is not None else 0.0), _ptr(beta), pre,
                                    _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(out), _ptr(final_state),
                                    B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0), 64, _ptr(workspace),
                                    _nbytes(workspace), _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return out, final_state, workspace


def _chunk_bwd_ex(saved, q, k, v, g, beta, do, initial_state, cu_seqlens, dht, scale,
                  use_gate_in_kernel, A_log, dt_bias, lower_bound, use_qk_l2norm_in_kernel,
                  l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel, allow_neg_eigval, want_dh0,
                  workspace, dev_status, debug):
    if saved and workspace is None:
        raise ValueError("the backward from saved checkpoints needs the training forward's workspace")
    lib = load_library()
    B, T, H, HV, K, V, N, qkv, bdt, dev = _common(q, k, v, g, beta, initial_state, cu_seqlens,
                                                  raw_gate=use_gate_in_kernel)
    gate, pre = _options(g, HV, K, use_gate_in_kernel, A_log, dt_bias, lower_bound,
                         use_qk_l2norm_in_kernel, l2norm_q, l2norm_k, use_beta_sigmoid_in_kernel,
                         allow_neg_eigval)
    _bwd_inputs(q, v, do, dht, N, HV, K, V, dev)
    _check_buffers(dev, [], workspace=workspace, dev_status=dev_status)
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    dg = torch.zeros(B, T, HV, K, dtype=torch.float32, device=dev)
    dbeta = torch.zeros_like(beta)
    dh0 = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev) if want_dh0 else None
    dA = torch.empty(HV, dtype=torch.float32, device=dev) if use_gate_in_kernel else None
    ddt = torch.empty(HV * K, dtype=torch.float32, device=dev) if (use_gate_in_kernel and dt_bias is not None) else None
    if workspace is None:
        need = lib.kda_chunk_bwd_ex_workspace_bytes(B, T, H, HV, K, V, N, int(cu_seqlens is not None), qkv)
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=dev)
    dev_status = _debug_status(debug, dev_status, dev)
    fn = lib.kda_chunk_bwd_ex_saved if saved else lib.kda_chunk_bwd_ex
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), gate, _ptr(A_log), _ptr(dt_bias),
            int(lower_bound is not None),
            float(lower_bound if lower_bound is not None else 0.0), _ptr(beta), pre,
            _ptr(initial_state), _ptr(cu_seqlens), N, _ptr(do), _ptr(dht), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(dA), _ptr(ddt),
            B, T, H, HV, K, V, qkv, bdt, float(scale or 0.0), 64, _ptr(workspace),
            _nbytes(workspace), _ptr(dev_status), _stream(dev))
    if rc != 0:
        raise KdaError(rc, lib.kda_last_error().decode())
    _debug_raise(debug, dev_status, dev)
    return dq, dk, dv, dg, dbeta, dh0, dA, ddt
