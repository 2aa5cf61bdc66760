"""KDA (Kimi Delta Attention) forward on MI355X: a thin Python binding over libkda.so.

The binding only marshals arguments: it checks shapes and dtypes, allocates outputs
and the workspace with PyTorch (device memory), and passes raw pointers plus the
current HIP stream to the C ABI declared in ``include/kda.h``. Every arithmetic step
runs in the library's HIP kernels. There is no CPU fallback: without the built
library on a GPU every call raises.

Entry points (same names as the C ABI):
  kda_chunk_fwd(q, k, v, g, beta, ...)      chunked prefill forward
  kda_chunk_fwd_gated(q, k, v, g_raw, beta, A_log, ...)
                                             the same with the gate activation fused in
  kda_chunk_fwd_ex(q, k, v, g, beta, ...)   every option: fused gate activation, q/k L2
                                             norm and beta sigmoid in the loads, timing events
  kda_recurrent_fwd(q, k, v, g, beta, ...)  per-token recurrent forward (decode)
  kda_recurrent_fwd_ex(q, k, v, g, beta, ...)  the same with the options of kda_chunk_fwd_ex
  kda_chunk_bwd(q, k, v, g, beta, do, ...)  chunked backward: dq, dk, dv, dg, dbeta, dh0
  kda_chunk_bwd_ex(...)                      the same through the fused input options
                                             (raw gate -> dA_log, ddt_bias; q/k norm; beta sigmoid)
  kda_chunk_fwd_train(q, k, v, g, beta, ...) a training forward: o and the final state, with
                                             the backward's checkpoints kept in a workspace
  kda_chunk_bwd_saved(..., do, workspace, ...)  kda_chunk_bwd from that workspace (no recompute)
  kda_chunk_fwd_ex_train / kda_chunk_bwd_ex_saved   the same with kda_chunk_fwd_ex's options
  kda_chunk_fwd_workspace_bytes(...)         workspace size queries (also _bwd_)
  kda_chunk_fwd_noalloc(...)                 kda_chunk_fwd with no allocation at all: the
                                             intermediates live in a per-GPU scratch array
                                             (problems up to kda_noalloc_scratch_bytes())
  kda_last_error()                           reason for the last failure
Every entry point takes ``debug=True`` (except the allocation-free one): wait for the call
and raise KdaDeviceCheckError when a device-side check flagged the inputs.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    KDA_BF16,
    KDA_DEV_BAD_CU_SEQLENS,
    KDA_F32,
    KDA_GATE_LOG2,
    KDA_GATE_RAW_BF16,
    KDA_GATE_RAW_F32,
    KDA_PRE_BETA_SIGMOID,
    KDA_PRE_L2NORM_K,
    KDA_PRE_L2NORM_Q,
    KDA_PRE_NEG_EIGVAL,
    KDA_STATE_KV,
    KDA_STATE_VK,
    KdaDeviceCheckError,
    KdaError,
    kda_chunk_bwd,
    kda_chunk_bwd_ex,
    kda_chunk_bwd_ex_saved,
    kda_chunk_bwd_saved,
    kda_chunk_bwd_workspace_bytes,
    kda_chunk_fwd,
    kda_chunk_fwd_ex,
    kda_chunk_fwd_ex_train,
    kda_chunk_fwd_gated,
    kda_chunk_fwd_noalloc,
    kda_chunk_fwd_train,
    kda_chunk_fwd_workspace_bytes,
    kda_last_error,
    kda_noalloc_scratch_bytes,
    kda_recurrent_fwd,
    kda_recurrent_fwd_ex,
    library_path,
    load_library,
)

__all__ = [
    "kda_chunk_fwd", "kda_chunk_bwd", "kda_chunk_bwd_ex", "kda_chunk_bwd_workspace_bytes", "kda_chunk_fwd_gated", "kda_chunk_fwd_ex", "kda_recurrent_fwd",
    "kda_recurrent_fwd_ex", "kda_chunk_fwd_workspace_bytes",
    "kda_last_error", "KdaError", "KdaDeviceCheckError", "kda_chunk_fwd_noalloc",
    "kda_noalloc_scratch_bytes", "KDA_BF16", "KDA_F32", "KDA_DEV_BAD_CU_SEQLENS", "load_library",
    "library_path", "KDA_GATE_LOG2", "KDA_GATE_RAW_F32", "KDA_GATE_RAW_BF16", "KDA_PRE_L2NORM_Q",
    "KDA_PRE_L2NORM_K", "KDA_PRE_BETA_SIGMOID", "KDA_PRE_NEG_EIGVAL", "KDA_STATE_KV", "KDA_STATE_VK",
]
