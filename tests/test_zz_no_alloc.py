"""The allocation-free chunked forward (kda_chunk_fwd_noalloc), called through the C ABI,
against kda_chunk_fwd with a caller workspace on the same inputs: two calls in a row on
one GPU, the second smaller, both bitwise equal to the workspace entry point (same
kernels, deterministic) and within the oracle's bound."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_64_amd import inputs
from tests.util import check, log, to_device, valid_rows

pytestmark = pytest.mark.gpu


def _c_noalloc(lib, d, out, ht, status):
    vp = ctypes.c_void_p
    q = d["q"]
    B, T, H, K = q.shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    cu = d["cu_seqlens"]
    N = cu.numel() - 1 if cu is not None else B
    dt = 1 if q.dtype == torch.bfloat16 else 0
    bdt = 1 if d["beta"].dtype == torch.bfloat16 else 0
    p = lambda t: None if t is None else vp(t.data_ptr())
    stream = vp(torch.cuda.current_stream().cuda_stream)
    return lib.kda_chunk_fwd_noalloc(p(q), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]),
                                     p(d["initial_state"]), p(cu), N, p(out), p(ht), B, T, H, HV,
                                     K, V, dt, bdt, 0.0, 64, p(status), stream)


def _case(d, name, dtype):
    import gated_delta_rule_64_amd as kda
    lib = kda.load_library()
    cu = d["cu_seqlens"]
    N = cu.numel() - 1 if cu is not None else d["q"].shape[0]
    HV, K, V = d["v"].shape[2], d["q"].shape[3], d["v"].shape[3]
    need = kda.kda_chunk_fwd_workspace_bytes(*d["q"].shape[:3], HV, K, V, N, cu is not None,
                                             d["q"].dtype)
    assert need <= lib.kda_noalloc_scratch_bytes(), (name, need)
    log(f"[no-alloc {name}] q {tuple(d['q'].shape)} HV={HV} N={N}, workspace {need} bytes")
    o_ref, ht_ref = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                      d["initial_state"], cu, output_final_state=True)
    # NaN sentinels: anything the allocation-free call fails to write shows up
    out = torch.full_like(d["v"], float("nan"))
    ht = torch.full((N, HV, K, V), float("nan"), dtype=torch.float32, device=d["v"].device)
    status = torch.zeros(1, dtype=torch.int32, device=d["v"].device)
    rc = _c_noalloc(lib, d, out, ht, status)
    assert rc == 0, lib.kda_last_error()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    if cu is not None:
        # rows past cu[N] are outside the contract: the reference call left them as
        # torch.empty_like made them, so compare valid rows only
        n = int(cu[-1].item())
        assert torch.equal(out[:, :n], o_ref[:, :n]), "o differs from the workspace entry point"
        assert torch.isnan(out[:, n:].float()).all(), "rows past cu[N] were written"
    else:
        assert torch.equal(out, o_ref), "o differs from the workspace entry point"
    assert torch.equal(ht, ht_ref), "final state differs from the workspace entry point"
    o64, ht64 = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], cu)
    if cu is not None:
        m = valid_rows(cu.cpu(), d["q"].shape[1])
        check("o", out[:, torch.from_numpy(m).to(out.device)], o64[:, m], dtype)
    else:
        check("o", out, o64, dtype)
    check("final_state", ht, ht64, dtype)


def test_noalloc_two_calls_second_smaller():
    # call 1: packed bf16, 9 slots (one empty), ~1.9 k tokens, H=2 HV=8 K=V=128, h0
    w = inputs.Workload("noalloc_packed", 1, 0, 2, 8, 128, 128, torch.bfloat16, torch.bfloat16,
                        31, -5.0, 0.05, True, n_slots=9, len_lo=1, len_hi=400, n_empty=1)
    d = to_device(inputs.make(w))
    _case(d, "packed bf16", torch.bfloat16)
    # call 2, smaller: dense bf16 B=1 T=200 H=2 HV=4 K=V=128, h0
    w2 = inputs.Workload("noalloc_dense", 1, 200, 2, 4, 128, 128, torch.bfloat16, torch.bfloat16,
                         32, -5.0, 0.05, True)
    _case(to_device(inputs.make(w2)), "dense bf16 (smaller)", torch.bfloat16)


def test_noalloc_rejects_oversize_without_enqueueing():
    import gated_delta_rule_64_amd as kda
    lib = kda.load_library()
    d = to_device(inputs.make(inputs.Workload("tiny2", 1, 64, 1, 1, 64, 64, torch.float32,
                                              torch.float32, 33, None, None, True)))
    out = torch.empty_like(d["v"])
    # the sizes of the long-context problem: far beyond the scratch array
    vp = ctypes.c_void_p
    rc = lib.kda_chunk_fwd_noalloc(vp(d["q"].data_ptr()), vp(d["k"].data_ptr()),
                                   vp(d["v"].data_ptr()), vp(d["g"].data_ptr()),
                                   vp(d["beta"].data_ptr()), None, None, 1, vp(out.data_ptr()),
                                   None, 1, 8192, 16, 32, 128, 128, 1, 1, 0.0, 64, None,
                                   vp(torch.cuda.current_stream().cuda_stream))
    assert rc == -5   # KDA_ERR_WORKSPACE
    assert b"allocation-free" in lib.kda_last_error()
