"""Seeded synthetic inputs for KDA workloads.

This module only draws random numbers and shapes them; it holds none of the method's
arithmetic. Both the HIP path and the CPU oracle are fed from here (the oracle always
receives the exact tensors the GPU received, copied back to host), so the two never
disagree about their inputs.

Recipe (shared by every workload; draw order q, k, v, gate, beta, initial state):
  * q, k ~ N(0, 1) in fp32, L2-normalised over the key dimension per (token, head),
    then cast to the input dtype;
  * v ~ N(0, 1) cast to the input dtype;
  * gate = log2(sigmoid(x)) in fp32 with x ~ N(2, 1), optionally clamped from below
    (the per-token log2 decay; always <= 0);
  * beta = sigmoid(N(0, 1)) cast to the beta dtype;
  * initial state ~ N(0, 0.05^2) in fp32 (std 0.05) when the workload has one.
Packed (varlen) workloads draw the sequence lengths first.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    dtype: torch.dtype            # q, k, v (and o)
    beta_dtype: torch.dtype
    seed: int
    gate_clamp: Optional[float]   # lower bound on the per-token log2 gate, or None
    h0_std: Optional[float]       # None -> no initial state (zeros)
    final_state: bool
    # packed sequences: number of slots, length range, number of empty slots, tail rows
    n_slots: int = 0
    len_lo: int = 1
    len_hi: int = 1024
    n_empty: int = 0
    decode: bool = False          # one token per sequence (cu = arange)


WORKLOADS = {
    # B=1 T=256 H=HV=2 K=V=64, all fp32, h0 = 0, chunk 64, seed 0
    "tiny": Workload("tiny", 1, 256, 2, 2, 64, 64, torch.float32, torch.float32, 0,
                     None, None, True),
    # B=2 T=4096 H=HV=16 K=V=128 bf16, gate clamped >= -5, h0 ~ N(0, 0.05), final state
    "c2": Workload("c2", 2, 4096, 16, 16, 128, 128, torch.bfloat16, torch.bfloat16, 1,
                   -5.0, 0.05, True),
    # long context: B=1 T=8192 H=16 HV=32 (GVA, 2 value heads per q/k head), h0 = None
    "c3": Workload("c3", 1, 8192, 16, 32, 128, 128, torch.bfloat16, torch.bfloat16, 2,
                   -5.0, None, False),
    # packed: 64 slots, lengths U[1, 1024], 4 repeated offsets (empty), H=HV=16
    "vl": Workload("vl", 1, 0, 16, 16, 128, 128, torch.bfloat16, torch.bfloat16, 3,
                   -5.0, 0.05, True, n_slots=64, len_lo=1, len_hi=1024, n_empty=4),
    # decode: 4096 sequences x 32 heads, one token each, fp32 states in and out
    "dec": Workload("dec", 1, 4096, 32, 32, 128, 128, torch.bfloat16, torch.bfloat16, 4,
                    None, 0.05, True, n_slots=4096, decode=True),
}


def packed_lengths(gen: torch.Generator, w: Workload):
    """Slot lengths for a packed workload: U[len_lo, len_hi], then ``n_empty`` random
    slots set to 0 (repeated offsets)."""
    lens = torch.randint(w.len_lo, w.len_hi + 1, (w.n_slots,), generator=gen)
    if w.n_empty:
        empty = torch.randperm(w.n_slots, generator=gen)[: w.n_empty]
        lens[empty] = 0
    return lens


def make(w: Workload | str, device="cpu", *, T: Optional[int] = None,
         B: Optional[int] = None, seed: Optional[int] = None, tail: int = 64):
    """Draw one workload. Returns a dict with q, k, v, g, beta, initial_state (or None),
    cu_seqlens (int32 or None), N and the workload itself. ``T``/``B``/``seed`` override
    the workload's values (for smaller test instances). For packed workloads the
    physical row count is cu[N] rounded up to a multiple of 64 plus ``tail`` rows that
    belong to no sequence."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    Bn = w.B if B is None else B
    cu = None
    if w.decode:
        N = w.n_slots if T is None else T
        Tn = N
        cu = torch.arange(N + 1, dtype=torch.int32)
    elif w.n_slots:
        cpu_gen = torch.Generator()
        cpu_gen.manual_seed(seed)
        lens = packed_lengths(cpu_gen, w)
        cu = torch.zeros(w.n_slots + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
        N = w.n_slots
        used = int(cu[-1])
        Tn = ((used + 63) // 64) * 64 + tail
    else:
        N = Bn
        Tn = w.T if T is None else T
    H, HV, K, V = w.H, w.HV, w.K, w.V

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    q = randn(Bn, Tn, H, K)
    q = q / q.norm(dim=-1, keepdim=True)
    k = randn(Bn, Tn, H, K)
    k = k / k.norm(dim=-1, keepdim=True)
    v = randn(Bn, Tn, HV, V)
    x = randn(Bn, Tn, HV, K) + 2.0
    g = torch.log2(torch.sigmoid(x))
    if w.gate_clamp is not None:
        g = g.clamp_min(w.gate_clamp)
    beta = torch.sigmoid(randn(Bn, Tn, HV))
    h0 = None
    if w.h0_std is not None:
        h0 = randn(N, HV, K, V) * w.h0_std
    out = dict(
        q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype), g=g.contiguous(),
        beta=beta.to(w.beta_dtype), initial_state=h0,
        cu_seqlens=None if cu is None else cu.to(device), N=N, workload=w,
    )
    return out
