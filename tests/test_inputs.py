"""The seeded input generators (CPU tier): determinism and the workload recipe.

Every parity test and the bench draw their inputs here, so a change of draw order, seed
use or recipe would silently change every case; these tests pin the shapes and dtypes
of each workload, the recipe's value ranges, and bitwise reproducibility.
"""
import pytest
import torch

from gated_delta_rule_64_amd import inputs


def _eq(a, b):
    if a is None or b is None:
        return a is None and b is None
    return torch.equal(a, b)


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("c2", {"T": 300}), ("c3", {"T": 200}),
                                     ("vl", {}), ("dec", {"T": 50})])
def test_reproducible_and_seed_sensitive(name, kw):
    a = inputs.make(name, **kw)
    b = inputs.make(name, **kw)
    for key in ("q", "k", "v", "g", "beta", "initial_state", "cu_seqlens"):
        assert _eq(a[key], b[key]), f"{name}: {key} differs between two draws"
    c = inputs.make(name, seed=a["workload"].seed + 1000, **kw)
    assert not torch.equal(a["q"], c["q"]) and not torch.equal(a["g"], c["g"])


@pytest.mark.parametrize("name,kw,shape", [
    ("tiny", {}, (1, 256, 2, 2, 64, 64)),
    ("c2", {"T": 300}, (2, 300, 16, 16, 128, 128)),
    ("c3", {"T": 200}, (1, 200, 16, 32, 128, 128)),
])
def test_dense_shapes_dtypes_and_recipe(name, kw, shape):
    d = inputs.make(name, **kw)
    w = d["workload"]
    B, T, H, HV, K, V = shape
    assert d["q"].shape == (B, T, H, K) and d["k"].shape == (B, T, H, K)
    assert d["v"].shape == (B, T, HV, V) and d["g"].shape == (B, T, HV, K)
    assert d["beta"].shape == (B, T, HV) and d["cu_seqlens"] is None and d["N"] == B
    assert d["q"].dtype == w.dtype and d["beta"].dtype == w.beta_dtype and d["g"].dtype == torch.float32
    # q, k unit rows (up to the input dtype's rounding)
    tol = 1e-5 if w.dtype == torch.float32 else 1e-2
    for t in (d["q"], d["k"]):
        assert (t.float().norm(dim=-1) - 1).abs().max() < tol
    # per-token log2 decay: <= 0, clamped where the workload says so
    assert (d["g"] <= 0).all()
    if w.gate_clamp is not None:
        assert d["g"].min() >= w.gate_clamp
    b = d["beta"].float()
    assert (b > 0).all() and (b < 1).all()
    if w.h0_std is None:
        assert d["initial_state"] is None
    else:
        h0 = d["initial_state"]
        assert h0.shape == (B, HV, K, V) and h0.dtype == torch.float32
        assert abs(float(h0.std()) - w.h0_std) < 0.1 * w.h0_std


def test_packed_workload_offsets():
    d = inputs.make("vl")
    w = d["workload"]
    cu = d["cu_seqlens"]
    assert cu.dtype == torch.int32 and cu.numel() == w.n_slots + 1 and int(cu[0]) == 0
    lens = (cu[1:] - cu[:-1]).long()
    assert (lens >= 0).all() and int((lens == 0).sum()) == w.n_empty
    nz = lens[lens > 0]
    assert int(nz.min()) >= w.len_lo and int(nz.max()) <= w.len_hi
    T = d["q"].shape[1]
    # physical rows: cu[N] rounded up to 64, plus a tail of 64 rows owned by no sequence
    assert T == (int(cu[-1]) + 63) // 64 * 64 + 64
    assert d["initial_state"].shape == (w.n_slots, w.HV, w.K, w.V)


def test_decode_workload_offsets():
    d = inputs.make("dec", T=50)
    cu = d["cu_seqlens"]
    assert torch.equal(cu, torch.arange(51, dtype=torch.int32))
    assert d["q"].shape == (1, 50, 32, 128) and d["N"] == 50
    assert d["initial_state"].shape == (50, 32, 128, 128)
