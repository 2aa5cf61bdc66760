"""Parity of the HIP library with the fp64 oracle on MI355X (marked gpu).

Every case feeds the oracle the exact tensors the GPU received (copied back to host),
and compares element by element: max|err| <= 1e-4 for fp32 inputs, <= 2e-2 * RMS of
the oracle output for bf16 inputs; integer-exact items (empty-slot state, rows outside
every sequence, NULL state vs zeros) are compared bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import chunked as chunked_ref
from gated_delta_rule_64_amd import inputs
from tests.util import E4M3_VALUES, acc_tile_index, check, frag_tile_index, log, to64, to_device, valid_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import gated_delta_rule_64_amd as kda
    kda.load_library()   # raises loudly when the HIP library is missing
    assert torch.cuda.is_available()
    yield


def run(path, d, final=True, scale=None, **kw):
    import gated_delta_rule_64_amd as kda
    fn = kda.kda_chunk_fwd if path == "chunk" else kda.kda_recurrent_fwd
    o, ht = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], d["cu_seqlens"],
               output_final_state=final, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, ht


def oracle_of(d, scale=None):
    return oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                            d["cu_seqlens"], scale)


def small(B, T, H, HV, K, V, dtype, seed, h0=True, gate_lo=None, clamp=-5.0):
    """A seeded case drawn with the workload recipe at custom sizes."""
    w = inputs.Workload("custom", B, T, H, HV, K, V, dtype, dtype, seed, clamp,
                        0.05 if h0 else None, True)
    d = inputs.make(w)
    if gate_lo is not None:
        d["g"] = torch.empty_like(d["g"]).uniform_(gate_lo, 0.0, generator=torch.Generator().manual_seed(seed + 99))
    return to_device(d)


# ------------------------------------------------------------------------------------
# tiny (fp32): both paths, NULL state vs explicit zeros
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_tiny_fp32(path):
    d = to_device(inputs.make("tiny"))
    log(f"[tiny fp32 {path}] B=1 T=256 H=HV=2 K=V=64")
    o, ht = run(path, d)
    o_ref, ht_ref = oracle_of(d)
    check("o", o, o_ref, torch.float32)
    check("final_state", ht, ht_ref, torch.float32)
    z = dict(d, initial_state=torch.zeros(1, 2, 64, 64, device=DEV))
    o2, ht2 = run(path, z)
    assert torch.equal(o, o2) and torch.equal(ht, ht2), "NULL state must equal explicit zeros bitwise"


# ------------------------------------------------------------------------------------
# full-size bf16 configurations
# ------------------------------------------------------------------------------------
def test_chunk_c2_full():
    d = to_device(inputs.make("c2"))
    log("[c2 chunk] B=2 T=4096 H=HV=16 K=V=128 bf16, h0 ~ N(0, 0.05)")
    o, ht = run("chunk", d)
    o_ref, ht_ref = oracle_of(d)
    check("o", o, o_ref, torch.bfloat16)
    check("final_state", ht, ht_ref, torch.bfloat16)


def test_chunk_c3_full():
    d = to_device(inputs.make("c3"))
    log("[c3 chunk] B=1 T=8192 H=16 HV=32 K=V=128 bf16, h0 = None, no final state")
    o, ht = run("chunk", d, final=False)
    assert ht is None
    o_ref, _ = oracle_of(d)
    check("o", o, o_ref, torch.bfloat16)


def test_chunk_varlen_full():
    d = to_device(inputs.make("vl"))
    cu = d["cu_seqlens"].cpu()
    T = d["q"].shape[1]
    log(f"[vl chunk] 64 slots, {int(cu[-1])} tokens, T_phys={T}, H=HV=16 K=V=128 bf16")
    sentinel = torch.full_like(d["v"], float("nan"))
    h0 = d["initial_state"]
    o, ht = run("chunk", d, out=sentinel)
    o_ref, ht_ref = oracle_of(d)
    m = valid_rows(cu, T)
    check("o", o[:, m], o_ref[:, m], torch.bfloat16)
    check("final_state", ht, ht_ref, torch.bfloat16)
    lens = (cu[1:] - cu[:-1]).numpy()
    empty = np.nonzero(lens == 0)[0]
    assert len(empty) == 4
    for n in empty:
        assert torch.equal(ht[n], h0[n]), f"empty slot {n} state must pass through bitwise"
    tail = o[:, ~m]
    assert tail.numel() > 0 and torch.isnan(tail).all(), "rows past the last offset must stay untouched"


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (128, 64)])
def test_chunk_packed_many_chains(K, V):
    """Packed batches with many more chains than CUs (the wide-slice scan instance where
    V = 128): 160 slots of 1..200 tokens (10 empty) x HV = 8 heads with GVA 2, initial
    states, a NaN sentinel tail; every slot against the oracle, empty slots bitwise."""
    w = inputs.Workload("many", 1, 0, 4, 8, K, V, torch.bfloat16, torch.bfloat16, 41, -5.0, 0.05, True,
                        n_slots=160, len_lo=1, len_hi=200, n_empty=10)
    d = to_device(inputs.make(w))
    cu = d["cu_seqlens"].cpu()
    T = d["q"].shape[1]
    log(f"[packed many chains] 160 slots, {int(cu[-1])} tokens, H=4 HV=8 K={K} V={V} bf16")
    o, ht = run("chunk", d, out=torch.full_like(d["v"], float("nan")))
    o_ref, ht_ref = oracle_of(d)
    m = valid_rows(cu, T)
    check("o", o[:, m], o_ref[:, m], torch.bfloat16)
    check("final_state", ht, ht_ref, torch.bfloat16)
    lens = (cu[1:] - cu[:-1]).numpy()
    for n in np.nonzero(lens == 0)[0]:
        assert torch.equal(ht[n], d["initial_state"][n]), f"empty slot {n} state must pass through bitwise"
    assert torch.isnan(o[:, ~m]).all(), "rows past the last offset must stay untouched"


@pytest.mark.parametrize("V,HV", [(128, 32), (64, 64)])
def test_chunk_dense_many_chains(V, HV):
    """Dense batches with exactly enough chains for the wide-slice scan and its compact
    records (chains x V / 32 = 512 blocks): B = 4 sequences of 213 tokens, GVA 4,
    initial and final states, against the oracle; and the same problem one chain short
    of the threshold (the other record layout) must agree with it to the tolerance."""
    K, B, T = 128, 4, 3 * 64 + 21
    d = small(B, T, HV // 4, HV, K, V, torch.bfloat16, seed=43)
    log(f"[dense many chains] B={B} T={T} H={HV // 4} HV={HV} K={K} V={V} bf16, {B * HV} chains")
    o, ht = run("chunk", d)
    o_ref, ht_ref = oracle_of(d)
    check("o", o, o_ref, torch.bfloat16)
    check("final_state", ht, ht_ref, torch.bfloat16)
    # the first 3 sequences alone: 3 x HV chains, below the threshold
    d3 = dict(d, q=d["q"][:3], k=d["k"][:3], v=d["v"][:3], g=d["g"][:3], beta=d["beta"][:3],
              initial_state=d["initial_state"][:3])
    o3, ht3 = run("chunk", d3)
    check("o (narrow slices)", o3, to64(o[:3]), torch.bfloat16, want_rounded=True)
    check("final_state (narrow slices)", ht3, to64(ht[:3]), torch.bfloat16)


def _decode_vs_oracle_batched(d, o, ht, batch=512):
    """Every (sequence, head) pair of a one-token decode against the oracle, run on
    batches of sequences so host memory stays bounded (the fp64 states of all 4096
    sequences would take 17 GB). The bound is the workload's: 2e-2 x RMS over all pairs."""
    from tests.util import half_ulp_bf16
    N = d["cu_seqlens"].numel() - 1
    worst_o = worst_s = 0.0
    ss_o = ss_s = 0.0
    n_o = n_s = 0
    for a in range(0, N, batch):
        idx = torch.arange(a, min(N, a + batch), device=DEV)
        sub = dict(q=d["q"][0, idx].unsqueeze(1), k=d["k"][0, idx].unsqueeze(1),
                   v=d["v"][0, idx].unsqueeze(1), g=d["g"][0, idx].unsqueeze(1),
                   beta=d["beta"][0, idx].unsqueeze(1), initial_state=d["initial_state"][idx],
                   cu_seqlens=None)
        o_ref, ht_ref = oracle_of(sub)
        go = to64(o[0, idx].unsqueeze(1))
        assert np.isfinite(go).all()
        worst_o = max(worst_o, float((np.abs(go - o_ref) - half_ulp_bf16(o_ref)).max()))
        gs = to64(ht[idx])
        worst_s = max(worst_s, float(np.abs(gs - ht_ref).max()))
        ss_o += float((o_ref ** 2).sum()); n_o += o_ref.size
        ss_s += float((ht_ref ** 2).sum()); n_s += ht_ref.size
        del sub, o_ref, ht_ref, go, gs
    bound_o = 2e-2 * (ss_o / n_o) ** 0.5
    bound_s = 2e-2 * (ss_s / n_s) ** 0.5
    log(f"  o: max err beyond output rounding {worst_o:.3e}, bound {bound_o:.3e}, "
        f"ratio {worst_o / bound_o:.3f}  ({n_o} values)")
    log(f"  final_state: max err {worst_s:.3e}, bound {bound_s:.3e}, ratio {worst_s / bound_s:.3f}")
    assert worst_o <= bound_o and worst_s <= bound_s


def test_recurrent_decode_full():
    """The decode workload at full size (4096 sequences x 32 heads: a flat grid of
    262,144 waves): every (sequence, head) pair against the oracle, and bitwise
    determinism of two runs."""
    d = inputs.make("dec", device=DEV)
    log("[dec recurrent] N=4096 HV=32 K=V=128, 1 token each, fp32 states; all pairs vs the oracle")
    o, ht = run("recurrent", d)
    o2, ht2 = run("recurrent", d)
    assert torch.equal(o, o2) and torch.equal(ht, ht2), "decode must be deterministic"
    del o2, ht2
    _decode_vs_oracle_batched(d, o, ht)


def test_retrieval_identity_decode_full():
    """beta = 1 and q = k give o = scale * v whatever the state, for every one of the
    131,072 (sequence, head) pairs of the decode workload: an indexing check of the flat
    grid at full size with no oracle run."""
    d = inputs.make("dec", device=DEV)
    d["q"] = d["k"]
    d["beta"] = torch.ones_like(d["beta"])
    log("[dec retrieval identity] N=4096 HV=32 K=V=128, beta = 1, q = k")
    o, ht = run("recurrent", d)
    want = to64(d["v"]) * 128 ** -0.5
    check("o vs scale*v (all pairs)", o, want, torch.bfloat16)


# ------------------------------------------------------------------------------------
# cross-checks and exact properties
# ------------------------------------------------------------------------------------
def test_chunk_vs_recurrent_bf16():
    d = small(2, 1000, 4, 8, 128, 128, torch.bfloat16, seed=11)
    o1, s1 = run("chunk", d)
    o2, s2 = run("recurrent", d)
    o_ref, s_ref = oracle_of(d)
    check("chunk o", o1, o_ref, torch.bfloat16)
    check("recurrent o", o2, o_ref, torch.bfloat16)
    check("chunk vs recurrent", o1, to64(o2), torch.bfloat16, want_rounded=True)
    check("chunk state", s1, s_ref, torch.bfloat16)
    check("recurrent state", s2, s_ref, torch.bfloat16)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_retrieval_identity_c3_scale(path):
    """beta = 1, q = k: o_t = scale * v_t whatever the history -- an indexing check at the
    long-context size that needs no oracle run."""
    d = to_device(inputs.make("c3"))
    d["q"] = d["k"]
    d["beta"] = torch.ones_like(d["beta"])
    o, _ = run(path, d, final=False)
    want = to64(d["v"]) * 128 ** -0.5
    check("o vs scale*v", o, want, torch.bfloat16)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_gva_equals_repeated_heads(path):
    d = small(1, 300, 2, 6, 128, 128, torch.bfloat16, seed=5)
    o1, s1 = run(path, d)
    r = dict(d, q=d["q"].repeat_interleave(3, dim=2).contiguous(),
             k=d["k"].repeat_interleave(3, dim=2).contiguous())
    o2, s2 = run(path, r)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged_dense(path, dtype):
    """T not a multiple of 64 (short last chunk), several batch rows."""
    for T in (1, 63, 65, 130):
        d = small(3, T, 2, 4, 64, 128, dtype, seed=T)
        o, s = run(path, d)
        o_ref, s_ref = oracle_of(d)
        check(f"T={T} o", o, o_ref, dtype)
        check(f"T={T} state", s, s_ref, dtype)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_packed_edge_lengths(path, dtype):
    lens = [1, 63, 64, 0, 65, 130, 0, 2]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    T = int(cu[-1]) + 40
    d = small(1, T, 2, 2, 128, 64, dtype, seed=3)
    d["cu_seqlens"] = cu.to(DEV)
    h0 = torch.randn(len(lens), 2, 128, 64, generator=torch.Generator().manual_seed(1)).to(DEV) * 0.05
    d["initial_state"] = h0
    out = torch.full_like(d["v"], float("nan"))
    o, s = run(path, d, out=out)
    o_ref, s_ref = oracle_of(d)
    m = valid_rows(cu, T)
    check("o", o[:, m], o_ref[:, m], dtype)
    check("state", s, s_ref, dtype)
    for n, L in enumerate(lens):
        if L == 0:
            assert torch.equal(s[n], h0[n])
    assert torch.isnan(o[:, ~m]).all()


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_packed_equals_dense_runs(path):
    lens = [200, 64, 17]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    d = small(1, int(cu[-1]), 4, 4, 128, 128, torch.bfloat16, seed=8)
    d["cu_seqlens"] = cu.to(DEV)
    d["initial_state"] = torch.randn(3, 4, 128, 128, generator=torch.Generator().manual_seed(2)).to(DEV) * 0.05
    o, s = run(path, d)
    for n in range(3):
        a, b = int(cu[n]), int(cu[n + 1])
        sub = dict(q=d["q"][:, a:b].contiguous(), k=d["k"][:, a:b].contiguous(), v=d["v"][:, a:b].contiguous(),
                   g=d["g"][:, a:b].contiguous(), beta=d["beta"][:, a:b].contiguous(),
                   initial_state=d["initial_state"][n:n + 1].contiguous(), cu_seqlens=None)
        od, sd = run(path, sub)
        # chunks restart at every sequence start, so packed and dense runs do the same work
        assert torch.equal(o[:, a:b], od), n
        assert torch.equal(s[n], sd[0]), n


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_invalid_cu_seqlens_flagged_not_faulting(path):
    import gated_delta_rule_64_amd as kda
    T = 300
    d = small(1, T, 2, 2, 128, 128, torch.bfloat16, seed=4)
    h0 = torch.randn(3, 2, 128, 128, generator=torch.Generator().manual_seed(3)).to(DEV) * 0.05
    d["initial_state"] = h0
    for bad in ([0, 100, 50, 200], [5, 100, 150, 200], [0, 100, 200, 400], [0, -7, 100, 200]):
        d["cu_seqlens"] = torch.tensor(bad, dtype=torch.int32, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        fs = torch.full((3, 2, 128, 128), 7.0, device=DEV)
        run(path, d, dev_status=status, final_state=fs)
        assert int(status.item()) & kda.KDA_DEV_BAD_CU_SEQLENS, bad
        for n in range(3):
            a, b = bad[n], bad[n + 1]
            if not (0 <= a <= b <= T and (n > 0 or a == 0)):
                assert (fs[n] == 7.0).all(), f"slot {n} of {bad} must be left untouched"
    good = torch.tensor([0, 100, 150, 300], dtype=torch.int32, device=DEV)
    d["cu_seqlens"] = good
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    run(path, d, dev_status=status)
    assert int(status.item()) == 0


@pytest.mark.parametrize("path", ["chunk", "recurrent", "chunk_bwd"])
def test_debug_mode_raises_on_bad_offsets(path):
    """debug=True waits for the call and raises KdaDeviceCheckError when the device-side
    offset check fires (a fresh status word when the caller gives none); well-formed
    offsets pass, and without debug the same malformed call returns normally."""
    import gated_delta_rule_64_amd as kda
    T = 300
    d = small(1, T, 2, 2, 128, 128, torch.bfloat16, seed=4)
    d["initial_state"] = torch.randn(3, 2, 128, 128, generator=torch.Generator().manual_seed(3)).to(DEV) * 0.05
    do = torch.randn(1, T, 2, 128, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)

    def call(cu, **kw):
        args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
        if path == "chunk_bwd":
            return kda.kda_chunk_bwd(*args, do, d["initial_state"], cu, **kw)
        fn = kda.kda_chunk_fwd if path == "chunk" else kda.kda_recurrent_fwd
        return fn(*args, d["initial_state"], cu, output_final_state=True, **kw)

    bad = torch.tensor([0, 100, 50, 200], dtype=torch.int32, device=DEV)
    good = torch.tensor([0, 100, 150, 300], dtype=torch.int32, device=DEV)
    with pytest.raises(kda.KdaDeviceCheckError) as e:
        call(bad, debug=True)
    assert e.value.status & kda.KDA_DEV_BAD_CU_SEQLENS and isinstance(e.value, kda.KdaError)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    with pytest.raises(kda.KdaDeviceCheckError):
        call(bad, debug=True, dev_status=status)
    assert int(status.item()) & kda.KDA_DEV_BAD_CU_SEQLENS
    call(good, debug=True)
    call(bad)                 # no debug: no exception, nothing synchronised
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_inplace_state_and_null_final(path):
    d = small(2, 129, 2, 2, 128, 128, torch.bfloat16, seed=6)
    o1, s1 = run(path, d)
    st = d["initial_state"].clone()
    o2, s2 = run(path, dict(d, initial_state=st), final_state=st)
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, st)
    o3, s3 = run(path, d, final=False)
    assert s3 is None and torch.equal(o1, o3)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_deterministic(path):
    d = small(2, 700, 4, 8, 128, 128, torch.bfloat16, seed=9)
    a = run(path, d)
    b = run(path, d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_split_resume(path):
    d = small(1, 512, 2, 4, 128, 128, torch.bfloat16, seed=12)
    o, s = run(path, d)
    t1 = 192

    def part(a, b, h0):
        return dict(q=d["q"][:, a:b].contiguous(), k=d["k"][:, a:b].contiguous(),
                    v=d["v"][:, a:b].contiguous(), g=d["g"][:, a:b].contiguous(),
                    beta=d["beta"][:, a:b].contiguous(), initial_state=h0, cu_seqlens=None)
    oa, sa = run(path, part(0, t1, d["initial_state"]))
    ob, sb = run(path, part(t1, 512, sa))
    check("resumed o", torch.cat([oa, ob], 1), to64(o), torch.bfloat16)
    check("resumed state", sb, to64(s), torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_extreme_decay(path, dtype):
    """Per-token gates down to -15 (mixed with mild ones): the chunk path's steep-decay
    branch (exact diagonal blocks) must stay finite and within tolerance."""
    d = small(1, 256, 2, 2, 128, 128, dtype, seed=13, gate_lo=-15.0)
    g = d["g"].clone()
    g[:, 64:128] = -15.0
    d["g"] = g
    o, s = run(path, d)
    o_ref, s_ref = oracle_of(d)
    check("o", o, o_ref, dtype)
    check("state", s, s_ref, dtype)


@pytest.mark.parametrize("seed", [0, 1])
def test_chunk_stage2_records_fp32(seed):
    """The intra kernel's per-chunk records (Aqk, w, u, qg, kg^T, 2^G) against the fp64
    chunk algebra, fp32 inputs."""
    import gated_delta_rule_64_amd as kda
    d = small(1, 128 + 37, 2, 2, 64, 64, torch.float32, seed=seed)
    B, T, H, K = d["q"].shape
    HV, V = 2, 64
    nbytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, B, 0, torch.float32)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    run("chunk", d, workspace=ws)
    _, _, stages = chunked_ref.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                                       None, None, return_stages=True)
    rec = (64 * K * 4 * 3 + 64 * V * 4 + 64 * 64 * 4 + 4 * K + 255) // 256 * 256
    raw = ws.cpu()
    NT = (T + 63) // 64
    sched = (((3 * B + 1) * 4 + 15) // 16 * 16 + B * NT * 8 + 255) // 256 * 256
    for st in stages:
        hv, c = st["hv"], st["start"] // 64
        base = sched + (hv * NT + c) * rec
        L = st["length"]

        def flat(off, n):
            return raw[base + off: base + off + 4 * n].view(torch.float32).double().numpy()

        def frag(off, R, KC):   # fp32 path: 4-wide contraction steps, 1 value per lane
            return flat(off, R * KC)[frag_tile_index(R, KC, 4, 1)]
        # record layout (fp32 path): w | qg | kg^T | Aqk (fragment order) | u (accumulator
        # order) | 2^G, after the schedule
        off = 0
        w = frag(off, 64, K); off += 64 * K * 4
        qg = frag(off, 64, K); off += 64 * K * 4
        kgT = frag(off, K, 64); off += K * 64 * 4
        aqk = frag(off, 64, 64); off += 64 * 64 * 4
        u = flat(off, 64 * V)[acc_tile_index(64, V)]; off += 64 * V * 4
        eg = flat(off, K)
        scale = K ** -0.5
        for name, got, want in (("Aqk", aqk[:L, :L], st["Aqk"]), ("w", w[:L], st["w"]),
                                ("u", u[:L], st["u"]), ("qg", qg[:L], scale * st["qg"]),
                                ("kgT", kgT[:, :L], st["kg"].T), ("2^G", eg, np.exp2(st["G"]))):
            err = np.abs(got - want).max()
            assert err <= 2e-5 * max(1.0, np.abs(want).max()), (name, hv, c, err)
        assert np.abs(aqk[L:]).max(initial=0) == 0 and np.abs(w[L:]).max(initial=0) == 0


@pytest.mark.parametrize("HV", [4, 128], ids=["bf16-residuals", "fp8-residuals"])
@pytest.mark.parametrize("steep", [False, True])
def test_chunk_stage2_records_bf16(steep, HV):
    """The bf16 intra kernel's records against the fp64 chunk algebra of the same (bf16)
    inputs, K = V = 128, two q/k heads shared by HV value heads, a short last chunk. Each
    stored quantity is decoded from its layout (hi + lo where it carries a residual). With
    4 value heads the records hold bf16 residual tiles; with 128 (chains x V / 32 = 512
    scan blocks) they are compact, the residuals fp8 tiles with per-lane scale words.
    ``steep`` puts gates down to -15 into the second chunk so its diagonal blocks take
    the exact one-sided branch."""
    import gated_delta_rule_64_amd as kda
    K = V = 128
    compact = HV == 128
    d = small(1, 128 + 37, 2, HV, K, V, torch.bfloat16, seed=21)
    if steep:
        g = d["g"].clone()
        g[:, 64:128, 1] = -15.0
        d["g"] = g
    B, T, H, _ = d["q"].shape
    nbytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, B, 0, torch.bfloat16)
    # zero-filled: the forward does not write Aqk's all-zero fragments (rows 0-31,
    # columns 32-63), which its scan never reads
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    run("chunk", d, workspace=ws)
    _, _, stages = chunked_ref.chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                                       None, None, return_stages=True)
    # record: w, qg, kg^T, Aqk (bf16, fragment order), then either their residuals as a
    # second bf16 tile each (in place after each) or, compact, the fp8 residuals of qg,
    # kg^T, Aqk (same order, a byte per value) and their scale words [bands][64]; u; 2^G
    if compact:
        lo_at = 64 * K * 2 * 3 + 64 * 64 * 2
        sc_at = lo_at + 2 * 64 * K + 64 * 64
        u_at = sc_at + (4 + K // 16 + 4) * 64 * 4
    else:
        u_at = 64 * K * 2 * 5 + 64 * 64 * 2 * 2
    rec = (u_at + 64 * V * 4 + 4 * K + 255) // 256 * 256
    assert nbytes == (((3 * B + 1) * 4 + 15) // 16 * 16 + B * ((T + 63) // 64) * 8 + B * 4 + 255) // 256 * 256 \
        + HV * B * ((T + 63) // 64) * rec
    raw = ws.cpu()
    NT = (T + 63) // 64
    sched = (((3 * B + 1) * 4 + 15) // 16 * 16 + B * NT * 8 + 255) // 256 * 256
    scale = K ** -0.5
    # relative bounds: single-bf16 tiles (w) and the fp32 u built from the bf16 T beta
    # carry bf16 rounding; hi + lo in bf16 is fp32-level, a bf16 tile plus its fp8
    # residual carries about 12 bits of each value relative to the largest of the eight
    # its lane holds; 2^G is fp32
    split = 2e-4 if compact else 2e-5
    bounds = {"Aqk": split, "w": 1e-2, "u": 1e-2, "qg": split, "kgT": split, "2^G": 2e-5}
    worst = {}
    for st in stages:
        hv, c = st["hv"], st["start"] // 64
        base = sched + (hv * NT + c) * rec
        L = st["length"]

        def bf(off, n):
            return raw[base + off: base + off + 2 * n].view(torch.bfloat16).double().numpy()

        def frag(off, R, KC):
            return bf(off, R * KC)[frag_tile_index(R, KC, 32, 8)]

        def lo8(off, sc_off, R, KC):
            codes = raw[base + off: base + off + R * KC].numpy()
            vals = E4M3_VALUES[codes][frag_tile_index(R, KC, 32, 8)]
            words = raw[base + sc_off: base + sc_off + (R // 16) * 64 * 4].numpy().view(np.uint32)
            row, col = np.arange(R)[:, None], np.arange(KC)[None, :]
            lane = row % 16 + 16 * ((col % 32) // 8)
            sbyte = (words[(row // 16) * 64 + lane] >> (8 * (col // 32)).astype(np.uint32)) & 0xFF
            return vals * np.exp2(sbyte.astype(np.float64) - 127.0)
        if compact:
            w = frag(0, 64, K)
            qg = frag(64 * K * 2, 64, K) + lo8(lo_at, sc_at, 64, K)
            kgT = frag(2 * 64 * K * 2, K, 64) + lo8(lo_at + 64 * K, sc_at + 4 * 64 * 4, K, 64)
            aqk = frag(3 * 64 * K * 2, 64, 64) + lo8(lo_at + 2 * 64 * K, sc_at + (4 + K // 16) * 64 * 4, 64, 64)
        else:
            off = 0
            w = frag(off, 64, K); off += 64 * K * 2
            qg = frag(off, 64, K) + frag(off + 64 * K * 2, 64, K); off += 2 * 64 * K * 2
            kgT = frag(off, K, 64) + frag(off + K * 64 * 2, K, 64); off += 2 * K * 64 * 2
            aqk = frag(off, 64, 64) + frag(off + 64 * 64 * 2, 64, 64)
        u = raw[base + u_at: base + u_at + 4 * 64 * V].view(torch.float32).double().numpy()[acc_tile_index(64, V)]
        off = u_at + 64 * V * 4
        eg = raw[base + off: base + off + 4 * K].view(torch.float32).double().numpy()
        for name, got, want in (("Aqk", aqk[:L, :L], st["Aqk"]), ("w", w[:L], st["w"]),
                                ("u", u[:L], st["u"]), ("qg", qg[:L], scale * st["qg"]),
                                ("kgT", kgT[:, :L], st["kg"].T), ("2^G", eg, np.exp2(st["G"]))):
            rel = np.abs(got - want).max() / max(1e-30, np.abs(want).max())
            worst[name] = max(worst.get(name, 0.0), rel)
            if rel > bounds[name]:
                bad = np.unravel_index(np.argmax(np.abs(got - want)), got.shape)
                log(f"  {name} hv={hv} chunk={c}: rel err {rel:.3e} at {bad}: got {got[bad]:.6e} want {want[bad]:.6e}")
        assert np.abs(aqk[L:]).max(initial=0) == 0 and np.abs(w[L:]).max(initial=0) == 0
        assert np.abs(qg[L:]).max(initial=0) == 0 and np.abs(kgT[:, L:]).max(initial=0) == 0
    log("  worst relative error per record: " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    for name, b in bounds.items():
        assert worst[name] <= b, (name, worst[name], b)


# ------------------------------------------------------------------------------------
# gate activation fused into Stage 1 (kda_chunk_fwd_gated)
# ------------------------------------------------------------------------------------
def _gate_params(B, T, HV, K, gdt, seed):
    """Raw gate input N(0, 2^2) in gdt, A_log = log(U[1, 2]) per head, dt_bias N(0, 0.5^2)."""
    gen = torch.Generator().manual_seed(seed)
    g_raw = torch.randn(B, T, HV, K, generator=gen).mul(2.0).to(gdt)
    A_log = torch.rand(HV, generator=gen).add(1.0).log()
    dt_bias = torch.randn(HV * K, generator=gen).mul(0.5)
    return g_raw.to(DEV), A_log.to(DEV), dt_bias.to(DEV)


def _gated_oracle(d, g_raw, A_log, dt_bias, bound):
    g2 = oracle.gate_activation(g_raw, A_log, dt_bias, bound)
    return oracle.recurrent(d["q"], d["k"], d["v"], g2, d["beta"], d["initial_state"], d["cu_seqlens"])


@pytest.mark.parametrize("bound", [None, -3.0])
@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32])
def test_gated_chunk_bf16(gdt, bound):
    """bf16 q/k/v, raw gates in gdt: the fused activation against the oracle's fp64
    activation followed by the recurrence (a short last chunk included)."""
    import gated_delta_rule_64_amd as kda
    d = small(1, 300, 2, 4, 128, 128, torch.bfloat16, seed=31)
    g_raw, A_log, dt_bias = _gate_params(1, 300, 4, 128, gdt, seed=77)
    log(f"[gated chunk] B1 T300 H2 HV4 K=V=128 bf16, raw gate {gdt}, lower_bound={bound}")
    o, ht = kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], g_raw, d["beta"], A_log, dt_bias, bound,
                                    d["initial_state"], None, output_final_state=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = _gated_oracle(d, g_raw, A_log, dt_bias, bound)
    check("o", o, o_ref, torch.bfloat16)
    check("state", ht, ht_ref, torch.bfloat16)


def test_gated_chunk_fp32_and_no_dt_bias():
    """fp32 everything (the fp32 Stage 1+2 kernel), dt_bias omitted: 1e-4 max-abs."""
    import gated_delta_rule_64_amd as kda
    d = small(1, 200, 2, 2, 64, 64, torch.float32, seed=32)
    g_raw, A_log, _ = _gate_params(1, 200, 2, 64, torch.float32, seed=78)
    o, ht = kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], g_raw, d["beta"], A_log, None, None,
                                    d["initial_state"], None, output_final_state=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = _gated_oracle(d, g_raw, A_log, None, None)
    check("o", o, o_ref, torch.float32)
    check("state", ht, ht_ref, torch.float32)


def test_gated_chunk_packed():
    """Packed sequences (one empty slot, a tail) with fused gates: o on valid rows, the
    tail untouched, every final state."""
    import gated_delta_rule_64_amd as kda
    lens = [130, 0, 64, 37, 200]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    Tp = cu[-1] + 40
    d = small(1, Tp, 2, 4, 128, 128, torch.bfloat16, seed=33)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=DEV)
    d["initial_state"] = torch.randn(len(lens), 4, 128, 128, generator=torch.Generator().manual_seed(5)).mul(0.05).to(DEV)
    g_raw, A_log, dt_bias = _gate_params(1, Tp, 4, 128, torch.bfloat16, seed=79)
    out = torch.full_like(d["v"], float("nan"))
    o, ht = kda.kda_chunk_fwd_gated(d["q"], d["k"], d["v"], g_raw, d["beta"], A_log, dt_bias, -6.0,
                                    d["initial_state"], d["cu_seqlens"], output_final_state=True,
                                    out=out)
    torch.cuda.synchronize()
    o_ref, ht_ref = _gated_oracle(d, g_raw, A_log, dt_bias, -6.0)
    rows = valid_rows(cu, Tp)
    check("o", o[0][torch.from_numpy(rows).to(DEV)], o_ref[0][rows], torch.bfloat16)
    assert torch.isnan(o[0, cu[-1]:].float()).all(), "tail must stay untouched"
    check("state", ht, ht_ref, torch.bfloat16)
    assert torch.equal(ht[1], d["initial_state"][1]), "empty slot passes its state bitwise"


@pytest.mark.parametrize("steep", [False, True])
@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_head_dims(dtype, K, V, steep):
    """Every (K, V) the chunk kernels are built for, both input precisions; ``steep`` puts
    per-token gates of -15 on one chunk of one head (the exact diagonal-block path)."""
    d = small(1, 200, 2, 4, K, V, dtype, seed=40 + K + V)
    if steep:
        g = d["g"].clone()
        g[:, 64:128, 2] = -15.0
        d["g"] = g
    log(f"[head dims] K={K} V={V} {dtype} steep={steep}")
    o, s = run("chunk", d)
    o_ref, s_ref = oracle_of(d)
    check("o", o, o_ref, dtype)
    check("state", s, s_ref, dtype)


# ------------------------------------------------------------------------------------
# input preprocessing fused into the loads: q / k L2 normalisation, beta sigmoid (x2)
# ------------------------------------------------------------------------------------
PRE_CASES = [  # (l2norm_q, l2norm_k, beta sigmoid, allow_neg_eigval)
    (True, True, True, False),
    (True, False, True, True),
    (False, True, False, False),
    (False, False, True, True),
]


def _raw_inputs(d, seed, lq=True, lk=True, sig=True, zero_rows=True, span=3.0):
    """Inputs for the preprocessing flags: q (lq) and k (lk) un-normalised, every
    (token, head) row of the unit-norm draw times 10^U[-span, span] with about 2% of rows
    zero; beta (sig) replaced by pre-activations N(0, 2^2) in beta's dtype. Tensors whose
    preprocessing is off keep the recipe's values (a delta rule on un-normalised keys or
    beta outside (0, 2) diverges)."""
    gen = torch.Generator().manual_seed(seed)

    def scaled(x):
        B, T, H, _ = x.shape
        s = torch.pow(10.0, torch.empty(B, T, H, 1).uniform_(-span, span, generator=gen))
        y = x.cpu().float() * s
        if zero_rows:
            y = torch.where(torch.rand(B, T, H, 1, generator=gen) < 0.02, torch.zeros_like(y), y)
        return y.to(x.dtype).to(DEV)

    q = scaled(d["q"])
    k = scaled(d["k"])
    logits = torch.randn(tuple(d["beta"].shape), generator=gen).mul(2.0).to(d["beta"].dtype).to(DEV)
    return dict(d, q=q if lq else d["q"], k=k if lk else d["k"], beta=logits if sig else d["beta"])


def _pre_oracle(r, lq, lk, sig, neg, g2=None):
    """The oracle's preprocessing (fp64) followed by the recurrence."""
    q = oracle.l2norm(r["q"]) if lq else r["q"]
    k = oracle.l2norm(r["k"]) if lk else r["k"]
    beta = oracle.beta_sigmoid(r["beta"], neg) if sig else r["beta"]
    return oracle.recurrent(q, k, r["v"], r["g"] if g2 is None else g2, beta, r["initial_state"],
                            r["cu_seqlens"])


def _run_ex(path, r, lq, lk, sig, neg, **kw):
    import gated_delta_rule_64_amd as kda
    fn = kda.kda_chunk_fwd_ex if path == "chunk" else kda.kda_recurrent_fwd_ex
    o, ht = fn(r["q"], r["k"], r["v"], kw.pop("g", r["g"]), r["beta"], r["initial_state"],
               r["cu_seqlens"], output_final_state=True, l2norm_q=lq, l2norm_k=lk,
               use_beta_sigmoid_in_kernel=sig, allow_neg_eigval=neg, **kw)
    torch.cuda.synchronize()
    return o, ht


@pytest.mark.parametrize("lq,lk,sig,neg", PRE_CASES, ids=lambda x: str(int(x)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_preprocess(path, dtype, lq, lk, sig, neg):
    """Normalisation and beta activation in the loads against the oracle's fp64
    preprocessing: row scales over six decades, zero rows, a short last chunk."""
    d = small(1, 230, 2, 4, 128, 128, dtype, seed=50)
    r = _raw_inputs(d, 51, lq, lk, sig)
    log(f"[preprocess {path}] {dtype} l2norm_q={lq} l2norm_k={lk} sigmoid={sig} neg_eigval={neg}")
    o, ht = _run_ex(path, r, lq, lk, sig, neg)
    o_ref, ht_ref = _pre_oracle(r, lq, lk, sig, neg)
    check("o", o, o_ref, dtype)
    check("state", ht, ht_ref, dtype)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_preprocess_fused_equals_explicit(path):
    """bf16 inputs with the fused normalisation and beta activation against the explicit
    route: q / k normalised and beta activated beforehand in fp32 torch, then the plain
    fp32 call (v widened exactly). Within the bf16 bound of the explicit result."""
    d = small(1, 200, 2, 4, 128, 128, torch.bfloat16, seed=52)
    r = _raw_inputs(d, 53)
    o, ht = _run_ex(path, r, True, True, True, True)

    def norm(x):
        xf = x.float()
        return xf / torch.sqrt((xf * xf).sum(-1, keepdim=True) + 1e-6)

    e = dict(r, q=norm(r["q"]), k=norm(r["k"]), v=r["v"].float(),
             beta=torch.sigmoid(r["beta"].float()) * 2.0)
    o2, ht2 = run(path, e)
    check("o vs explicit", o, to64(o2), torch.bfloat16)
    check("state vs explicit", ht, to64(ht2), torch.bfloat16)


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_preprocess_with_gate_packed(path):
    """Every option at once in packed mode: raw bf16 gate with dt_bias and a lower bound,
    both normalisations, beta = 2 sigmoid; an empty slot and a tail of unowned rows."""
    lens = [130, 0, 64, 37, 200]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    Tp = cu[-1] + 40
    d = small(1, Tp, 2, 4, 128, 128, torch.bfloat16, seed=54)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=DEV)
    d["initial_state"] = torch.randn(len(lens), 4, 128, 128, generator=torch.Generator().manual_seed(6)).mul(0.05).to(DEV)
    r = _raw_inputs(d, 55)
    g_raw, A_log, dt_bias = _gate_params(1, Tp, 4, 128, torch.bfloat16, seed=80)
    out = torch.full_like(r["v"], float("nan"))
    log(f"[preprocess + gate, packed {path}] lens={lens}")
    o, ht = _run_ex(path, r, True, True, True, True, g=g_raw, use_gate_in_kernel=True,
                    A_log=A_log, dt_bias=dt_bias, lower_bound=-6.0, out=out)
    g2 = oracle.gate_activation(g_raw, A_log, dt_bias, -6.0)
    o_ref, ht_ref = _pre_oracle(r, True, True, True, True, g2=g2)
    rows = valid_rows(cu, Tp)
    check("o", o[0][torch.from_numpy(rows).to(DEV)], o_ref[0][rows], torch.bfloat16)
    assert torch.isnan(o[0, cu[-1]:].float()).all(), "tail must stay untouched"
    check("state", ht, ht_ref, torch.bfloat16)
    assert torch.equal(ht[1], d["initial_state"][1]), "empty slot passes its state bitwise"


def test_preprocess_c3_full():
    """The long-context workload (B=1 T=8192 H=16 HV=32 K=V=128 bf16) with every fusion
    on, as the benchmark's fused-input leg runs it: un-normalised q / k, beta logits,
    raw bf16 gates with dt_bias. Whole output against the oracle."""
    import gated_delta_rule_64_amd as kda
    d = to_device(inputs.make("c3"))
    r = _raw_inputs(d, 56, zero_rows=False)
    g_raw, A_log, dt_bias = _gate_params(1, 8192, 32, 128, torch.bfloat16, seed=81)
    log("[c3 chunk, all input fusions] B=1 T=8192 H=16 HV=32 K=V=128 bf16")
    o, ht = kda.kda_chunk_fwd_ex(r["q"], r["k"], r["v"], g_raw, r["beta"], None, None,
                                 use_gate_in_kernel=True, A_log=A_log, dt_bias=dt_bias,
                                 use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True,
                                 allow_neg_eigval=True)
    torch.cuda.synchronize()
    assert ht is None
    g2 = oracle.gate_activation(g_raw, A_log, dt_bias, None)
    o_ref, _ = _pre_oracle(dict(r, initial_state=None, cu_seqlens=None), True, True, True, True, g2=g2)
    check("o", o, o_ref, torch.bfloat16)


# ------------------------------------------------------------------------------------
# chunked backward: every gradient against the fp64 adjoint oracle
# ------------------------------------------------------------------------------------
def _bwd_inputs(d, seed, dht=True):
    """Output gradient N(0, 1) in q's dtype; final-state gradient N(0, 0.1^2) fp32."""
    gen = torch.Generator().manual_seed(seed)
    do = torch.randn(tuple(d["v"].shape), generator=gen).to(d["v"].dtype).to(DEV)
    N = d["initial_state"].shape[0] if d["initial_state"] is not None else (
        d["cu_seqlens"].numel() - 1 if d["cu_seqlens"] is not None else d["q"].shape[0])
    HV, K, V = d["v"].shape[2], d["q"].shape[3], d["v"].shape[3]
    dht_t = torch.randn(N, HV, K, V, generator=gen).mul(0.1).to(DEV) if dht else None
    return do, dht_t


def _check_bwd(d, do, dht, dtype, rows=None, label=""):
    import gated_delta_rule_64_amd as kda
    got = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["initial_state"],
                            d["cu_seqlens"], dht)
    torch.cuda.synchronize()
    ref = oracle.recurrent_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["initial_state"],
                               d["cu_seqlens"], dht)
    names = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]
    for name, x, y in zip(names, got, ref):
        if rows is not None and name != "dh0":
            x, y = x[:, rows], y[:, rows]
        # fp32 gradients (dg, dh0) of bf16 inputs are held to the bf16 bound as well
        check(f"{label}{name}", x, y, dtype)
    return got, ref


def test_chunk_bwd_deterministic():
    """The backward's gradients are the same bits on every call: its row and channel sums
    (dbeta, the chunk-end dG term) are added in a fixed order, not by LDS atomics whose
    order follows the waves' timing. Three calls at the c2 shape (with dht) and a packed
    batch."""
    import gated_delta_rule_64_amd as kda
    for d in (small(2, 1024 + 37, 4, 8, 128, 128, torch.bfloat16, seed=68), _train_case("packed_many_chains")):
        do, dht = _bwd_inputs(d, 69)
        runs = [kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["initial_state"],
                                  d["cu_seqlens"], dht) for _ in range(3)]
        torch.cuda.synchronize()
        for rep in runs[1:]:
            for name, x, y in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], rep, runs[0]):
                assert torch.equal(x, y), f"{name} differs between calls"
    log("  three backward calls bitwise equal (dense and packed)")


def _train_case(case):
    if case == "dense_gva_bf16":
        return small(2, 200, 2, 4, 128, 128, torch.bfloat16, seed=64)
    if case == "dense_fp32_k64":
        return small(1, 300, 2, 2, 64, 128, torch.float32, seed=65)
    # packed, 160 slots x 8 heads: kda_chunk_fwd takes 32-column slices (compact records)
    w = inputs.Workload("many", 1, 0, 4, 8, 128, 128, torch.bfloat16, torch.bfloat16, 66, -5.0, 0.05, True,
                        n_slots=160, len_lo=1, len_hi=200, n_empty=10)
    return to_device(inputs.make(w))


@pytest.mark.parametrize("case", ["dense_gva_bf16", "dense_fp32_k64", "packed_many_chains"])
def test_chunk_train_forward_and_saved_backward(case):
    """The training forward's o and final state against kda_chunk_fwd (bit for bit where
    that forward's scan also takes 16-column slices, else to the tolerance) and the
    oracle; the backward from its workspace bit for bit equal to the full backward's,
    twice in a row from the same workspace."""
    import gated_delta_rule_64_amd as kda
    d = _train_case(case)
    dtype = d["q"].dtype
    cu = d["cu_seqlens"]
    log(f"[train forward + saved backward] {case}")
    o, ht, ws = kda.kda_chunk_fwd_train(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], cu,
                                        output_final_state=True)
    o_f, ht_f = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], cu,
                                  output_final_state=True)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle_of(d)
    rows = valid_rows(cu.cpu(), d["q"].shape[1]) if cu is not None else None
    if rows is None:
        check("o", o, o_ref, dtype)
    else:
        check("o", o[:, rows], o_ref[:, rows], dtype)
    check("final_state", ht, ht_ref, dtype)
    if case == "packed_many_chains":
        check("o (vs kda_chunk_fwd)", o[:, rows], to64(o_f[:, rows]), dtype, want_rounded=True)
        check("final_state (vs kda_chunk_fwd)", ht, to64(ht_f), dtype)
    else:
        assert torch.equal(o, o_f) and torch.equal(ht, ht_f), "16-column slices: same bits as kda_chunk_fwd"
    do, dht = _bwd_inputs(d, 67)
    full = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["initial_state"], cu, dht)
    for rep in range(2):
        saved = kda.kda_chunk_bwd_saved(d["q"], d["k"], d["v"], d["g"], d["beta"], do, ws,
                                        d["initial_state"], cu, dht)
        torch.cuda.synchronize()
        for name, x, y in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], saved, full):
            assert torch.equal(x, y), f"{name} differs from kda_chunk_bwd's (call {rep})"
    log("  saved backward == full backward bitwise (two calls)")


def test_chunk_many_slots():
    """Packed offsets with more slots (2,100) than the schedule sorts by length (2,048),
    so the scans take the slots in index order: lengths 0..70 (every tenth slot empty,
    some crossing a chunk boundary), forward and backward against the oracle, empty
    slots' states passed through bitwise."""
    rng = np.random.default_rng(96)
    lens = rng.integers(1, 71, size=2100)
    lens[::10] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Tp = int(cu[-1]) + 8
    d = small(1, Tp, 1, 2, 64, 64, torch.bfloat16, seed=97)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=DEV)
    d["initial_state"] = torch.randn(len(lens), 2, 64, 64, generator=torch.Generator().manual_seed(98)).mul(0.05).to(DEV)
    log(f"[many slots] 2100 slots, {int(cu[-1])} tokens, HV2 K=V=64 bf16")
    o, ht = run("chunk", d)
    o_ref, ht_ref = oracle_of(d)
    m = valid_rows(cu, Tp)
    check("o", o[:, m], o_ref[:, m], torch.bfloat16)
    check("final_state", ht, ht_ref, torch.bfloat16)
    for n in np.nonzero(lens == 0)[0][:20]:
        assert torch.equal(ht[n], d["initial_state"][n]), f"empty slot {n} state must pass through bitwise"
    do, dht = _bwd_inputs(d, 99)
    _check_bwd(d, do, dht, torch.bfloat16, rows=torch.from_numpy(m), label="many slots ")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_bwd_dense_gva(dtype):
    """B=2, T=200 (a short last chunk), H=2, HV=4 (GVA), K=V=128, initial state and a
    final-state gradient: dq, dk, dv, dg, dbeta, dh0 against the oracle."""
    d = small(2, 200, 2, 4, 128, 128, dtype, seed=60)
    do, dht = _bwd_inputs(d, 61)
    log(f"[bwd dense] B2 T200 H2 HV4 K=V=128 {dtype}")
    _check_bwd(d, do, dht, dtype)


def test_chunk_bwd_packed():
    """Packed sequences with an empty slot and a tail of unowned rows: gradients on the
    valid rows, the empty slot's dh0 equal to its dht bitwise, the tail untouched (zero)."""
    lens = [130, 0, 64, 37, 200]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    Tp = cu[-1] + 40
    d = small(1, Tp, 2, 4, 128, 128, torch.bfloat16, seed=62)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=DEV)
    d["initial_state"] = torch.randn(len(lens), 4, 128, 128, generator=torch.Generator().manual_seed(7)).mul(0.05).to(DEV)
    do, dht = _bwd_inputs(d, 63)
    log(f"[bwd packed] lens={lens}")
    rows = valid_rows(cu, Tp)
    got, _ = _check_bwd(d, do, dht, torch.bfloat16, rows=torch.from_numpy(rows))
    assert torch.equal(got[5][1], dht[1]), "empty slot passes dht to dh0 bitwise"
    for x in got[:5]:
        assert not x[0, cu[-1]:].float().abs().any(), "tail rows must stay untouched"


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_chunk_bwd_head_dims(K, V):
    d = small(1, 150, 2, 2, K, V, torch.bfloat16, seed=64 + K + V)
    do, dht = _bwd_inputs(d, 65)
    log(f"[bwd head dims] K={K} V={V}")
    _check_bwd(d, do, dht, torch.bfloat16)


def test_chunk_bwd_steep_gates():
    """Per-token gates of -15 on one chunk of one head (decay factors down to 2^-945
    inside a chunk): every factor is one-sided, nothing overflows."""
    d = small(1, 200, 2, 4, 128, 128, torch.bfloat16, seed=66)
    g = d["g"].clone()
    g[:, 64:128, 2] = -15.0
    d["g"] = g
    do, dht = _bwd_inputs(d, 67)
    _check_bwd(d, do, dht, torch.bfloat16)


def test_chunk_bwd_c3_full():
    """The long-context workload (B=1 T=8192 H=16 HV=32 K=V=128 bf16, no initial state,
    no final-state gradient), every gradient against the oracle."""
    d = to_device(inputs.make("c3"))
    do, _ = _bwd_inputs(d, 68, dht=False)
    log("[bwd c3] B=1 T=8192 H=16 HV=32 K=V=128 bf16")
    _check_bwd(d, do, None, torch.bfloat16)


# ------------------------------------------------------------------------------------
# decode serving: transposed state layout, intermediate states, graph replay
# ------------------------------------------------------------------------------------
def _packed_case(lens, HV=4, seed=70, dtype=torch.bfloat16, KV=128):
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    Tp = cu[-1] + 8
    d = small(1, Tp, 2, HV, KV, KV, dtype, seed=seed)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=DEV)
    d["initial_state"] = torch.randn(len(lens), HV, KV, KV, generator=torch.Generator().manual_seed(seed + 1)).mul(0.05).to(DEV)
    return d, cu


@pytest.mark.parametrize("lens,KV", [([5, 0, 1, 9], 128), ([1] * 18 + [0, 2, 3, 0, 1, 1], 128), ([5, 0, 1, 9], 64)],
                         ids=["packed", "about_one_token", "packed_k64"])
def test_recurrent_state_layout_vk(lens, KV):
    """States stored transposed ([V][K] per head): both layouts within the tolerance of
    the oracle, and within fp32 rounding of each other (the layouts sum a state's rows in
    different orders, so agreement is to a rounding step, not bitwise). The second case
    has at most 1.5 rows per sequence (33 rows, 24 slots), which takes the decode launch
    of the [K][V] layout."""
    import gated_delta_rule_64_amd as kda
    d, cu = _packed_case(lens, KV=KV)
    o1, s1 = kda.kda_recurrent_fwd_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"],
                                      d["cu_seqlens"], output_final_state=True)
    h0t = d["initial_state"].transpose(-1, -2).contiguous()
    o2, s2 = kda.kda_recurrent_fwd_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], h0t, d["cu_seqlens"],
                                      output_final_state=True, state_layout="vk")
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle_of(d)
    rows = torch.from_numpy(valid_rows(cu, d["q"].shape[1])).to(DEV)
    s2 = s2.transpose(-1, -2)
    for tag, o, s in (("kv", o1, s1), ("vk", o2, s2)):
        check(f"{tag} o", o[0][rows], o_ref[0][rows.cpu().numpy()], torch.bfloat16)
        check(f"{tag} final state", s, ht_ref, torch.bfloat16)
    # fp32 states: a few rounding steps of the largest entry apart; bf16 outputs: at most
    # one bf16 rounding step (a relative 2^-8 of the value) apart
    smax = float(s1.abs().max())
    assert float((s1 - s2).abs().max()) <= 16 * 2.0 ** -24 * smax
    a, b = o1[0][rows].float(), o2[0][rows].float()
    assert bool(((a - b).abs() <= a.abs() * 2.0 ** -7 + 1e-6).all())


@pytest.mark.parametrize("layout", ["kv", "vk"])
def test_recurrent_intermediate_states(layout):
    """The state after every token: equal to the final state at each sequence's last
    token (bitwise), and to the oracle's final state of the prefix at sampled tokens."""
    import gated_delta_rule_64_amd as kda
    lens = [7, 0, 3, 12]
    d, cu = _packed_case(lens, seed=72)
    h0 = d["initial_state"] if layout == "kv" else d["initial_state"].transpose(-1, -2).contiguous()
    o, ht, inter = kda.kda_recurrent_fwd_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], h0, d["cu_seqlens"],
                                            output_final_state=True, state_layout=layout,
                                            output_intermediate_states=True)
    torch.cuda.synchronize()
    if layout == "vk":
        inter = inter.transpose(-1, -2)
        ht = ht.transpose(-1, -2)
    for n, ln in enumerate(lens):
        if ln:
            assert torch.equal(inter[cu[n + 1] - 1], ht[n]), f"sequence {n}: last intermediate != final"
    for n, t_in in [(0, 0), (0, 4), (2, 1), (3, 11), (3, 6)]:
        r = cu[n] + t_in
        sub = dict(q=d["q"][:, cu[n]:r + 1], k=d["k"][:, cu[n]:r + 1], v=d["v"][:, cu[n]:r + 1],
                   g=d["g"][:, cu[n]:r + 1], beta=d["beta"][:, cu[n]:r + 1],
                   initial_state=d["initial_state"][n:n + 1], cu_seqlens=None)
        _, ht_ref = oracle_of(sub)
        check(f"state after token {t_in} of sequence {n}", inter[r], ht_ref[0], torch.bfloat16)


def _graph_variants(N, Tp, seed):
    """Offsets and histories for successive replays: one token each, repeated offsets
    (empty slots) with two-token sequences, then a shorter terminal offset."""
    gen = torch.Generator().manual_seed(seed)
    a = list(range(N + 1))
    b = [0]
    for n in range(N):
        b.append(b[-1] + (0 if n % 3 == 1 else (2 if n % 3 == 2 else 1)))
    c = [min(x, Tp // 4) for x in a]
    out = []
    for cu in (a, b, c):
        assert cu[-1] <= Tp
        out.append((torch.tensor(cu, dtype=torch.int32), torch.randn(N, 4, 128, 128, generator=gen).mul(0.05)))
    return out


@pytest.mark.parametrize("path", ["recurrent", "chunk"])
def test_graph_replay_mutated_boundaries_and_history(path):
    """Capture one call in a HIP graph, then replay it with new offsets and new initial
    states copied into its input buffers (eager work and syncs between replays); every
    replay must equal an eager call on the same inputs, bitwise."""
    import gated_delta_rule_64_amd as kda
    N, Tp = 48, 96
    d = small(1, Tp, 2, 4, 128, 128, torch.bfloat16, seed=74)
    variants = _graph_variants(N, Tp, 75)
    cu_buf = variants[0][0].to(DEV).clone()
    h0_buf = variants[0][1].to(DEV).clone()
    out = torch.zeros_like(d["v"])
    ht = torch.zeros(N, 4, 128, 128, device=DEV)
    ws = None
    if path == "chunk":
        ws = torch.empty(kda.kda_chunk_fwd_workspace_bytes(1, Tp, 2, 4, 128, 128, N, 1), dtype=torch.uint8, device=DEV)

    def call(cu, h0, o, s):
        if path == "chunk":
            kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0, cu, output_final_state=True,
                              out=o, final_state=s, workspace=ws)
        else:
            kda.kda_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], h0, cu, output_final_state=True,
                                  out=o, final_state=s)

    call(cu_buf, h0_buf, out, ht)      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(cu_buf, h0_buf, out, ht)
    torch.cuda.synchronize()
    for rep, (cu, h0) in enumerate(variants * 2):
        cu_buf.copy_(cu.to(DEV))
        h0_buf.copy_(h0.to(DEV))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ref = torch.full_like(d["v"], float("nan"))
        s_ref = torch.zeros_like(ht)
        call(cu_buf, h0_buf, o_ref, s_ref)      # eager, same inputs
        torch.cuda.synchronize()
        used = int(cu[-1])
        assert torch.equal(out[:, :used], o_ref[:, :used]), f"replay {rep}: o differs"
        assert torch.equal(ht, s_ref), f"replay {rep}: final state differs"
        assert torch.isnan(out[:, used:].float()).all(), f"replay {rep}: rows past the last offset were written"


BWD_EDGE = [  # (label, B, T, H, HV, K, V, dtype, h0, dht)
    ("single_token", 3, 1, 2, 2, 128, 128, torch.bfloat16, True, True),
    ("one_chunk", 1, 64, 2, 4, 128, 64, torch.bfloat16, True, False),
    ("chunk_plus_one", 2, 65, 1, 2, 64, 128, torch.float32, False, True),
    ("fp32_k64", 1, 130, 2, 2, 64, 64, torch.float32, True, True),
    # bf16 kernels at K = 64 (the pair kernel's eight-wave shape), four value heads per
    # q/k head summed in the pair kernel, a ragged last chunk
    ("bf16_k64_gva4", 1, 150, 1, 4, 64, 128, torch.bfloat16, True, True),
    ("bf16_k64_v64", 2, 100, 2, 2, 64, 64, torch.bfloat16, False, True),
]


@pytest.mark.parametrize("case", BWD_EDGE, ids=[c[0] for c in BWD_EDGE])
def test_chunk_bwd_edges(case):
    label, B, T, H, HV, K, V, dtype, h0, dht = case
    d = small(B, T, H, HV, K, V, dtype, seed=80 + T, h0=h0)
    do, dht_t = _bwd_inputs(d, 81, dht=dht)
    log(f"[bwd edge {label}] B{B} T{T} H{H} HV{HV} K{K} V{V} {dtype}")
    _check_bwd(d, do, dht_t, dtype)


def test_chunk_bwd_zero_beta_and_short_packed():
    """beta exactly 0 on a third of the tokens (dbeta then needs M itself, not L = beta M),
    packed slots of length 1 between empty ones, and no dh0 wanted."""
    import gated_delta_rule_64_amd as kda
    lens = [0, 1, 0, 0, 70, 1]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    Tp = cu[-1] + 3
    d = small(1, Tp, 2, 2, 128, 128, torch.bfloat16, seed=84)
    d["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=DEV)
    d["initial_state"] = torch.randn(len(lens), 2, 128, 128, generator=torch.Generator().manual_seed(85)).mul(0.05).to(DEV)
    beta = d["beta"].clone()
    beta[:, ::3] = 0.0
    d["beta"] = beta
    do, dht = _bwd_inputs(d, 86)
    got = kda.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["initial_state"],
                            d["cu_seqlens"], dht, want_dh0=False)
    torch.cuda.synchronize()
    assert got[5] is None
    ref = oracle.recurrent_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["initial_state"],
                               d["cu_seqlens"], dht)
    rows = torch.from_numpy(valid_rows(cu, Tp))
    for name, x, y in zip(["dq", "dk", "dv", "dg", "dbeta"], got[:5], ref[:5]):
        check(name, x[:, rows], y[:, rows], torch.bfloat16)


# ------------------------------------------------------------------------------------
# backward through the fused input options
# ------------------------------------------------------------------------------------
def _bwd_ex_oracle(r, do, dht, g_raw, A_log, dt_bias, bound, lq, lk, sig, neg):
    """The oracle composed: the options' forward transforms, the recurrence's gradients,
    then each option's chain rule."""
    qn = oracle.l2norm(r["q"]) if lq else r["q"]
    kn = oracle.l2norm(r["k"]) if lk else r["k"]
    ba = oracle.beta_sigmoid(r["beta"], neg) if sig else r["beta"]
    g2 = oracle.gate_activation(g_raw, A_log, dt_bias, bound) if g_raw is not None else r["g"]
    dq, dk, dv, dg2, dba, dh0 = oracle.recurrent_bwd(qn, kn, r["v"], g2, ba, do, r["initial_state"],
                                                     r["cu_seqlens"], dht)
    if lq:
        dq = oracle.l2norm_bwd(r["q"], dq)
    if lk:
        dk = oracle.l2norm_bwd(r["k"], dk)
    if sig:
        dba = oracle.beta_sigmoid_bwd(r["beta"], dba, neg)
    dA = ddt = None
    dg = dg2
    if g_raw is not None:
        dg, dA, ddt = oracle.gate_activation_bwd(g_raw, A_log, dt_bias, bound, dg2)
    return dq, dk, dv, dg, dba, dh0, dA, ddt


BWD_EX = [  # (gate raw, lower bound, l2norm q, l2norm k, sigmoid, neg eigval, dtype)
    (True, None, True, True, True, False, torch.bfloat16),
    (True, -4.0, False, True, False, False, torch.bfloat16),
    (False, None, True, False, True, True, torch.bfloat16),
    (True, None, True, True, True, True, torch.float32),
]


@pytest.mark.parametrize("case", BWD_EX, ids=lambda c: f"gate{int(c[0])}_lb{c[1]}_q{int(c[2])}k{int(c[3])}_sig{int(c[4])}{int(c[5])}_{str(c[6])[6:]}")
def test_chunk_bwd_ex(case):
    """Gradients through the fused options with respect to the raw inputs (and A_log,
    dt_bias) against the composed oracle. Row scales 10^U[-0.5, 0.5]: the normalisation's
    gradient grows as 1 / |row|, so rows far below unit norm would only test fp32's
    relative precision against an absolute bound."""
    import gated_delta_rule_64_amd as kda
    raw, bound, lq, lk, sig, neg, dtype = case
    d = small(1, 200, 2, 4, 128, 128, dtype, seed=90)
    r = _raw_inputs(d, 91, lq, lk, sig, zero_rows=False, span=0.5)
    g_raw = A_log = dt_bias = None
    if raw:
        g_raw, A_log, dt_bias = _gate_params(1, 200, 4, 128, torch.bfloat16 if dtype == torch.bfloat16 else torch.float32, seed=92)
    do, dht = _bwd_inputs(d, 93)
    got = kda.kda_chunk_bwd_ex(r["q"], r["k"], r["v"], g_raw if raw else r["g"], r["beta"], do,
                               r["initial_state"], None, dht, use_gate_in_kernel=raw, A_log=A_log,
                               dt_bias=dt_bias, lower_bound=bound, l2norm_q=lq, l2norm_k=lk,
                               use_beta_sigmoid_in_kernel=sig, allow_neg_eigval=neg)
    torch.cuda.synchronize()
    ref = _bwd_ex_oracle(r, do, dht, g_raw, A_log, dt_bias, bound, lq, lk, sig, neg)
    log(f"[bwd ex] gate raw={raw} bound={bound} l2norm q={lq} k={lk} sigmoid={sig} neg={neg} {dtype}")
    for name, x, y in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0", "dA_log", "ddt_bias"], got, ref):
        if y is None:
            assert x is None, name
            continue
        check(name, x, np.asarray(y).reshape(tuple(x.shape)), dtype)


@pytest.mark.parametrize("case", BWD_EX, ids=lambda c: f"gate{int(c[0])}_lb{c[1]}_q{int(c[2])}k{int(c[3])}_sig{int(c[4])}{int(c[5])}_{str(c[6])[6:]}")
def test_chunk_train_ex_forward_and_saved_backward(case):
    """The training split with the fused options: the forward's o and final state against
    the composed oracle and kda_chunk_fwd_ex; the backward from its workspace bit for bit
    equal to kda_chunk_bwd_ex's, twice in a row from the same workspace."""
    import gated_delta_rule_64_amd as kda
    raw, bound, lq, lk, sig, neg, dtype = case
    d = small(1, 200, 2, 4, 128, 128, dtype, seed=90)
    r = _raw_inputs(d, 91, lq, lk, sig, zero_rows=False, span=0.5)
    g_raw = A_log = dt_bias = None
    if raw:
        g_raw, A_log, dt_bias = _gate_params(1, 200, 4, 128, torch.bfloat16 if dtype == torch.bfloat16 else torch.float32, seed=92)
    opts = dict(use_gate_in_kernel=raw, A_log=A_log, dt_bias=dt_bias, lower_bound=bound, l2norm_q=lq,
                l2norm_k=lk, use_beta_sigmoid_in_kernel=sig, allow_neg_eigval=neg)
    g_in = g_raw if raw else r["g"]
    log(f"[train ex] gate raw={raw} bound={bound} l2norm q={lq} k={lk} sigmoid={sig} neg={neg} {dtype}")
    o, ht, ws = kda.kda_chunk_fwd_ex_train(r["q"], r["k"], r["v"], g_in, r["beta"], r["initial_state"],
                                           None, output_final_state=True, **opts)
    o_f, ht_f = kda.kda_chunk_fwd_ex(r["q"], r["k"], r["v"], g_in, r["beta"], r["initial_state"], None,
                                     output_final_state=True, **opts)
    torch.cuda.synchronize()
    g2 = oracle.gate_activation(g_raw, A_log, dt_bias, bound) if raw else None
    o_ref, ht_ref = _pre_oracle(r, lq, lk, sig, neg, g2=g2)
    check("o", o, o_ref, dtype)
    check("final_state", ht, ht_ref, dtype)
    check("o (vs kda_chunk_fwd_ex)", o, to64(o_f), dtype, want_rounded=True)
    check("final_state (vs kda_chunk_fwd_ex)", ht, to64(ht_f), dtype)
    do, dht = _bwd_inputs(d, 93)
    full = kda.kda_chunk_bwd_ex(r["q"], r["k"], r["v"], g_in, r["beta"], do, r["initial_state"], None,
                                dht, **opts)
    for rep in range(2):
        saved = kda.kda_chunk_bwd_ex_saved(r["q"], r["k"], r["v"], g_in, r["beta"], do, ws,
                                           r["initial_state"], None, dht, **opts)
        torch.cuda.synchronize()
        for name, x, y in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0", "dA_log", "ddt_bias"], saved, full):
            if y is None:
                assert x is None, name
                continue
            assert torch.equal(x, y), f"{name} differs from kda_chunk_bwd_ex's (call {rep})"
    log("  saved backward == full backward bitwise (two calls)")


# ------------------------------------------------------------------------------------
# the in-place timing entry point: NULL event slots are skipped, results unchanged
# ------------------------------------------------------------------------------------
def test_timed_entry_null_event_slots():
    import ctypes

    import bench
    import gated_delta_rule_64_amd as kda
    d = small(1, 1000, 4, 8, 128, 128, torch.bfloat16, seed=12, h0=False)
    o_ref, _ = run("chunk", d, final=False)
    lib = kda.load_library()
    vp = ctypes.c_void_p
    lib.kda_chunk_fwd_timed.restype = ctypes.c_int
    lib.kda_chunk_fwd_timed.argtypes = list(lib.kda_chunk_fwd.argtypes) + [vp]
    hip = bench.hip_runtime()
    ev = bench.Events(hip, 4)
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    ws_bytes = kda.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, B, 0, kda.KDA_BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    sptr = vp(torch.cuda.current_stream().cuda_stream)
    for slots in ((None, None, ev.ev[2], ev.ev[3]), tuple(ev.ev[i] for i in range(4))):
        log(f"[timed entry] events recorded: {[s is not None for s in slots]}")
        out = torch.full_like(d["v"], float("nan"))
        arr = (vp * 4)(*slots)
        rc = lib.kda_chunk_fwd_timed(
            vp(d["q"].data_ptr()), vp(d["k"].data_ptr()), vp(d["v"].data_ptr()), vp(d["g"].data_ptr()),
            vp(d["beta"].data_ptr()), None, None, B, vp(out.data_ptr()), None, B, T, H, HV, K, V,
            kda.KDA_BF16, kda.KDA_BF16, 0.0, 64, vp(ws.data_ptr()), ws_bytes, None, sptr, ctypes.cast(arr, vp))
        assert rc == 0, lib.kda_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref)
        assert ev.ms(2, 3) > 0.0
    ev.close()


# ------------------------------------------------------------------------------------
# degenerate inputs: no rows at all (dense T = 0) and packed offsets whose every slot is
# empty; states pass through bitwise, o is never written
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_degenerate_inputs(path):
    import gated_delta_rule_64_amd as kda
    gen = torch.Generator().manual_seed(21)
    H, HV, K, V = 2, 4, 128, 128
    fn = kda.kda_chunk_fwd if path == "chunk" else kda.kda_recurrent_fwd

    def tensors(B, T, N):
        q = torch.randn(B, T, H, K, generator=gen).to(torch.bfloat16).to(DEV)
        k = torch.randn(B, T, H, K, generator=gen).to(torch.bfloat16).to(DEV)
        v = torch.randn(B, T, HV, V, generator=gen).to(torch.bfloat16).to(DEV)
        g = (-torch.rand(B, T, HV, K, generator=gen)).to(DEV)
        beta = torch.rand(B, T, HV, generator=gen).to(torch.bfloat16).to(DEV)
        h0 = (torch.randn(N, HV, K, V, generator=gen) * 0.05).to(DEV)
        return q, k, v, g, beta, h0

    log(f"[degenerate {path}] dense B=2 T=0")
    q, k, v, g, beta, h0 = tensors(2, 0, 2)
    o, ht = fn(q, k, v, g, beta, h0, None, output_final_state=True)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(ht, h0)
    o, ht = fn(q, k, v, g, beta, None, None, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(ht, torch.zeros_like(h0))

    log(f"[degenerate {path}] packed N=3, every slot empty, 70 unowned rows")
    q, k, v, g, beta, h0 = tensors(1, 70, 3)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    out = torch.full_like(v, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    o, ht = fn(q, k, v, g, beta, h0, cu, output_final_state=True, out=out, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.isnan(o.float()).all(), "rows outside every sequence are not written"
    assert torch.equal(ht, h0), "empty slots pass their states through bitwise"


def test_degenerate_inputs_bwd():
    """The backward on the same degenerate inputs: the final-state gradient passes to the
    initial state's bitwise (the state does), and rows outside every sequence get zero
    gradients."""
    import gated_delta_rule_64_amd as kda
    gen = torch.Generator().manual_seed(22)
    H, HV, K, V = 2, 4, 128, 128

    def tensors(B, T, N):
        q = torch.randn(B, T, H, K, generator=gen).to(torch.bfloat16).to(DEV)
        k = torch.randn(B, T, H, K, generator=gen).to(torch.bfloat16).to(DEV)
        v = torch.randn(B, T, HV, V, generator=gen).to(torch.bfloat16).to(DEV)
        g = (-torch.rand(B, T, HV, K, generator=gen)).to(DEV)
        beta = torch.rand(B, T, HV, generator=gen).to(torch.bfloat16).to(DEV)
        do = torch.randn(B, T, HV, V, generator=gen).to(torch.bfloat16).to(DEV)
        h0 = (torch.randn(N, HV, K, V, generator=gen) * 0.05).to(DEV)
        dht = torch.randn(N, HV, K, V, generator=gen).to(DEV)
        return q, k, v, g, beta, do, h0, dht

    log("[degenerate bwd] dense B=2 T=0")
    q, k, v, g, beta, do, h0, dht = tensors(2, 0, 2)
    dq, dk, dv, dg, db, dh0 = kda.kda_chunk_bwd(q, k, v, g, beta, do, h0, None, dht)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.equal(dh0, dht)

    log("[degenerate bwd] packed N=3, every slot empty, 70 unowned rows")
    q, k, v, g, beta, do, h0, dht = tensors(1, 70, 3)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    dq, dk, dv, dg, db, dh0 = kda.kda_chunk_bwd(q, k, v, g, beta, do, h0, cu, dht)
    torch.cuda.synchronize()
    assert torch.equal(dh0, dht)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg), ("dbeta", db)):
        assert (t.float() == 0).all(), f"{name} must be zero outside every sequence"
