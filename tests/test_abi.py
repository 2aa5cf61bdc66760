"""The C ABI library without a GPU: it loads, exports every declared entry point, sizes
its workspace as documented, and rejects bad arguments on the host before enqueueing
anything (no test here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_64_amd import _lib
    if not os.path.exists(_lib.library_path()):
        from gated_delta_rule_64_amd import build
        build.build()
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_recurrent_fwd", "kda_chunk_fwd_workspace_bytes",
              "kda_last_error", "kda_abi_version"):
        assert n in names
    assert "kda_chunk_fwd_gated" in names
    assert "kda_chunk_fwd_ex" in names and "kda_recurrent_fwd_ex" in names


def _header_int(name):
    m = re.search(r"#define\s+%s\s+(\d+)" % name, open(HEADER).read())
    if m:
        return int(m.group(1))
    m = re.search(r"\b%s\s*=\s*(-?\d+)" % name, open(HEADER).read())
    return int(m.group(1))


def test_binding_constants_match_the_header():
    from gated_delta_rule_64_amd import _lib
    for name in ("KDA_F32", "KDA_BF16", "KDA_DEV_BAD_CU_SEQLENS", "KDA_GATE_LOG2",
                 "KDA_GATE_RAW_F32", "KDA_GATE_RAW_BF16", "KDA_PRE_L2NORM_Q", "KDA_PRE_L2NORM_K",
                 "KDA_PRE_BETA_SIGMOID", "KDA_PRE_NEG_EIGVAL", "KDA_STATE_KV", "KDA_STATE_VK"):
        assert getattr(_lib, name) == _header_int(name), name


def test_library_exports_every_declared_symbol(lib):
    from gated_delta_rule_64_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version(lib):
    assert lib.kda_abi_version() == _header_int("KDA_ABI_VERSION")


def _rec_bytes(K, V, elem, compact=False):
    # w, qg, kg^T and Aqk in the compute type; u and 2^G in fp32. On the bf16 path qg,
    # kg^T and Aqk carry their residual as a second bf16 tile, or, in compact records
    # (launches whose scan takes 32-column slices: chains x V / 32 >= 512), as fp8 tiles
    # (a byte per value) with a 32-bit scale word per 16-row band and lane
    b = 64 * K * elem + 2 * 64 * K * elem + 64 * 64 * elem + 64 * V * 4 + 4 * K
    if elem == 2 and compact:
        b += 2 * 64 * K + 64 * 64 + (64 // 16 + K // 16 + 64 // 16) * 64 * 4
    elif elem == 2:
        b += 2 * 64 * K * elem + 64 * 64 * elem
    return (b + 255) // 256 * 256


def _sched_bytes(N, ncmax):
    # first/end chunk and validity per sequence, chunk count, the chunk table, then the
    # slot order
    s = ((3 * N + 1) * 4 + 15) // 16 * 16 + ncmax * 8 + N * 4
    return (s + 255) // 256 * 256


@pytest.mark.parametrize("K,V,dt,elem", [(128, 128, 1, 2), (64, 64, 0, 4), (128, 64, 1, 2)])
def test_workspace_bytes_dense(lib, K, V, dt, elem):
    B, T, H, HV = 2, 4096 + 17, 4, 8
    nt = (T + 63) // 64
    got = lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, B, 0, dt)
    assert got == _sched_bytes(B, B * nt) + HV * B * nt * _rec_bytes(K, V, elem)


def test_workspace_bytes_packed(lib):
    # 64 x 16 chains: the compact records of the 32-column scan
    N, T, HV = 64, 33000, 16
    got = lib.kda_chunk_fwd_workspace_bytes(1, T, 16, HV, 128, 128, N, 1, 1)
    ncmax = T // 64 + N
    assert got == _sched_bytes(N, ncmax) + HV * ncmax * _rec_bytes(128, 128, 2, compact=True)


@pytest.mark.parametrize("B,HV,V,compact", [(16, 8, 128, True), (1, 127, 128, False),
                                            (1, 128, 128, True), (2, 128, 64, True),
                                            (1, 255, 64, False)])
def test_workspace_bytes_compact_threshold(lib, B, HV, V, compact):
    """bf16 records are compact exactly where the scan takes 32-column slices:
    chains x V / 32 >= 512 blocks."""
    T, K = 200, 128
    nt = (T + 63) // 64
    got = lib.kda_chunk_fwd_workspace_bytes(B, T, 2, HV, K, V, B, 0, 1)
    assert got == _sched_bytes(B, B * nt) + HV * B * nt * _rec_bytes(K, V, 2, compact=compact)
    # the fp32 path never is
    got32 = lib.kda_chunk_fwd_workspace_bytes(B, T, 2, HV, K, V, B, 0, 0)
    assert got32 == _sched_bytes(B, B * nt) + HV * B * nt * _rec_bytes(K, V, 4)


def test_workspace_bytes_invalid(lib):
    assert lib.kda_chunk_fwd_workspace_bytes(1, 64, 1, 1, 96, 128, 1, 0, 1) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 64, 1, 1, 128, 128, 1, 0, 7) == 0


FAKE = 0x10000  # aligned non-NULL host value: every call below fails validation first


def _chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=1, o=FAKE, ht=None,
             B=1, T=64, H=2, HV=2, K=128, V=128, qd=1, bd=1, scale=0.0, cs=64,
             ws=FAKE, wsb=1 << 40, st=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], a["N"],
                             a["o"], a["ht"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                             a["qd"], a["bd"], a["scale"], a["cs"], a["ws"], a["wsb"], a["st"],
                             a["stream"])


def _rec(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=1, o=FAKE, ht=None,
             B=1, T=1, H=2, HV=2, K=128, V=128, qd=1, bd=1, scale=0.0, st=None, stream=None)
    a.update(kw)
    return lib.kda_recurrent_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                                 a["N"], a["o"], a["ht"], a["B"], a["T"], a["H"], a["HV"], a["K"],
                                 a["V"], a["qd"], a["bd"], a["scale"], a["st"], a["stream"])


def _gated(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gd=1, A=FAKE, dt=None, hlb=0, lb=0.0, beta=FAKE,
             h0=None, cu=None, N=1, o=FAKE, ht=None, B=1, T=64, H=2, HV=2, K=128, V=128, qd=1,
             bd=1, scale=0.0, cs=64, ws=FAKE, wsb=1 << 40, st=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], a["g"], a["gd"], a["A"], a["dt"],
                                   a["hlb"], a["lb"], a["beta"], a["h0"], a["cu"], a["N"], a["o"],
                                   a["ht"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                   a["qd"], a["bd"], a["scale"], a["cs"], a["ws"], a["wsb"],
                                   a["st"], a["stream"])


def _ex(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gate=0, A=None, dt=None, hlb=0, lb=0.0, beta=FAKE,
             pre=0, h0=None, cu=None, N=1, o=FAKE, ht=None, B=1, T=64, H=2, HV=2, K=128, V=128,
             qd=1, bd=1, scale=0.0, cs=64, ws=FAKE, wsb=1 << 40, st=None, stream=None, ev=None)
    a.update(kw)
    return lib.kda_chunk_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["gate"], a["A"], a["dt"],
                                a["hlb"], a["lb"], a["beta"], a["pre"], a["h0"], a["cu"], a["N"],
                                a["o"], a["ht"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                a["qd"], a["bd"], a["scale"], a["cs"], a["ws"], a["wsb"],
                                a["st"], a["stream"], a["ev"])


def _rec_ex(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gate=0, A=None, dt=None, hlb=0, lb=0.0, beta=FAKE,
             pre=0, lay=0, h0=None, cu=None, N=1, o=FAKE, ht=None, inter=None, B=1, T=1, H=2, HV=2,
             K=128, V=128, qd=1, bd=1, scale=0.0, st=None, stream=None)
    a.update(kw)
    return lib.kda_recurrent_fwd_ex(a["q"], a["k"], a["v"], a["g"], a["gate"], a["A"], a["dt"],
                                    a["hlb"], a["lb"], a["beta"], a["pre"], a["lay"], a["h0"],
                                    a["cu"], a["N"], a["o"], a["ht"], a["inter"], a["B"], a["T"],
                                    a["H"], a["HV"], a["K"], a["V"], a["qd"], a["bd"], a["scale"],
                                    a["st"], a["stream"])


def _bwd(lib, fn="kda_chunk_bwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=1, do=FAKE, dht=None,
             dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, db=FAKE, dh0=None, B=1, T=64, H=2, HV=2, K=128,
             V=128, qd=1, bd=1, scale=0.0, cs=64, ws=FAKE, wsb=1 << 40, st=None, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], a["N"],
                            a["do"], a["dht"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"],
                            a["dh0"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["qd"],
                            a["bd"], a["scale"], a["cs"], a["ws"], a["wsb"], a["st"], a["stream"])


def _train(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=1, o=FAKE, fs=None,
             B=1, T=64, H=2, HV=2, K=128, V=128, qd=1, bd=1, scale=0.0, cs=64, ws=FAKE,
             wsb=1 << 40, st=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_train(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], a["N"],
                                   a["o"], a["fs"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                   a["qd"], a["bd"], a["scale"], a["cs"], a["ws"], a["wsb"], a["st"],
                                   a["stream"])


CASES = [
    ("null q", dict(q=None), -1),
    ("HV % H", dict(H=3, HV=4), -2),
    ("negative T", dict(T=-1), -2),
    ("B != N dense", dict(B=2, N=1), -2),
    ("packed needs B == 1", dict(B=2, N=1, cu=FAKE), -2),
    ("dtype", dict(qd=5), -3),
    ("beta dtype", dict(bd=2), -3),
    ("misaligned q", dict(q=FAKE + 4), -2),
]


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_chunk_rejects(lib, name, kw, code):
    assert _chunk(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_recurrent_rejects(lib, name, kw, code):
    assert _rec(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_gated_rejects_common(lib, name, kw, code):
    assert _gated(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("call", ["chunk_ex", "recurrent_ex"])
def test_ex_rejects_common(lib, call, name, kw, code):
    f = _ex if call == "chunk_ex" else _rec_ex
    assert f(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


@pytest.mark.parametrize("call", ["chunk_ex", "recurrent_ex"])
def test_ex_option_rejects(lib, call):
    f = _ex if call == "chunk_ex" else _rec_ex
    assert f(lib, gate=3) == -7                       # unknown gate source
    assert b"gate" in lib.kda_last_error()
    assert f(lib, pre=16) == -7                       # unknown preprocessing bit
    assert f(lib, pre=8) == -7                        # doubled beta without the sigmoid
    assert b"NEG_EIGVAL" in lib.kda_last_error()
    assert f(lib, A=FAKE) == -7                       # activation arguments with a log2 gate
    assert f(lib, hlb=1, lb=-1.0) == -7
    assert f(lib, gate=2, A=None) == -1               # raw gate: A_log required
    assert f(lib, gate=1, A=FAKE, dt=FAKE + 4) == -2  # misaligned dt_bias
    assert f(lib, gate=2, A=FAKE, hlb=1, lb=0.0) == -2
    assert f(lib, gate=2, A=FAKE, g=None) == -1       # the raw gate itself
    assert f(lib, gate=2, A=FAKE, g=FAKE + 8) == -2


def test_chunk_ex_then_chunk_checks(lib):
    # valid options, then the chunked path's own checks as usual
    ok = dict(gate=2, A=FAKE, dt=FAKE, hlb=1, lb=-5.0, pre=15)
    assert _ex(lib, cs=32, **ok) == -4
    assert _ex(lib, ws=None, **ok) == -5
    assert _rec_ex(lib, K=32, **ok) == -4
    assert _ex(lib, cu=FAKE, N=0, T=0, **ok) == 0
    assert _rec_ex(lib, cu=FAKE, N=0, T=0, **ok) == 0
    assert lib.kda_last_error().decode() == ""


def test_gated_specific_rejects(lib):
    assert _gated(lib, gd=7) == -3                    # raw gate dtype
    assert b"g_dtype" in lib.kda_last_error()
    assert _gated(lib, A=None) == -1                  # A_log required
    assert _gated(lib, g=None) == -1                  # the raw gate itself
    assert _gated(lib, dt=FAKE + 4) == -2             # misaligned dt_bias
    assert _gated(lib, hlb=1, lb=0.5) == -2           # a lower bound must be negative
    assert _gated(lib, hlb=1, lb=float("nan")) == -2
    assert _gated(lib, hlb=1, lb=float("-inf")) == -2
    assert _gated(lib, cs=32) == -4                   # then the chunk checks as usual
    assert _gated(lib, ws=None) == -5


def test_chunk_specific_rejects(lib):
    assert _chunk(lib, cs=32) == -4
    assert b"chunk_size" in lib.kda_last_error()
    assert _chunk(lib, K=96) == -4
    assert _chunk(lib, V=256) == -4
    assert _chunk(lib, ws=None) == -5
    assert _chunk(lib, wsb=16) == -5
    assert _chunk(lib, ws=FAKE + 16) == -5


def test_recurrent_specific_rejects(lib):
    assert _rec(lib, K=32) == -4
    assert _rec(lib, V=96) == -4


def test_empty_problem_is_a_noop(lib):
    # N = 0 sequences: nothing to do, nothing enqueued
    assert _chunk(lib, cu=FAKE, N=0, T=0) == 0
    assert _rec(lib, cu=FAKE, N=0, T=0) == 0
    assert _gated(lib, cu=FAKE, N=0, T=0) == 0
    assert lib.kda_last_error().decode() == ""


def test_binding_rejects_bad_tensors():
    import torch
    from gated_delta_rule_64_amd import kda_chunk_fwd
    q = torch.zeros(1, 64, 2, 128)
    with pytest.raises(ValueError):
        kda_chunk_fwd(q, q, torch.zeros(1, 64, 2, 128), torch.zeros(1, 64, 2, 128),
                      torch.zeros(1, 64, 2))
    with pytest.raises(TypeError):
        kda_chunk_fwd(q, q, torch.zeros(1, 64, 2, 128), torch.zeros(1, 64, 2, 128, dtype=torch.float64),
                      torch.zeros(1, 64, 2))


@pytest.mark.parametrize("fn", ["kda_chunk_bwd", "kda_chunk_bwd_saved"])
@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_bwd_rejects_common(lib, name, kw, code, fn):
    assert _bwd(lib, fn, **kw) == code
    assert lib.kda_last_error().decode() != ""


@pytest.mark.parametrize("fn", ["kda_chunk_bwd", "kda_chunk_bwd_saved"])
def test_bwd_specific_rejects(lib, fn):
    for out in ("do", "dq", "dk", "dv", "dg", "db"):
        assert _bwd(lib, fn, **{out: None}) == -1, out
    assert _bwd(lib, fn, dht=FAKE + 4) == -2
    assert _bwd(lib, fn, cs=32) == -4
    assert _bwd(lib, fn, K=96) == -4
    assert _bwd(lib, fn, V=256) == -4
    assert _bwd(lib, fn, ws=None) == -5
    assert _bwd(lib, fn, wsb=16) == -5
    assert _bwd(lib, fn, ws=FAKE + 16) == -5
    assert _bwd(lib, fn, cu=FAKE, N=0, T=0) == 0
    assert lib.kda_last_error().decode() == ""


@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_train_forward_rejects_common(lib, name, kw, code):
    assert _train(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


def test_train_forward_specific_rejects(lib):
    """The training forward takes the backward's workspace (its size, not the forward's),
    needs o, and checks o and the final state like kda_chunk_fwd."""
    B, T, H, HV, K, V = 1, 64, 2, 2, 128, 128
    fwd_bytes = lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, B, 0, 1)
    bwd_bytes = lib.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, B, 0, 1)
    assert bwd_bytes > fwd_bytes
    assert _train(lib, o=None) == -1
    assert _train(lib, o=FAKE + 4) == -2
    assert _train(lib, fs=FAKE + 4) == -2
    assert _train(lib, cs=32) == -4
    assert _train(lib, K=96) == -4
    assert _train(lib, ws=None) == -5
    assert _train(lib, wsb=fwd_bytes) == -5
    assert b"need %d" % bwd_bytes in lib.kda_last_error()
    assert _train(lib, ws=FAKE + 16) == -5
    assert _train(lib, cu=FAKE, N=0, T=0) == 0
    assert lib.kda_last_error().decode() == ""


def _bwd_ex(lib, fn="kda_chunk_bwd_ex", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gate=0, A=None, dt=None, hlb=0, lb=0.0, beta=FAKE,
             pre=0, h0=None, cu=None, N=1, do=FAKE, dht=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE,
             db=FAKE, dh0=None, dA=None, ddt=None, B=1, T=64, H=2, HV=2, K=128, V=128, qd=1, bd=1,
             scale=0.0, cs=64, ws=FAKE, wsb=1 << 40, st=None, stream=None)
    a.update(kw)
    return getattr(lib, fn)(a["q"], a["k"], a["v"], a["g"], a["gate"], a["A"], a["dt"], a["hlb"],
                            a["lb"], a["beta"], a["pre"], a["h0"], a["cu"], a["N"], a["do"], a["dht"],
                            a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dh0"], a["dA"], a["ddt"],
                            a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["qd"], a["bd"],
                            a["scale"], a["cs"], a["ws"], a["wsb"], a["st"], a["stream"])


def _train_ex(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gate=0, A=None, dt=None, hlb=0, lb=0.0, beta=FAKE,
             pre=0, h0=None, cu=None, N=1, o=FAKE, ht=None, B=1, T=64, H=2, HV=2, K=128, V=128,
             qd=1, bd=1, scale=0.0, cs=64, ws=FAKE, wsb=1 << 40, st=None, stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_ex_train(a["q"], a["k"], a["v"], a["g"], a["gate"], a["A"], a["dt"],
                                      a["hlb"], a["lb"], a["beta"], a["pre"], a["h0"], a["cu"], a["N"],
                                      a["o"], a["ht"], a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"],
                                      a["qd"], a["bd"], a["scale"], a["cs"], a["ws"], a["wsb"],
                                      a["st"], a["stream"])


@pytest.mark.parametrize("call", ["kda_chunk_bwd_ex", "kda_chunk_bwd_ex_saved", "kda_chunk_fwd_ex_train"])
@pytest.mark.parametrize("name,kw,code", CASES, ids=[c[0] for c in CASES])
def test_bwd_ex_and_train_ex_reject_common(lib, name, kw, code, call):
    f = _train_ex if call == "kda_chunk_fwd_ex_train" else (lambda l, **k: _bwd_ex(l, call, **k))
    assert f(lib, **kw) == code
    assert lib.kda_last_error().decode() != ""


@pytest.mark.parametrize("fn", ["kda_chunk_bwd_ex", "kda_chunk_bwd_ex_saved"])
def test_bwd_ex_specific_rejects(lib, fn):
    for out in ("do", "dq", "dk", "dv", "dg", "db"):
        assert _bwd_ex(lib, fn, **{out: None}) == -1, out
    raw = dict(gate=2, A=FAKE, dA=FAKE)
    assert _bwd_ex(lib, fn, **dict(raw, dA=None)) == -1           # dA_log with a raw gate
    assert _bwd_ex(lib, fn, **dict(raw, dt=FAKE)) == -1           # ddt_bias with dt_bias
    assert _bwd_ex(lib, fn, **dict(raw, dt=FAKE, ddt=FAKE + 4)) == -2
    assert _bwd_ex(lib, fn, gate=3) == -7
    assert _bwd_ex(lib, fn, pre=8) == -7
    assert _bwd_ex(lib, fn, cs=32) == -4
    assert _bwd_ex(lib, fn, K=96) == -4
    assert _bwd_ex(lib, fn, ws=None) == -5
    assert _bwd_ex(lib, fn, wsb=16) == -5
    assert _bwd_ex(lib, fn, ws=FAKE + 16) == -5
    assert _bwd_ex(lib, fn, cu=FAKE, N=0, T=0, **dict(raw, dt=FAKE, ddt=FAKE, pre=15)) == 0
    assert lib.kda_last_error().decode() == ""


def test_train_ex_forward_specific_rejects(lib):
    """The fused-option training forward takes kda_chunk_bwd_ex's workspace and needs o;
    no gradient outputs are asked for."""
    B, T, H, HV, K, V = 1, 64, 2, 2, 128, 128
    need = lib.kda_chunk_bwd_ex_workspace_bytes(B, T, H, HV, K, V, B, 0, 1)
    assert need > lib.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, B, 0, 1)
    assert _train_ex(lib, o=None) == -1
    assert _train_ex(lib, o=FAKE + 4) == -2
    assert _train_ex(lib, ht=FAKE + 4) == -2
    assert _train_ex(lib, gate=3) == -7
    assert _train_ex(lib, gate=2, A=None) == -1
    assert _train_ex(lib, cs=32) == -4
    assert _train_ex(lib, ws=None) == -5
    assert _train_ex(lib, wsb=need - 1) == -5
    assert b"need %d" % need in lib.kda_last_error()
    ok = dict(gate=2, A=FAKE, dt=FAKE, hlb=1, lb=-5.0, pre=15)
    assert _train_ex(lib, cu=FAKE, N=0, T=0, **ok) == 0
    assert lib.kda_last_error().decode() == ""


def test_bwd_workspace_bytes(lib):
    """The forward's schedule and records (in the recompute's layout), then per (value
    head, chunk) fp32 checkpoints, reverse-scan operands and intermediates, then
    per-value-head dq, dk."""
    B, T, H, HV, K, V = 2, 4096 + 17, 4, 8, 128, 128
    nt = (T + 63) // 64
    items = HV * B * nt
    al = lambda x: (x + 255) // 256 * 256
    # the recompute's schedule and records (bf16 residual tiles)
    off = al(_sched_bytes(B, B * nt) + items * _rec_bytes(K, V, 2))
    for per in (K * V, 64 * V, 2 * 64 * 64, K * V, 64 * V, 2 * 64 * K + 64 * V + K * V,
                3 * 64 * K + 64 * 64 + K, 64 * K + 64 * 64):
        off = al(off + items * per * 4)
    for _ in range(2):
        off = al(off + B * T * HV * K * 4)
    assert lib.kda_chunk_bwd_workspace_bytes(B, T, H, HV, K, V, B, 0, 1) == off
    assert lib.kda_chunk_bwd_workspace_bytes(1, 64, 1, 1, 96, 128, 1, 0, 1) == 0


def test_recurrent_ex_layout_and_intermediate_rejects(lib):
    assert _rec_ex(lib, lay=2) == -7
    assert b"state_layout" in lib.kda_last_error()
    assert _rec_ex(lib, inter=FAKE + 4) == -2
    assert _rec_ex(lib, lay=1, inter=FAKE, cu=FAKE, N=0, T=0) == 0


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (128, 64)])
def test_bench_record_bytes_match_the_library_layout(lib, K, V):
    """The bench prices the Stage 1+2 and scan kernels with its own count of one record's
    bytes; it must equal the record stride of the library's workspace layout (the
    workspace grows by exactly HV records per added chunk of a dense sequence)."""
    import bench
    B, H, HV, nt = 1, 2, 4, 41
    total = lib.kda_chunk_fwd_workspace_bytes(B, 64 * nt, H, HV, K, V, B, 0, 1)
    records = total - _sched_bytes(B, B * nt)
    assert records % (HV * nt) == 0
    rec = records // (HV * nt)
    # the library pads each record to 256 bytes; the bench counts the bytes it holds
    assert rec == (bench.record_bytes(K, V, 2) + 255) // 256 * 256
    assert rec - bench.record_bytes(K, V, 2) < 256


def test_bwd_rejects_misaligned_gradient_buffers(lib):
    # every buffer the backward kernels read or write with vector accesses
    for name in ("do", "dq", "dk", "dg", "db"):
        assert _bwd(lib, **{name: FAKE + 4}) == -2, name
        assert b"16-byte aligned" in lib.kda_last_error()


def _noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=1, o=FAKE, ht=None,
             B=1, T=64, H=2, HV=2, K=128, V=128, qd=1, bd=1, scale=0.0, cs=64, st=None,
             stream=None)
    a.update(kw)
    return lib.kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"],
                                     a["N"], a["o"], a["ht"], a["B"], a["T"], a["H"], a["HV"],
                                     a["K"], a["V"], a["qd"], a["bd"], a["scale"], a["cs"],
                                     a["st"], a["stream"])


def test_noalloc_scratch_limit(lib):
    """The allocation-free entry point holds KDA_NOALLOC_SCRATCH_MB MiB per GPU; a problem
    whose intermediates exceed it is rejected on the host before any GPU call."""
    cap = lib.kda_noalloc_scratch_bytes()
    assert cap == _header_int("KDA_NOALLOC_SCRATCH_MB") << 20
    # the long-context problem (538 MB of records) is far beyond it
    assert _noalloc(lib, T=8192, H=16, HV=32) == -5
    assert b"allocation-free" in lib.kda_last_error()
    # the largest dense T at H=2 HV=8 that fits, and the next chunk that does not
    fits = [T for T in range(64, 1 << 16, 64)
            if lib.kda_chunk_fwd_workspace_bytes(1, T, 2, 8, 128, 128, 1, 0, 1) <= cap]
    assert _noalloc(lib, T=fits[-1] + 64, HV=8) == -5
    # argument errors inside the limit are the forward's own (checked before any GPU call)
    assert _noalloc(lib, q=None) == -1
    assert _noalloc(lib, cs=32) == -4
    assert _noalloc(lib, cu=FAKE, N=0, T=0) == 0


def test_binding_checks_caller_buffers():
    """Buffers the caller passes in (out, final_state, intermediate states, workspace,
    dev_status) must fit the problem exactly: the C ABI cannot see their sizes."""
    import torch
    from gated_delta_rule_64_amd import _lib
    dev = torch.device("cuda:0")   # never touched: the shape and dtype checks come first
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(1, 64, 4, 128, dtype=torch.bfloat16)
    N, HV, K, V = 1, 4, 128, 128
    ok_out = torch.zeros_like(v)
    # o: v's shape in q's dtype
    with pytest.raises(ValueError, match="out"):
        _lib._fwd_outputs(q, v, N, HV, K, V, dev, torch.zeros(1, 64, 4, 64, dtype=torch.bfloat16), None, False)
    with pytest.raises(TypeError, match="out"):
        _lib._fwd_outputs(q, v, N, HV, K, V, dev, torch.zeros(1, 64, 4, 128), None, False)
    # final state: fp32 [N, HV, K, V], or the transposed layout when asked for
    with pytest.raises(ValueError, match="final_state"):
        _lib._fwd_outputs(q, v, N, HV, K, V, dev, ok_out, torch.zeros(N, HV, V, K + 1), True)
    with pytest.raises(TypeError, match="final_state"):
        _lib._fwd_outputs(q, v, N, HV, K, V, dev, ok_out, torch.zeros(N, HV, K, V, dtype=torch.float64), True)
    with pytest.raises(ValueError, match="final_state"):
        _lib._fwd_outputs(q, v, N, HV, K, V, dev, ok_out, torch.zeros(N, HV, K, V), True,
                          state_shape=(N, HV, V, K + 1))
    # intermediate states, dev_status
    with pytest.raises(ValueError, match="intermediate_states"):
        _lib._check_buffers(dev, [("intermediate_states", torch.zeros(63, HV, K, V), (64, HV, K, V), torch.float32)])
    with pytest.raises(TypeError, match="dev_status"):
        _lib._check_buffers(dev, [], dev_status=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(TypeError, match="dev_status"):
        _lib._check_buffers(dev, [], dev_status=torch.zeros(0, dtype=torch.int32))
    # host tensors are refused once shapes and dtypes pass
    with pytest.raises(ValueError, match="workspace"):
        _lib._check_buffers(dev, [], workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dev_status"):
        _lib._check_buffers(dev, [], dev_status=torch.zeros(1, dtype=torch.int32))


def test_binding_input_table_messages():
    """Each input is checked against its layout and named in the error."""
    import torch
    from gated_delta_rule_64_amd import kda_chunk_fwd, kda_recurrent_fwd_ex
    bf = torch.bfloat16
    q = torch.zeros(1, 64, 2, 128, dtype=bf)
    v = torch.zeros(1, 64, 4, 128, dtype=bf)
    g = torch.zeros(1, 64, 4, 128)
    b = torch.zeros(1, 64, 4, dtype=bf)
    with pytest.raises(ValueError, match="^k:"):
        kda_chunk_fwd(q, torch.zeros(1, 64, 2, 64, dtype=bf), v, g, b)
    with pytest.raises(TypeError, match="^v:"):
        kda_chunk_fwd(q, q, v.float(), g, b)
    with pytest.raises(ValueError, match="^g:"):
        kda_chunk_fwd(q, q, v, torch.zeros(1, 64, 2, 128), b)
    with pytest.raises(TypeError, match="^g:"):
        kda_chunk_fwd(q, q, v, g.to(bf), b)
    with pytest.raises(ValueError, match="^beta:"):
        kda_chunk_fwd(q, q, v, g, torch.zeros(1, 64, 2, dtype=bf))
    with pytest.raises(ValueError, match="^initial_state:"):
        kda_chunk_fwd(q, q, v, g, b, torch.zeros(1, 4, 128, 64))
    with pytest.raises(TypeError, match="^cu_seqlens:"):
        kda_chunk_fwd(q, q, v, g, b, None, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="B must be 1"):
        kda_chunk_fwd(q.expand(2, -1, -1, -1), q.expand(2, -1, -1, -1), v.expand(2, -1, -1, -1),
                      g.expand(2, -1, -1, -1), b.expand(2, -1, -1), None, torch.zeros(2, dtype=torch.int32))
    # the transposed decode layout checks the initial state as [N, HV, V, K]
    vv = torch.zeros(1, 64, 4, 64, dtype=bf)
    with pytest.raises(ValueError, match="^initial_state:"):
        kda_recurrent_fwd_ex(q, q, vv, g, b, torch.zeros(1, 4, 128, 64), state_layout="vk")
    # all shapes right: then the host tensors are refused
    with pytest.raises(ValueError, match="GPU tensor"):
        kda_recurrent_fwd_ex(q, q, vv, g, b, torch.zeros(1, 4, 64, 128), state_layout="vk")
