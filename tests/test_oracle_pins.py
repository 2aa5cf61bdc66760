"""The fp64 oracle against what the mathematics fixes (no GPU needed)."""
import numpy as np
import pytest

import oracle
from oracle import chunked as chunked_ref
from tests import pins


def oracle_impl(q, k, v, g, beta, h0, cu, scale):
    return oracle.recurrent(q, k, v, g, beta, h0, cu, scale, nthreads=2)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)


def test_exact_K16():
    pins.pin_exact(oracle_impl, seed=21, B=1, T=5, H=1, HV=1, K=16, V=2)


def test_invalid_cu_seqlens_raises():
    q, k, v, g, beta, _ = pins.random_case(0, B=1, T=6, K=4, V=4)
    for cu in ([1, 3, 6], [0, 4, 2], [0, 3, 7], [0, -1, 6]):
        with pytest.raises(ValueError):
            oracle.recurrent(q, k, v, g, beta, None, np.array(cu, np.int32), 0.5)


def test_thread_count_independent():
    q, k, v, g, beta, h0 = pins.random_case(5, B=3, T=20, H=2, HV=4, K=8, V=8)
    a = oracle.recurrent(q, k, v, g, beta, h0, None, 0.3, nthreads=1)
    b = oracle.recurrent(q, k, v, g, beta, h0, None, 0.3, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("bt", [1, 3, 16, 64])
def test_chunked_equals_token(bt):
    """The chunk algebra (any chunk size, short last chunk) == the token recurrence."""
    q, k, v, g, beta, h0 = pins.random_case(30 + bt, B=2, T=150, H=2, HV=4, K=16, V=12, gate_lo=-4)
    o1, s1 = oracle.recurrent(q, k, v, g, beta, h0, None, 0.25)
    o2, s2 = chunked_ref.chunked(q, k, v, g, beta, h0, None, 0.25, chunk_size=bt)
    assert np.abs(o1 - o2).max() <= 1e-11 * max(1, np.abs(o1).max())
    assert np.abs(s1 - s2).max() <= 1e-11 * max(1, np.abs(s1).max())


def test_chunked_packed_and_extreme_decay():
    """Packed sequences (chunks restart at each start) at per-token gates down to -15."""
    r = np.random.default_rng(3)
    lens = [70, 0, 64, 1, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, _ = pins.random_case(4, B=1, T=int(cu[-1]) + 10, K=8, V=8, gate_lo=-15)
    h0 = r.standard_normal((len(lens), 1, 8, 8))
    o1, s1 = oracle.recurrent(q, k, v, g, beta, h0, cu, 0.4)
    o2, s2 = chunked_ref.chunked(q, k, v, g, beta, h0, cu, 0.4, chunk_size=64)
    valid = slice(0, int(cu[-1]))
    assert np.abs(o1[:, valid] - o2[:, valid]).max() <= 1e-11
    assert np.abs(s1 - s2).max() <= 1e-11
    assert np.isnan(o1[:, int(cu[-1]):]).all() and np.isnan(o2[:, int(cu[-1]):]).all()


def test_chunked_stage_identities():
    """Stage 2 outputs satisfy their defining equations: (I + L) Akk = I, Akk unit
    lower triangular, Aqk lower triangular with diagonal scale * q.k."""
    q, k, v, g, beta, _ = pins.random_case(9, B=1, T=64, K=16, V=8)
    _, _, st = chunked_ref.chunked(q, k, v, g, beta, None, None, 0.25, return_stages=True)
    s = st[0]
    C = 64
    assert np.allclose((np.eye(C) + s["L"]) @ s["Akk"], np.eye(C), atol=1e-12)
    assert np.allclose(np.triu(s["Akk"], 1), 0) and np.allclose(np.diag(s["Akk"]), 1)
    assert np.allclose(np.triu(s["Aqk"], 1), 0)
    assert np.allclose(np.diag(s["Aqk"]), 0.25 * np.sum(q[0, :, 0] * k[0, :, 0], -1))
