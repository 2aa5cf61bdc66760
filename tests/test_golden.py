"""The oracle still reproduces its committed regression fixture bit for bit."""
import os

import numpy as np

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_regression_fixture():
    ref = np.load(os.path.join(HERE, "oracle_regression.npz"))
    got = make_golden.compute()
    for key in ("dense_o", "dense_ht", "packed_o", "packed_ht"):
        a, b = ref[key], got[key]
        assert a.shape == b.shape
        assert np.array_equal(np.isnan(a), np.isnan(b))
        assert np.array_equal(np.nan_to_num(a), np.nan_to_num(b)), key
