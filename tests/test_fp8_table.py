"""The e4m3 decoding table the GPU record tests use, against facts of the OCP FP8
E4M3 format: largest finite value 448, smallest normal 2^-6, smallest subnormal 2^-9,
1.0 at code 0x38, one NaN code per sign, sign in bit 7, codes increasing in value."""
import numpy as np

from tests.util import E4M3_VALUES


def test_e4m3_table_fixed_points():
    v = E4M3_VALUES
    assert v[0x00] == 0.0 and v[0x80] == 0.0
    assert v[0x01] == 2.0 ** -9
    assert v[0x07] == 7 * 2.0 ** -9          # largest subnormal
    assert v[0x08] == 2.0 ** -6              # smallest normal
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2


def test_e4m3_table_order_and_sign():
    pos = E4M3_VALUES[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(E4M3_VALUES[0x80:0xFF], -pos)
    # 3 mantissa bits: within a binade the step is 2^(e - 3)
    assert E4M3_VALUES[0x39] - E4M3_VALUES[0x38] == 2.0 ** -3
