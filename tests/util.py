"""Helpers for the GPU parity tests: tolerance checks against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

FP32_ATOL = 1e-4        # max-abs bound for fp32 inputs
BF16_RMS_FRAC = 2e-2    # max-abs bound relative to RMS of the oracle output for bf16 inputs


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(x):
    return x.detach().to("cpu").double().numpy()


def max_err(got, want, mask=None):
    got = to64(got) if isinstance(got, torch.Tensor) else got
    if mask is not None:
        got, want = got[mask], want[mask]
    return float(np.abs(got - want).max()) if got.size else 0.0


def half_ulp_bf16(x):
    """Half a unit in the last place of bf16 (8 significant bits) at each value of x."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def check(name, got, want, dtype, mask=None, want_rounded=False):
    """Assert the tolerance of the input precision; returns (err, bound).

    fp32 inputs: max|got - want| <= 1e-4.
    bf16 inputs: max|got - want| <= 2e-2 * RMS(want) on the arithmetic; when ``got`` is
    itself stored in bf16 (the output o), each element may in addition differ by the
    half-ulp that rounding the exact value to bf16 costs (the output dtype is fixed by
    the contract, so that rounding is not error of the computation). When ``want`` is a
    bf16-stored output too (``want_rounded``: two GPU paths compared with each other),
    each side carries its own half-ulp, so the allowance is one ulp.
    """
    stored_bf16 = isinstance(got, torch.Tensor) and got.dtype == torch.bfloat16
    got = to64(got) if isinstance(got, torch.Tensor) else got
    if mask is not None:
        got, want = got[mask], want[mask]
    if got.size == 0:
        return 0.0, 0.0
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    diff = np.abs(got - want)
    err = float(diff.max())
    if dtype == torch.float32:
        bound = FP32_ATOL
        excess = err
    else:
        bound = BF16_RMS_FRAC * float(np.sqrt(np.mean(want ** 2)))
        allow = half_ulp_bf16(want) * (2.0 if want_rounded else 1.0)
        excess = float((diff - allow).max()) if stored_bf16 else err
    log(f"  {name}: max|err| = {err:.3e}  beyond output rounding = {excess:.3e}  "
        f"bound = {bound:.3e}  ratio = {excess / max(bound, 1e-300):.3f}")
    assert excess <= bound, f"{name}: error {excess:.3e} > {bound:.3e}"
    return excess, bound


def valid_rows(cu, T):
    """Boolean [T] mask of rows that belong to some sequence."""
    m = np.zeros(T, dtype=bool)
    cu = [int(x) for x in cu]
    for a, b in zip(cu[:-1], cu[1:]):
        m[a:b] = True
    return m


def to_device(d, device="cuda"):
    out = {}
    for k, v in d.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def frag_tile_index(R, KC, ks, kpl):
    """Element offsets of a fragment-order tile (see the record layout in the library):
    64-lane blocks per (16-row band b, contraction step st), band-major; lane
    l = row % 16 + 16 * ((col % ks) // kpl) holds kpl consecutive columns."""
    row = np.arange(R)[:, None]
    col = np.arange(KC)[None, :]
    b, st = row // 16, col // ks
    lane = row % 16 + 16 * ((col % ks) // kpl)
    return ((b * (KC // ks) + st) * 64 + lane) * kpl + col % kpl


def acc_tile_index(R, NCOL):
    """Element offsets of an accumulator-order fp32 tile holding x[row][col] for rows
    0..R-1 (R = 64) and columns 0..NCOL-1, four consecutive rows of one column per lane."""
    row = np.arange(R)[:, None]
    col = np.arange(NCOL)[None, :]
    return (((col // 16) * 4 + row // 16) * 64 + col % 16 + 16 * ((row % 16) // 4)) * 4 + row % 4


def _e4m3_value(code):
    """OCP FP8 E4M3 (exponent bias 7, no infinities, S.1111.111 is NaN)."""
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of each of the 256 e4m3 codes (decoding residual tiles stored in fp8)
E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)])
