"""Pins for the oracle's narrowing quantisers (FP32 -> E4M3 / E2M1 code).

E4M3 is pinned to torch's float32 -> float8_e4m3fn cast (round to nearest
even) wherever that cast does not overflow to NaN, and to saturation beyond.
E2M1 is pinned to a hand-worked tie table and to an independent formulation
with numpy's round-half-even integer rounding inside each binade.  Both get
round-trip, error-bound, monotonicity and sign-symmetry property checks.
"""
import math

import numpy as np
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from golden_io import value_code_table

f32 = st.floats(width=32, allow_nan=False, allow_infinity=False)


def _torch_e4m3(t):
    return int(torch.tensor([t], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(7)
    mags = np.exp(rng.uniform(np.log(2.0 ** -14), np.log(463.0), 40000)).astype(np.float32)
    signs = np.where(rng.random(40000) < 0.5, -1, 1).astype(np.float32)
    ts = list(mags * signs)
    # all exact midpoints between consecutive finite codes, and 1 ulp either side
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    for a, b in zip(vals, vals[1:]):
        m = np.float32((a + b) / 2)
        assert float(m) == (a + b) / 2
        ts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9)), -m]
    ts += [np.float32(v) for v in vals] + [np.float32(0.0), np.float32(-0.0), np.float32(1e-40)]
    for t in ts:
        t = np.float32(t)
        if abs(float(t)) >= 464.0:
            continue
        assert oracle.quant_e4m3(t) == _torch_e4m3(float(t)), float(t)


def test_e4m3_saturates_never_nan():
    for t in [448.0, 448.5, 463.9, 464.0, 464.1, 479.0, 480.0, 1e6, 3.4e38]:
        assert oracle.quant_e4m3(t) == 0x7E
        assert oracle.quant_e4m3(-t) == 0xFE
    assert oracle.quant_e4m3(float("inf")) == 0x7E
    assert oracle.quant_e4m3(float("nan")) == 0x00


def test_e2m1_hand_worked_ties():
    for t, code in value_code_table("e2m1_rounding.txt"):
        assert oracle.quant_e2m1(np.float32(t)) == code, t


def _e2m1_by_binade_rint(t):
    """Independent statement: RNE to the E2M1 grid via numpy.rint per binade."""
    a = abs(float(t))
    if a >= 6.0:
        q = 6.0
    elif a < 2.0:
        q = float(np.rint(a * 2.0)) / 2.0      # spacing 0.5 on [0, 2)
    elif a < 4.0:
        q = float(np.rint(a))                  # spacing 1 on [2, 4)
    else:
        q = 2.0 * float(np.rint(a / 2.0))      # spacing 2 on [4, 6]
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    code = mags.index(q)
    return code | (8 if math.copysign(1.0, float(t)) < 0 else 0)


@settings(max_examples=3000, deadline=None)
@given(f32)
def test_e2m1_matches_binade_rint(t):
    assert oracle.quant_e2m1(t) == _e2m1_by_binade_rint(t)


def test_e2m1_dense_grid_matches_binade_rint():
    for t in np.arange(-7.0, 7.0, 1.0 / 64, dtype=np.float64).astype(np.float32):
        assert oracle.quant_e2m1(t) == _e2m1_by_binade_rint(t), float(t)


def test_round_trip_every_code():
    for c in range(16):
        assert oracle.quant_e2m1(oracle.e2m1_value(c)) == c
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.quant_e4m3(oracle.e4m3_value(c)) == c


def _half_spacing_e4m3(a):
    if a < 2.0 ** -6:
        return 2.0 ** -10
    e = math.floor(math.log2(a))
    return 2.0 ** (e - 3) / 2


def _half_spacing_e2m1(a):
    return 0.25 if a < 2 else (0.5 if a < 4 else 1.0)


@settings(max_examples=3000, deadline=None)
@given(f32)
def test_e4m3_error_bound_and_sign(t):
    code = oracle.quant_e4m3(t)
    v = oracle.e4m3_value(code)
    a = abs(t)
    if a <= 448.0:
        assert abs(a - abs(v)) <= _half_spacing_e4m3(min(a, 447.99)) * (1 + 1e-12)
    else:
        assert abs(v) == 448.0
    assert (code >> 7) == (1 if math.copysign(1.0, t) < 0 else 0)
    assert oracle.quant_e4m3(-t) == code ^ 0x80


@settings(max_examples=3000, deadline=None)
@given(f32)
def test_e2m1_error_bound_and_sign(t):
    code = oracle.quant_e2m1(t)
    v = oracle.e2m1_value(code)
    a = abs(t)
    if a <= 6.0:
        assert abs(a - abs(v)) <= _half_spacing_e2m1(a)
    else:
        assert abs(v) == 6.0
    assert oracle.quant_e2m1(-t) == code ^ 0x8


@settings(max_examples=1000, deadline=None)
@given(f32, f32)
def test_monotonic(t1, t2):
    if t1 > t2:
        t1, t2 = t2, t1
    assert oracle.e4m3_value(oracle.quant_e4m3(t1)) <= oracle.e4m3_value(oracle.quant_e4m3(t2))
    assert oracle.e2m1_value(oracle.quant_e2m1(t1)) <= oracle.e2m1_value(oracle.quant_e2m1(t2))
