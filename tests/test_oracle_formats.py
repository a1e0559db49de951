"""Pins for the oracle's element-format decoders (CPU only).

E2M1 is pinned to the OCP value table (tests/golden/e2m1_values.txt), E4M3 to
torch's float8_e4m3fn decode of all 256 bytes plus the OCP landmarks, and the
FP16 helpers to numpy's float16 conversions.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from golden_io import code_value_table


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_all_16_codes_match_ocp_table():
    table = code_value_table("e2m1_values.txt")
    assert [c for c, _ in table] == list(range(16))
    for code, value in table:
        assert _same(oracle.e2m1_value(code), value), hex(code)


def test_e4m3_all_256_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for code in range(256):
        assert _same(oracle.e4m3_value(code), float(ref[code])), hex(code)


def test_e4m3_landmarks():
    for code, value in code_value_table("e4m3_landmarks.txt"):
        assert _same(oracle.e4m3_value(code), value), hex(code)
    nan_codes = [c for c in range(256) if math.isnan(oracle.e4m3_value(c))]
    assert nan_codes == [0x7F, 0xFF]


def test_format_maxima_agree_with_tensor_scale_constant():
    # The NVFP4 tensor scale divides by 6 * 448: the largest E2M1 magnitude
    # times the largest finite E4M3 (= UE4M3) magnitude.
    e2m1_max = max(abs(oracle.e2m1_value(c)) for c in range(16))
    e4m3_max = max(abs(v) for v in (oracle.e4m3_value(c) for c in range(256)) if not math.isnan(v))
    assert e2m1_max == 6.0 and e4m3_max == 448.0
    assert e2m1_max * e4m3_max == 2688.0


def test_positive_codes_are_monotonic():
    e2 = [oracle.e2m1_value(c) for c in range(8)]
    assert all(a < b for a, b in zip(e2, e2[1:]))
    e4 = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(e4, e4[1:]))
    # negative half mirrors the positive half
    for c in range(8):
        assert _same(oracle.e2m1_value(c | 8), -oracle.e2m1_value(c))
    for c in range(0x7F):
        assert _same(oracle.e4m3_value(c | 0x80), -oracle.e4m3_value(c))


def test_e4m3_binade_structure():
    # 8 equally spaced values per binade; subnormal spacing equals the first
    # normal binade's spacing (2^-9), so codes 0..0x0F are evenly spaced.
    vals = [oracle.e4m3_value(c) for c in range(0x7F)]
    for c in range(0x0F):
        assert vals[c + 1] - vals[c] == 2.0 ** -9
    for e in range(1, 16):
        base = e << 3
        top = min(base + 8, 0x7F)
        step = vals[base + 1] - vals[base]
        assert step == 2.0 ** (e - 7 - 3)
        for c in range(base, top - 1):
            assert vals[c + 1] - vals[c] == step


def test_ue4m3_valid_range():
    for b in range(256):
        v = oracle.ue4m3_value(b)
        if b <= 0x7E:
            assert v is not None and _same(v, oracle.e4m3_value(b))
        else:
            assert v is None, hex(b)


def test_f16_value_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in list(range(0, 65536, 1)):
        v = oracle.f16_value(b)
        r = float(ref[b])
        assert _same(v, r), hex(b)


def test_f16_round_matches_numpy_on_random_and_midpoints():
    rng = np.random.default_rng(123)
    vals = list(rng.standard_normal(20000) * np.exp(rng.uniform(-25, 12, 20000)))
    # exact midpoints between consecutive float16 values (ties), +- 1 ulp of
    # double around them, subnormal/normal boundary, overflow edge
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    hn = (np.arange(0, 0x7C00, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = (h + hn) / 2
    for m in mids:
        vals += [m, np.nextafter(m, 0), np.nextafter(m, np.inf)]
    vals += [0.0, -0.0, 65504.0, 65519.999, 65520.0, 65536.0, 1e30, -1e30, 2.0 ** -24, 2.0 ** -25,
             2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
             float("inf"), float("-inf")]
    for v in vals:
        got = oracle.f16_round(float(v))
        with np.errstate(over="ignore"):
            want = int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])
        assert got == want, (v, hex(got), hex(want))


def test_f16_round_nan():
    assert math.isnan(oracle.f16_value(oracle.f16_round(float("nan"))))
