"""Pins for the oracle's GEMM and argmax (CPU only).

The dequantised weights are rebuilt here from the golden E2M1 table and
torch's E4M3 decode (not from the oracle's decoders); products are then
checked against exact rational sums (fractions), correctly rounded sums
(math.fsum), numpy's float64 matmul, one-hot and constant special cases.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from golden_io import code_value_table

E2M1 = dict(code_value_table("e2m1_values.txt"))
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _indep_dequant_nvfp4(codes, scales, g):
    n, k2 = codes.shape
    k = 2 * k2
    out = np.zeros((n, k))
    for r in range(n):
        for i in range(k):
            b = int(codes[r, i // 2])
            c = (b & 0xF) if i % 2 == 0 else (b >> 4)
            out[r, i] = E2M1[c] * float(E4M3[int(scales[r, i // 16])]) * float(g)
    return out


def _indep_dequant_fp8(codes, rs):
    return E4M3[codes.astype(np.int64)] * rs.astype(np.float64)[:, None]


def _x_f64(x):
    return x.astype(np.float64)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 8), st.sampled_from([16, 32, 48]), st.integers(1, 8),
       st.integers(0, 2 ** 31 - 1))
def test_nvfp4_gemm_exact_rational_small(m, k, n, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (n, k // 16), dtype=np.uint8)
    g = np.float32(rng.uniform(1e-4, 10.0))
    x = (rng.standard_normal((m, k)) * 3).astype(np.float16)
    y = oracle.gemm_nvfp4(codes, scales, g, x)
    wh = _indep_dequant_nvfp4(codes, scales, g)
    xf = _x_f64(x)
    for mi in range(m):
        for r in range(n):
            terms = [xf[mi, i] * wh[r, i] for i in range(k)]
            exact = sum((Fraction(float(xf[mi, i])) * Fraction(float(wh[r, i])) for i in range(k)),
                        Fraction(0))
            # every product is exact in FP64; only the running sum rounds
            assert all(Fraction(t) == Fraction(float(xf[mi, i])) * Fraction(float(wh[r, i]))
                       for i, t in enumerate(terms))
            bound = (k - 1) * 2.0 ** -53 * sum(abs(t) for t in terms) * (1 + 1e-9)
            assert abs(Fraction(y[mi, r]) - exact) <= Fraction(bound)
            assert abs(y[mi, r] - math.fsum(terms)) <= bound


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 8), st.sampled_from([1, 16, 33]), st.integers(1, 8),
       st.integers(0, 2 ** 31 - 1))
def test_fp8_gemm_exact_rational_small(m, k, n, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11  # no NaN codes
    rs = rng.uniform(1e-5, 1.0, n).astype(np.float32)
    x = (rng.standard_normal((m, k)) * 3).astype(np.float16)
    y = oracle.gemm_fp8(codes, rs, x)
    wh = _indep_dequant_fp8(codes, rs)
    xf = _x_f64(x)
    for mi in range(m):
        for r in range(n):
            exact = sum((Fraction(float(xf[mi, i])) * Fraction(float(wh[r, i])) for i in range(k)),
                        Fraction(0))
            bound = (k - 1) * 2.0 ** -53 * float(np.abs(xf[mi] * wh[r]).sum()) * (1 + 1e-9)
            assert abs(Fraction(y[mi, r]) - exact) <= Fraction(bound)


def test_dequant_matches_independent_tables():
    w = synth.weights(12, 64, seed=21)
    codes, scales, g = oracle.pack_nvfp4(w)
    assert np.array_equal(oracle.dequant_nvfp4(codes, scales, g),
                          _indep_dequant_nvfp4(codes, scales, g))
    c8, rs = oracle.pack_fp8(w)
    assert np.array_equal(oracle.dequant_fp8(c8, rs), _indep_dequant_fp8(c8, rs))


def test_nvfp4_gemm_matches_numpy_matmul():
    n, k = 96, 512
    w = synth.weights(n, k, seed=1)
    x = synth.activations(8, k, seed=1)
    codes, scales, g = oracle.pack_nvfp4(w)
    y = oracle.gemm_nvfp4(codes, scales, g, x)
    ref = x.astype(np.float64) @ _indep_dequant_nvfp4(codes, scales, g).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())
    # the dequantise-then-multiply path of the oracle agrees too
    y2 = oracle.gemm_f64(oracle.dequant_nvfp4(codes, scales, g), x)
    assert np.array_equal(y, y2)


def test_fp8_gemm_matches_numpy_matmul():
    n, k = 80, 320
    w = synth.weights(n, k, seed=4)
    x = synth.activations(4, k, seed=4)
    codes, rs = oracle.pack_fp8(w)
    y = oracle.gemm_fp8(codes, rs, x)
    ref = x.astype(np.float64) @ _indep_dequant_fp8(codes, rs).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


def test_one_hot_activation_selects_a_column():
    n, k = 20, 64
    w = synth.weights(n, k, seed=8)
    codes, scales, g = oracle.pack_nvfp4(w)
    wh = _indep_dequant_nvfp4(codes, scales, g)
    c8, rs = oracle.pack_fp8(w)
    wh8 = _indep_dequant_fp8(c8, rs)
    for col in (0, 1, 15, 16, 33, 63):
        x = np.zeros((1, k), np.float16)
        x[0, col] = 1.0
        assert np.array_equal(oracle.gemm_nvfp4(codes, scales, g, x)[0], wh[:, col])
        assert np.array_equal(oracle.gemm_fp8(c8, rs, x)[0], wh8[:, col])


def test_unit_codes_give_row_sums():
    # every code 0x2 (1.0), every scale 0x38 (1.0), g = 1: y = sum_k x[m, k]
    n, k, m = 5, 64, 3
    codes = np.full((n, k // 2), 0x22, np.uint8)
    scales = np.full((n, k // 16), 0x38, np.uint8)
    x = synth.activations(m, k, seed=3)
    y = oracle.gemm_nvfp4(codes, scales, np.float32(1.0), x)
    for mi in range(m):
        assert y[mi, 0] == pytest.approx(math.fsum(x[mi].astype(np.float64)), abs=1e-12)
        assert np.all(y[mi] == y[mi, 0])


def test_linearity():
    # activations on a 1/8 grid in [-4, 4]: x1 + x2 is exact in fp16
    n, k = 16, 128
    w = synth.weights(n, k, seed=12)
    codes, scales, g = oracle.pack_nvfp4(w)
    rng = np.random.default_rng(12)
    x = (rng.integers(-32, 33, (2, k)) / 8.0).astype(np.float16)
    xs = (x[0:1].astype(np.float32) + x[1:2].astype(np.float32)).astype(np.float16)
    y = oracle.gemm_nvfp4(codes, scales, g, x)
    ys = oracle.gemm_nvfp4(codes, scales, g, xs)
    assert np.allclose(ys[0], y[0] + y[1], rtol=1e-12, atol=1e-14)


def test_argmax_lowest_index_and_signed_zero():
    lg = np.array([[1, 3, 3, 2], [-0.0, 0.0, -1, -0.0], [-5, -4, -4, -9], [np.inf, 1, np.inf, 0]],
                  np.float16)
    got = oracle.argmax_f16(lg)
    assert list(got) == [1, 0, 1, 0]
    rng = np.random.default_rng(0)
    for _ in range(50):
        lg = rng.integers(-3, 4, (4, 37)).astype(np.float16)
        assert list(oracle.argmax_f16(lg)) == list(np.argmax(lg, axis=1))


def test_duplicate_rows_tie_to_lower_index():
    n, k = 48, 64
    w = synth.weights(n, k, seed=30)
    x = synth.activations(8, k, seed=30)
    codes, scales, g = oracle.pack_nvfp4(w)
    y0 = oracle.gemm_nvfp4(codes, scales, g, x)
    best = np.argmax(y0, axis=1)
    # copy row best[0] into a later row and an earlier row
    b = int(best[0])
    src = b
    dst = (b + 17) % n
    codes[dst] = codes[src]
    scales[dst] = scales[src]
    y, am = oracle.lmhead_nvfp4(codes, scales, g, x)
    assert np.array_equal(y[:, dst], y[:, src])
    assert am[0] == min(src, dst)


# ---- greedy speculative verification (oracle.greedy_verify) -----------------
# Worked by hand from the rule: accept drafts while each equals the target's
# greedy token for its position; the next token is the target's token at the
# first position not accepted (a bonus token when every draft is accepted).
VERIFY_CASES = [
    # argmax (m rows)          drafts (m - 1)        accepted, next
    ([5, 7, 9, 2], [5, 7, 1], (2, 9)),
    ([5, 7, 9, 2], [5, 7, 9], (3, 2)),      # all accepted: bonus token
    ([5, 7, 9, 2], [4, 7, 9], (0, 5)),      # first draft rejected
    ([5, 7, 9, 2], [5, 1, 9], (1, 7)),      # a later match does not count
    ([3], [], (0, 3)),                       # M = 1: plain greedy decode
    ([0, 0, 0, 0, 0, 0, 0, 0], [0] * 7, (7, 0)),
    ([1, 2, 3, 4, 5, 6, 7, 8], [1, 2, 3, 4, 5, 6, 0], (6, 7)),
]


@pytest.mark.parametrize("argmax,draft,want", VERIFY_CASES)
def test_greedy_verify_worked_examples(argmax, draft, want):
    assert oracle.greedy_verify(argmax, draft) == want


@given(st.integers(1, 8).flatmap(lambda m: st.tuples(
    st.lists(st.integers(0, 3), min_size=m, max_size=m),
    st.lists(st.integers(0, 3), min_size=m - 1, max_size=m - 1))))
@settings(max_examples=300, deadline=None)
def test_greedy_verify_prefix_property(case):
    # characterised without the oracle's loop: the accepted drafts are exactly
    # a matching prefix, and it cannot be extended
    argmax, draft = case
    acc, nxt = oracle.greedy_verify(argmax, draft)
    assert 0 <= acc <= len(draft)
    assert draft[:acc] == argmax[:acc]
    assert acc == len(draft) or draft[acc] != argmax[acc]
    assert nxt == argmax[acc]


def test_greedy_verify_rejects_wrong_draft_count():
    with pytest.raises(ValueError):
        oracle.greedy_verify([1, 2], [1, 2])
