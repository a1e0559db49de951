"""The method's special cases through the contraction, against the oracle.

Weights with zero rows and blocks, negative-zero blocks, rows whose UE4M3
block scales are subnormal or round to zero, a constant-magnitude row, a
tie-heavy row and the saturated (scale 448) tensor-amax block go through the
NVFP4 and FP8 GEMMs (M = 1..8, with and without K splits), the lm_head
argmax and the prefill paths.  Power-of-two scaled copies of the tensor move
the tensor / row scale by exactly that power (the codes and block scales do
not change), and activations with FP16 subnormals, signed zeros and a few
columns near 3e4 exercise the FP16 operand range with outputs still inside
the FP16 range.

Scaled cases are compared after multiplying both the GPU output and the
oracle's FP64 output by the same power of two, which is exact, so the parity
bar stays relative to the outputs' size.  Outputs that underflow FP16
entirely (weights scaled by 2^-60) are compared bit for bit with the
oracle's FP16 rounding, signed zeros included.
"""
import numpy as np
import pytest

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import check_argmax, dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu


def special_weights(n, k, seed):
    """N(0, 0.02) weights with the special rows and blocks of the method."""
    rng = np.random.default_rng(seed)
    w = synth.weights(n, k, seed=seed)
    w[3, :] = 0.0                                               # zero row
    w[5, 32:48] = 0.0                                           # zero block
    w[6, 0:16] = -0.0                                           # negative-zero block
    w[7] *= np.float32(1e-30)                                   # block scales round to 0
    w[11] *= np.float32(2.0 ** -13)                             # subnormal UE4M3 block scales
    w[12, 16:32] = np.float32(2.0 ** -140)                      # FP32-subnormal weights
    w[9] = np.where(rng.random(k) < 0.5, -1, 1).astype(np.float32) * 0.07   # constant magnitude
    w[10, :] = np.float32(3.0e-2) * (np.arange(k) % 7 - 3).astype(np.float32)  # many ties
    w[20, 64:80] = np.float32(0.5)                              # the tensor amax block (scale 448)
    w[21, 64:80] = np.float32(-0.5)
    if n > 40:
        w[40] = w[9]                                            # duplicate row, another panel
    return w


def edge_activations(m, k, seed):
    """FP16 N(0, 1) rows with subnormals, signed zeros and large columns."""
    x = synth.activations(max(m, 8), k, seed=seed, m_max=max(m, 8))[:m].astype(np.float32)
    x[:, 8:40] *= np.float32(2.0 ** -16)                         # FP16 subnormals
    x[:, 40:44] = 0.0
    x[:, 44:48] = -0.0
    big = [100 % k, (3 * k) // 4]
    for i, c in enumerate(big):
        x[:, c] = np.float32(3.0e4) * (1 if i % 2 == 0 else -1)
    x = x.astype(np.float16)
    assert (np.abs(x[:, 8:40]) < np.float16(2.0 ** -14)).any()  # some subnormals present
    return x


def _oracle(fmt, w, x):
    if fmt == "nvfp4":
        codes, scales, g = oracle.pack_nvfp4(w)
        return oracle.gemm_nvfp4(codes, scales, g, x)
    codes, rs = oracle.pack_fp8(w)
    return oracle.gemm_fp8(codes, rs, x)


def _pack(qpn, fmt, w):
    return qpn.pack_nvfp4(dev(w)) if fmt == "nvfp4" else qpn.pack_fp8(dev(w))


def scaled_parity(y, y_ref, shift, what):
    """Parity of 2^shift * y against 2^shift * y_ref (both exact rescalings)."""
    assert np.abs(y_ref).max() < 6.0e4, f"{what}: outputs must stay in FP16 range"
    s = 2.0 ** shift
    return parity(np.asarray(y).astype(np.float64) * s, np.asarray(y_ref) * s, what)


# (weight exponent, activation exponent): outputs scale by 2^(a + b) and the
# comparison undoes that.  W * 2^20 needs smaller activations to stay in FP16.
SCALINGS = [(0, 0), (-20, 8), (20, -12)]
SHAPES = [(300, 2064), (300, 9008)]   # ragged panels and k-steps; the second splits K at M > 4


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", SHAPES)
def test_special_weights_gemm(fmt, n, k):
    qpn = need_gpu()
    base = special_weights(n, k, seed=n + k)
    x8 = synth.activations(8, k, seed=n + k)
    op = qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8
    for wexp, xexp in SCALINGS:
        w = base * np.float32(2.0 ** wexp)
        xs = (x8.astype(np.float32) * np.float32(2.0 ** xexp)).astype(np.float16)
        pw = _pack(qpn, fmt, w)
        for m in range(1, 9):
            pl = qpn.gemm_plan(op, m, n, k)
            what = f"special {fmt} {n}x{k} W*2^{wexp} X*2^{xexp} m={m} splits={pl.splits}"
            log(what)
            y = host(qpn.gemm(pw, dev(xs[:m])))
            y_ref = _oracle(fmt, w, xs[:m])
            scaled_parity(y, y_ref, -(wexp + xexp), what)
            # the zero row and the row whose block scales round to zero give exact zeros
            assert not y[:, 3].astype(np.float32).any() and not y[:, 7].astype(np.float32).any()


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_underflowing_outputs_match_bitwise(fmt):
    """Weights scaled by 2^-60: every output is below half the smallest FP16
    subnormal, so the GPU must return the oracle's FP16 rounding exactly:
    +0 or -0 with the sign of the FP64 sum (exact zeros as +0 or -0 too)."""
    qpn = need_gpu()
    n, k = 300, 2064
    w = special_weights(n, k, seed=3) * np.float32(2.0 ** -60)
    x8 = synth.activations(8, k, seed=3)
    pw = _pack(qpn, fmt, w)
    for m in (1, 4, 8):
        y = host(qpn.gemm(pw, dev(x8[:m])))
        y_ref = _oracle(fmt, w, x8[:m])
        r16 = oracle.round_f16(y_ref)
        assert not r16.astype(np.float32).any()
        nonzero = y_ref != 0
        # nonzero sums: the sign of the FP64 value decides the sign of zero
        assert np.array_equal(y.view(np.uint16)[nonzero], r16.view(np.uint16)[nonzero]), \
            f"{fmt} m={m}: signed-zero mismatch"
        assert not y.astype(np.float32).any()


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", SHAPES)
def test_extreme_activations_gemm(fmt, n, k):
    qpn = need_gpu()
    w = special_weights(n, k, seed=7 * n + k)
    x8 = edge_activations(8, k, seed=7 * n + k)
    pw = _pack(qpn, fmt, w)
    for m in range(1, 9):
        what = f"extreme activations {fmt} {n}x{k} m={m}"
        log(what)
        y = host(qpn.gemm(pw, dev(x8[:m])))
        scaled_parity(y, _oracle(fmt, w, x8[:m]), 0, what)


def test_subnormal_activations_alone():
    """Activations that are all FP16 subnormals: the sum is carried by
    operands the matrix unit must not flush to zero.  The weights are
    scaled by 2^8 so that the outputs stay FP16 normals."""
    qpn = need_gpu()
    n, k = 300, 2064
    w = special_weights(n, k, seed=9) * np.float32(2.0 ** 8)
    x8 = (synth.activations(8, k, seed=9).astype(np.float32) * np.float32(2.0 ** -16)).astype(np.float16)
    assert (np.abs(x8.astype(np.float32)) < 2.0 ** -14).mean() > 0.99
    for fmt in ("nvfp4", "fp8"):
        pw = _pack(qpn, fmt, w)
        for m in (1, 8):
            y = host(qpn.gemm(pw, dev(x8[:m])))
            # outputs are 2^-8 of the usual ones: compare at the usual scale
            scaled_parity(y, _oracle(fmt, w, x8[:m]), 8, f"subnormal activations {fmt} m={m}")


# (weight exponent, activation exponent, activations); the large activation
# columns leave no room to scale the outputs up
LM_CASES = [(0, 0, "normal"), (0, 0, "extreme"), (20, -12, "normal"), (-20, 8, "normal")]


@pytest.mark.parametrize("wexp,xexp,xkind", LM_CASES)
def test_special_weights_lmhead(wexp, xexp, xkind):
    """The lm_head on the special tensor: logits within the bar and the argmax
    the oracle's (gpu_util.check_argmax), plus extreme activations."""
    qpn = need_gpu()
    n, k = 4099, 1040
    w = special_weights(n, k, seed=17) * np.float32(2.0 ** wexp)
    pw = qpn.pack_nvfp4(dev(w))
    codes, scales, g = oracle.pack_nvfp4(w)
    x8 = synth.activations(8, k, seed=17) if xkind == "normal" else edge_activations(8, k, seed=17)
    x8 = (x8.astype(np.float32) * np.float32(2.0 ** xexp)).astype(np.float16)
    for m in (1, 3, 8):
        what = f"lmhead special W*2^{wexp} X*2^{xexp} {xkind} m={m}"
        log(what)
        lg, am = qpn.lmhead_nvfp4(pw, dev(x8[:m]))
        lg, am = host(lg), host(am)
        y_ref = oracle.gemm_nvfp4(codes, scales, g, x8[:m])
        scaled_parity(lg, y_ref, -(wexp + xexp), what)
        check_argmax(am, lg, y_ref, what)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_special_weights_prefill(fmt):
    """Prefill blocks (the 16-row skinny tile and the tiled MFMA kernel) on
    the special tensor with extreme activations and a scaled copy."""
    qpn = need_gpu()
    n, k = 300, 2064
    base = special_weights(n, k, seed=23)
    xe = edge_activations(48, k, seed=23)
    xn = synth.activations(48, k, seed=23, m_max=48)
    for wexp, xexp, x0 in ((0, 0, xe), (-20, 8, xn), (20, -12, xn)):
        w = base * np.float32(2.0 ** wexp)
        pw = _pack(qpn, fmt, w)
        xs = (x0.astype(np.float32) * np.float32(2.0 ** xexp)).astype(np.float16)
        for m in (9, 16, 40):
            what = f"prefill special {fmt} W*2^{wexp} X*2^{xexp} m={m}"
            log(what)
            y = host(qpn.prefill(pw, dev(xs[:m])))
            scaled_parity(y, _oracle(fmt, w, xs[:m]), -(wexp + xexp), what)
