"""GPU pack kernels against the oracle pack: bit-exact codes, scales and
tensor scale, read back through the blob's canonical export."""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from golden_io import worked_example
from gpu_util import dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu


def _gpu_pack_nvfp4(qpn, w):
    pw = qpn.pack_nvfp4(dev(w))
    codes, scales, g = qpn.debug_unpack_nvfp4(pw)
    return pw, host(codes), host(scales), np.float32(host(g)[0])


def _gpu_pack_fp8(qpn, w):
    pw = qpn.pack_fp8(dev(w))
    codes, rs = qpn.debug_unpack_fp8(pw)
    return pw, host(codes), host(rs)


def _check_nvfp4(qpn, w, what):
    log(f"pack nvfp4 {what} {w.shape}")
    _, c, s, g = _gpu_pack_nvfp4(qpn, w)
    oc, os_, og = oracle.pack_nvfp4(w)
    assert g.view(np.uint32) == np.float32(og).view(np.uint32), (what, g, og)
    assert np.array_equal(s, os_), f"{what}: {np.count_nonzero(s != os_)} scale mismatches"
    assert np.array_equal(c, oc), f"{what}: {np.count_nonzero(c != oc)} code-byte mismatches"


def _check_fp8(qpn, w, what):
    log(f"pack fp8 {what} {w.shape}")
    _, c, rs = _gpu_pack_fp8(qpn, w)
    oc, ors = oracle.pack_fp8(w)
    assert np.array_equal(rs.view(np.uint32), ors.view(np.uint32)), what
    assert np.array_equal(c, oc), f"{what}: {np.count_nonzero(c != oc)} code mismatches"


def test_worked_examples():
    qpn = need_gpu()
    ex = worked_example("nvfp4_worked_example.txt")
    _check_nvfp4(qpn, np.array([ex["w"][r] for r in range(3)], np.float32), "worked")
    ex8 = worked_example("fp8_worked_example.txt")
    _check_fp8(qpn, np.array([ex8["w"][r] for r in range(2)], np.float32), "worked")


@pytest.mark.parametrize("n,k", [(1, 16), (16, 128), (17, 144), (37, 80), (100, 1040), (130, 4096)])
def test_random_shapes_with_ragged_tails(n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n * 7 + k)
    _check_nvfp4(qpn, w, f"random {n}x{k}")
    _check_fp8(qpn, w, f"random {n}x{k}")


@pytest.mark.parametrize("n,k", [(24, 8), (5, 72), (33, 200)])
def test_fp8_k_multiple_of_8(n, k):
    qpn = need_gpu()
    _check_fp8(qpn, synth.weights(n, k, seed=3), f"fp8 k%16!=0 {n}x{k}")


def test_special_values():
    qpn = need_gpu()
    rng = np.random.default_rng(5)
    w = synth.weights(48, 256, seed=11)
    w[3, :] = 0.0                                    # zero row
    w[5, 32:48] = 0.0                                # zero block
    w[6, 0:16] = -0.0                                # negative-zero block
    w[7] *= np.float32(1e-30)                        # tiny row (fp32 subnormal block scales)
    w[8, 16:32] = np.float32(2.0 ** -140)            # subnormal weights
    w[9] = np.where(rng.random(256) < 0.5, -1, 1).astype(np.float32) * 0.07  # constant magnitude
    w[10, :] = np.float32(3.0e-2) * (np.arange(256) % 7 - 3).astype(np.float32)  # many ties
    _check_nvfp4(qpn, w, "special")
    _check_fp8(qpn, w, "special")
    # power-of-two scaled tensor: huge and tiny
    _check_nvfp4(qpn, w * np.float32(2.0 ** 60), "x2^60")
    _check_nvfp4(qpn, w * np.float32(2.0 ** -60), "x2^-60")
    _check_fp8(qpn, w * np.float32(2.0 ** -60), "x2^-60")


def test_degenerate_tensors():
    qpn = need_gpu()
    _check_nvfp4(qpn, np.zeros((20, 32), np.float32), "all-zero")
    _check_fp8(qpn, np.zeros((20, 32), np.float32), "all-zero")
    w = np.zeros((4, 48), np.float32)
    w[1, 7] = np.float32(2.0 ** -149)                 # g underflows to 0
    _check_nvfp4(qpn, w, "g-underflow")
    _check_fp8(qpn, w, "smallest-subnormal")


@pytest.mark.parametrize("n,k", [(2048, 2048), (5120, 17408), (17408, 5120)])
def test_full_size_nvfp4(n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=0)
    _check_nvfp4(qpn, w, f"full {n}x{k}")


@pytest.mark.parametrize("n,k", [(6144, 5120), (7168, 5120)])
def test_full_size_fp8(n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=0)
    _check_fp8(qpn, w, f"full {n}x{k}")


# ---- FP8 -> NVFP4 conversion of a packed weight ------------------------------

def _check_requant(qpn, w, what):
    """GPU FP8 pack then GPU conversion, against the oracle's FP8 pack then the
    oracle's conversion: bit-exact codes, scales and tensor scale."""
    log(f"requant {what} {w.shape}")
    pw8 = qpn.pack_fp8(dev(w))
    pw4 = qpn.requant_fp8_to_nvfp4(pw8)
    c, s, g = qpn.debug_unpack_nvfp4(pw4)
    c, s, g = host(c), host(s), np.float32(host(g)[0])
    oc8, ors = oracle.pack_fp8(w)
    oc, os_, og = oracle.requant_fp8_to_nvfp4(oc8, ors)
    assert g.view(np.uint32) == np.float32(og).view(np.uint32), (what, g, og)
    assert np.array_equal(s, os_), f"{what}: {np.count_nonzero(s != os_)} scale mismatches"
    assert np.array_equal(c, oc), f"{what}: {np.count_nonzero(c != oc)} code-byte mismatches"
    return pw4, (oc, os_, og)


def _row_spread(w):
    # rows with magnitudes over 2^-12 .. 2^12, so the FP8 row scales differ
    e = (np.arange(w.shape[0]) % 25 - 12).astype(np.float32)
    return (w * (2.0 ** e)[:, None]).astype(np.float32)


@pytest.mark.parametrize("n,k", [(1, 16), (16, 128), (17, 144), (37, 80), (100, 1040), (130, 4096)])
def test_requant_random_shapes_with_ragged_tails(n, k):
    qpn = need_gpu()
    _check_requant(qpn, _row_spread(synth.weights(n, k, seed=n * 5 + k)), f"random {n}x{k}")


def test_requant_special_values():
    qpn = need_gpu()
    w = synth.weights(48, 256, seed=23)
    w[3, :] = 0.0                                    # zero row (row scale 0)
    w[5, 32:48] = 0.0                                # zero block
    w[6, 0:16] = -0.0                                # -0 codes stay -0
    w[7] *= np.float32(1e-36)                        # subnormal FP32 row scale and products
    w[9] = np.where(np.arange(256) % 3 == 0, -1, 1).astype(np.float32) * 0.07
    _check_requant(qpn, w, "special")
    _check_requant(qpn, w * np.float32(2.0 ** 40), "x2^40")
    _check_requant(qpn, np.zeros((20, 32), np.float32), "all-zero")


@pytest.mark.parametrize("n,k", [(7168, 5120), (5120, 5120)])
def test_requant_full_size(n, k):
    """The layer's FP8 projections (QKV, O) converted to NVFP4, then the GEMM
    on the converted blob at M = 8 on sampled rows."""
    qpn = need_gpu()
    w = synth.weights(n, k, seed=41)
    pw4, (oc, os_, og) = _check_requant(qpn, w, f"full {n}x{k}")
    x = synth.activations(8, k, seed=41)
    y = host(qpn.gemm(pw4, dev(x)))
    rows = np.random.default_rng(n).choice(n, 256, replace=False)
    y_ref = oracle.gemm_nvfp4(oc[rows], os_[rows], og, x)
    parity(y[:, rows], y_ref, f"gemm on converted {n}x{k}")


def test_requant_invalid_source_gives_nan_outputs():
    """A source whose header is not an FP8 [n, k] blob: the converted blob is
    marked invalid and a GEMM on it writes NaN (all reads stay in bounds)."""
    qpn = need_gpu()
    n, k = 48, 256
    for bad in ("zeros", "nvfp4"):
        if bad == "zeros":
            src = torch.zeros(qpn.fp8_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
        else:  # an NVFP4 blob of the same shape, padded to the FP8 size
            pw = qpn.pack_nvfp4(dev(synth.weights(n, k, seed=1)))
            src = torch.zeros(qpn.fp8_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
            src[:pw.nbytes] = pw.blob
        out = qpn.requant_fp8_to_nvfp4(qpn.PackedWeight(src, n, k, qpn.FMT_FP8))
        y = host(qpn.gemm(out, dev(synth.activations(2, k, seed=1))))
        assert np.all(np.isnan(y.astype(np.float32))), bad
