"""Helpers for the GPU parity tests: device transfers, the oracle comparison
and the tolerance the tests hold the HIP path to."""
import sys

import numpy as np
import pytest
import torch

# Floating-point parity bar for GEMM outputs against the unrounded FP64
# oracle: per element |err| <= 1e-2 * rms(ref) + 1e-3, and relative Frobenius
# error <= 2e-3.  Headroom: FP16 output rounding contributes at most 2^-11
# relative per element (~2.8e-4 rms relative); FP32 accumulation over K <= 2^15
# adds ~1e-5 relative; so a failure means a layout, decode or scale error.
ELEM_RTOL_OF_RMS = 1e-2
ELEM_ATOL = 1e-3
FROB_RTOL = 2e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_quantized_skinny_qpn_amd import qpn  # raises if libqpn.so is not built
    return qpn


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def parity(y_gpu_f16, y_ref, what=""):
    """Assert the element and Frobenius bounds; return (max_err/bound, frob)."""
    y = np.asarray(y_gpu_f16).astype(np.float64)
    ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = ELEM_RTOL_OF_RMS * rms + ELEM_ATOL
    worst = float(err.max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(y - ref)) / nref if nref > 0 else float(np.linalg.norm(y - ref))
    assert worst <= bound, f"{what}: max |err| {worst:.3e} > {bound:.3e}"
    assert frob <= FROB_RTOL, f"{what}: relative Frobenius {frob:.3e} > {FROB_RTOL}"
    return worst / bound, frob


def plan_ids():
    """Every launch plan id the library accepts (probed through the C ABI)."""
    from fp8_quantized_skinny_qpn_amd import qpn
    ids = []
    for i in range(1, 65):
        try:
            qpn.debug_set_plan(i)
        except qpn.QpnError:
            continue
        ids.append(i)
    qpn.debug_set_plan(0)
    return ids
