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
    return qpn.plan_ids()


# Argmax parity (lm_head).  The oracle's argmax is the lowest index of the
# row maximum of the FP16-rounded FP64 logits.  The GPU accumulates in FP32,
# so its FP16 logit of a candidate can differ from the oracle's only when the
# candidate's FP64 logit lies within the FP32 accumulation error of an FP16
# rounding boundary (the midpoint between two adjacent FP16 values); the
# error is ~1e-5 at K = 5120, and AMBIGUITY_BAND is ten times that.  A row
# may therefore differ from the oracle only when the two candidates' FP64
# logits lie within AMBIGUITY_BAND of each other or of such a midpoint; the
# GPU's pick must then still be within 2 FP16 ulps of the maximum.  Every
# other row must match exactly.  The GPU's argmax must always equal the
# lowest-index argmax of the logits it returned.
AMBIGUITY_BAND = 1e-4

# (test, ambiguous rows, rows) of every argmax check in this session, shown
# in the terminal summary (tests/conftest.py)
ARGMAX_RECORDS = []


def ulp16(v):
    v = abs(float(v))
    if v < 2.0 ** -14:
        return 2.0 ** -24
    return 2.0 ** (np.floor(np.log2(v)) - 10)


def f16_midpoint_distance(v):
    """Distance from FP64 value v to the nearest FP16 rounding boundary."""
    import oracle
    h = oracle.round_f16(np.array([v], np.float64))[0]
    lo = np.nextafter(h, np.float16(-np.inf))
    hi = np.nextafter(h, np.float16(np.inf))
    hv = float(h)
    mids = [(hv + float(lo)) / 2 if np.isfinite(lo) else np.inf,
            (hv + float(hi)) / 2 if np.isfinite(hi) else np.inf]
    return min(abs(v - mid) for mid in mids)


def check_argmax(am_gpu, logits_gpu, y_ref, what, max_ambiguous=None):
    """Strict argmax parity; returns the number of ambiguous rows (which must
    not exceed max_ambiguous when given)."""
    import oracle
    lg = np.asarray(logits_gpu)
    am_gpu = np.asarray(am_gpu)
    assert np.array_equal(am_gpu, np.argmax(lg, axis=1).astype(np.int32)), f"{what}: self"
    r16 = oracle.round_f16(y_ref)
    am_ref = oracle.argmax_f16(r16)
    ambiguous, gaps = [], []
    for mi in range(y_ref.shape[0]):
        srt = np.sort(r16[mi].astype(np.float64))
        top16 = srt[-1]
        gaps.append((srt[-1] - srt[-2]) / ulp16(top16) if srt.size > 1 else np.inf)
        a, b = int(am_gpu[mi]), int(am_ref[mi])
        if a == b:
            continue
        ya, yb = float(y_ref[mi, a]), float(y_ref[mi, b])
        near = (abs(ya - yb) <= AMBIGUITY_BAND or f16_midpoint_distance(ya) <= AMBIGUITY_BAND
                or f16_midpoint_distance(yb) <= AMBIGUITY_BAND)
        assert near, (f"{what}: row {mi} GPU {a} (y_ref {ya!r}) vs oracle {b} (y_ref {yb!r}); "
                      f"no FP16 rounding boundary within {AMBIGUITY_BAND}")
        assert float(top16) - float(r16[mi, a]) <= 2 * ulp16(top16), \
            f"{what}: row {mi} GPU pick {a} is more than 2 ulps below the maximum"
        ambiguous.append((mi, a, b, ya, yb))
    log(f"{what}: top-2 gap in FP16 ulps per row {['%.1f' % g for g in gaps]}; "
        f"ambiguous rows {ambiguous}")
    ARGMAX_RECORDS.append((what, len(ambiguous), y_ref.shape[0]))
    if max_ambiguous is not None:
        assert len(ambiguous) <= max_ambiguous, f"{what}: ambiguous rows {ambiguous}"
    return len(ambiguous)
