"""NVFP4 lm_head with fused argmax against the oracle.

Logits: the GEMM parity bar.  Argmax: the oracle's lowest index of the
FP16-rounded FP64 logits, row by row (gpu_util.check_argmax).  A row may
differ only where a property of the arithmetic, not of the code, allows it:
the two candidates' FP64 logits lie within the FP32 accumulation error band
of each other or of an FP16 rounding boundary.  The count of such rows is
reported in the terminal summary; at the full 151936-row vocabulary with the
seed-0 inputs it must be zero (every row's top two FP16 logits are 23 or
more ulps apart there).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import check_argmax as _check_argmax
from gpu_util import dev, host, log, need_gpu, parity, plan_ids

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k", [(1000, 256), (4099, 1024), (160, 5120)])
def test_lmhead_small(n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n)
    x = synth.activations(8, k, seed=n)
    pw = qpn.pack_nvfp4(dev(w))
    codes, scales, g = oracle.pack_nvfp4(w)
    for m in (1, 3, 8):
        log(f"lmhead {n}x{k} m={m}")
        lg, am = qpn.lmhead_nvfp4(pw, dev(x[:m]))
        lg, am = host(lg), host(am)
        y_ref = oracle.gemm_nvfp4(codes, scales, g, x[:m])
        parity(lg, y_ref, f"lmhead {n}x{k} m={m}")
        _check_argmax(am, lg, y_ref, f"lmhead {n}x{k} m={m}")
        # the GEMM entry point returns the same logits
        assert np.array_equal(host(qpn.gemm(pw, dev(x[:m]))).view(np.uint16), lg.view(np.uint16))


def test_lmhead_duplicate_rows_tie_to_lowest_index():
    qpn = need_gpu()
    n, k = 777, 512
    w = synth.weights(n, k, seed=12)
    x = synth.activations(8, k, seed=12)
    codes, scales, g = oracle.pack_nvfp4(w)
    best = np.argmax(oracle.gemm_nvfp4(codes, scales, g, x), axis=1)
    # copy each row's winner to one earlier and one later position
    for mi, b in enumerate(best[:4]):
        lo, hi = int(b) // 2, min(n - 1, int(b) + 300 + mi)
        w[lo] = w[b]
        w[hi] = w[b]
    lg, am = qpn.lmhead_nvfp4(qpn.pack_nvfp4(dev(w)), dev(x))
    lg, am = host(lg), host(am)
    codes, scales, g = oracle.pack_nvfp4(w)
    y_ref = oracle.gemm_nvfp4(codes, scales, g, x)
    _check_argmax(am, lg, y_ref, "duplicates")
    for mi, b in enumerate(best[:4]):
        lo = int(b) // 2
        assert lg[mi, lo].view(np.uint16) == lg[mi, b].view(np.uint16)


def test_lmhead_one_hot_many_exact_ties():
    # Weights on a 0.01 grid in [-0.06, 0.06] with a +-0.06 element in every
    # 16-block: every block gets the same scale, so a column of What takes
    # only a handful of distinct values and its maximum repeats many times.
    qpn = need_gpu()
    n, k = 3000, 128
    rng = np.random.default_rng(21)
    w = (rng.integers(-6, 7, (n, k)) * 0.01).astype(np.float32)
    w[:, ::16] = np.float32(0.06)
    x = np.zeros((8, k), np.float16)
    for i in range(8):
        x[i, 9 * i + 3] = 1.0
    lg, am = qpn.lmhead_nvfp4(qpn.pack_nvfp4(dev(w)), dev(x))
    lg, am = host(lg), host(am)
    codes, scales, g = oracle.pack_nvfp4(w)
    y_ref = oracle.gemm_nvfp4(codes, scales, g, x)
    assert all((y_ref[i] == y_ref[i].max()).sum() > 10 for i in range(8))
    assert np.array_equal(am, oracle.argmax_f16(oracle.round_f16(y_ref)))
    assert np.array_equal(am, np.argmax(lg, axis=1))


def test_lmhead_zero_logit_rows():
    qpn = need_gpu()
    n, k = 64, 32
    w = -np.abs(synth.weights(n, k, seed=5))
    w[10, :] = 0.0          # logit exactly +0 (or -0 through the sign of the sum)
    w[40, :] = 0.0
    x = np.abs(synth.activations(2, k, seed=5)).astype(np.float16)
    lg, am = qpn.lmhead_nvfp4(qpn.pack_nvfp4(dev(w)), dev(x))
    assert list(host(am)) == [10, 10]


@pytest.mark.parametrize("m", [1, 8])
def test_lmhead_full_vocab(m):
    qpn = need_gpu()
    n, k = 151936, 5120
    log(f"lmhead full {n}x{k} m={m}: drawing weights")
    w = synth.weights(n, k, seed=0)
    x = synth.activations(8, k, seed=0)[:m]
    pw = qpn.pack_nvfp4(dev(w))
    lg, am = qpn.lmhead_nvfp4(pw, dev(x))
    lg, am = host(lg), host(am)
    del pw
    torch.cuda.empty_cache()
    log("lmhead full: oracle pack + FP64 GEMM")
    codes, scales, g = oracle.pack_nvfp4(w)
    del w
    y_ref = oracle.gemm_nvfp4(codes, scales, g, x)
    rows = np.random.default_rng(0).choice(n, 4096, replace=False)
    parity(lg[:, rows], y_ref[:, rows], f"lmhead full m={m} (sampled logits)")
    # seed 0: no row has a rounding boundary near its top candidates, so the
    # argmax must equal the oracle's on every row
    _check_argmax(am, lg, y_ref, f"lmhead full m={m}", max_ambiguous=0)


@pytest.mark.parametrize("plan", plan_ids())
def test_lmhead_every_plan(plan):
    qpn = need_gpu()
    n, k = 4099, 1040
    w = synth.weights(n, k, seed=plan)
    x = synth.activations(8, k, seed=plan)
    codes, scales, g = oracle.pack_nvfp4(w)
    pw = qpn.pack_nvfp4(dev(w))
    for m in (1, 2, 5, 8):
        log(f"lmhead plan {plan} {n}x{k} m={m}")
        lg, am = qpn.lmhead_nvfp4(pw, dev(x[:m]), plan=plan)
        lg, am = host(lg), host(am)
        y_ref = oracle.gemm_nvfp4(codes, scales, g, x[:m])
        parity(lg, y_ref, f"lmhead plan {plan} m={m}")
        _check_argmax(am, lg, y_ref, f"lmhead plan {plan} m={m}")


def test_lmhead_leaves_workspace_zeroed():
    """The argmax keys (and any split-K partials) are cleared after use, so one
    zero-filled workspace serves lm_head and GEMM calls of any shape."""
    qpn = need_gpu()
    n, k = 3000, 2048
    w = synth.weights(n, k, seed=5)
    x = synth.activations(8, k, seed=5)
    pw = qpn.pack_nvfp4(dev(w))
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    first = None
    for m in (8, 1, 8):
        lg, am = qpn.lmhead_nvfp4(pw, dev(x[:m]), workspace_=ws)
        assert not host(ws).any()
        y = host(qpn.gemm(pw, dev(x[:m]), ws=ws))
        assert not host(ws).any()
        assert np.array_equal(y.view(np.uint16), host(lg).view(np.uint16))
        if m == 8:
            if first is None:
                first = host(am)
            assert np.array_equal(host(am), first)


@pytest.mark.parametrize("n,k", [(4099, 1024), (151936, 5120)])
def test_lmhead_verify_every_accept_length(n, k):
    """Fused greedy verification: for each accepted length L of a k = m - 1
    draft round, (accepted, next token) equals the oracle's greedy_verify of
    the same argmax, with the logits and argmax as the plain lm_head's.  The
    m calls go back to back on one stream with a single synchronisation."""
    qpn = need_gpu()
    log(f"lmhead verify {n}x{k}: drawing weights")
    w = synth.weights(n, k, seed=n + 1)
    x = synth.activations(8, k, seed=n + 1)
    pw = qpn.pack_nvfp4(dev(w))
    for m in (1, 2, 8):
        lg0, am0 = qpn.lmhead_nvfp4(pw, dev(x[:m]))
        am0 = host(am0)
        drafts = []
        for L in range(m):
            d = am0[:m - 1].copy()
            if L < m - 1:
                d[L] = (d[L] + 1 + L) % n      # first mismatch at L
            drafts.append(d)
        log(f"lmhead verify {n}x{k} m={m}")
        outs = [qpn.lmhead_verify_nvfp4(pw, dev(x[:m]), dev(d)) for d in drafts]
        torch.cuda.synchronize()
        for L, (d, (lg, am, res)) in enumerate(zip(drafts, outs)):
            assert np.array_equal(host(lg).view(np.uint16), host(lg0).view(np.uint16))
            assert np.array_equal(host(am), am0)
            assert tuple(int(v) for v in host(res)) == oracle.greedy_verify(am0, d) == \
                (L, int(am0[L])), f"m={m} L={L}"
    # the argmax these verify rounds were decided on, against the oracle
    if n * k <= 4099 * 1024:
        codes, scales, g = oracle.pack_nvfp4(w)
        y_ref = oracle.gemm_nvfp4(codes, scales, g, x)
        lg, am, res = qpn.lmhead_verify_nvfp4(pw, dev(x), dev(np.zeros(7, np.int32)))
        parity(host(lg), y_ref, f"lmhead verify {n}x{k}")
        _check_argmax(host(am), host(lg), y_ref, f"lmhead verify {n}x{k}")
        assert tuple(int(v) for v in host(res)) == oracle.greedy_verify(host(am), np.zeros(7, np.int32))


def test_lmhead_verify_against_oracle_drafts():
    """Drafts built from the oracle's own argmax (so the expected acceptance
    is fixed by the oracle alone) on rows whose top two logits are far apart."""
    qpn = need_gpu()
    n, k = 2048, 256
    # one-hot rows: x row i selects weight row t_i, so logit t_i dominates
    targets = np.array([17, 900, 5, 2047, 1024, 33, 600, 1500])
    w = np.zeros((n, k), np.float32)
    w[:, :] = synth.weights(n, k, seed=3) * 0.01
    for i, t in enumerate(targets):
        w[t, i * 16:(i + 1) * 16] = 4.0
    x = np.zeros((8, k), np.float16)
    for i in range(8):
        x[i, i * 16:(i + 1) * 16] = 1.0
    codes, scales, g = oracle.pack_nvfp4(w)
    y_ref = oracle.gemm_nvfp4(codes, scales, g, x)
    am_ref = oracle.argmax_f16(oracle.round_f16(y_ref))
    assert np.array_equal(am_ref, targets)
    pw = qpn.pack_nvfp4(dev(w))
    for L in range(8):
        d = am_ref[:7].astype(np.int32).copy()
        if L < 7:
            d[L] = 0
        lg, am, res = qpn.lmhead_verify_nvfp4(pw, dev(x), dev(d))
        assert np.array_equal(host(am), am_ref)
        assert tuple(int(v) for v in host(res)) == oracle.greedy_verify(am_ref, d) == (L, int(am_ref[L]))
