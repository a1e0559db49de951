"""QPN GEMM (NVFP4 and FP8) through the C ABI against the FP64 oracle.

Small shapes that span several panels and k-steps plus a ragged tail are
compared element by element; the full-size decoder shapes run in the launch
configuration the benchmark times and are compared on sampled rows, which the
oracle packs itself (with the whole tensor's scale) and multiplies in FP64.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import dev, host, log, need_gpu, parity, plan_ids

pytestmark = pytest.mark.gpu

SMALL = [(1, 16), (16, 128), (37, 80), (100, 1040), (130, 4096), (300, 2064), (48, 9008)]


def _sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    rows |= {0, 1, 15, 16, n - 1, n - 2, n - 16, n // 2}
    return np.array(sorted(r for r in rows if 0 <= r < n), np.int64)


def _oracle_nvfp4_rows(w, rows, x):
    g, _ = oracle.nvfp4_tensor_scale(w)
    c, s = oracle.pack_nvfp4_rows(w[rows], g)
    return oracle.gemm_nvfp4(c, s, g, x)


def _oracle_fp8_rows(w, rows, x):
    c, rs = oracle.pack_fp8(w[rows])
    return oracle.gemm_fp8(c, rs, x)


@pytest.mark.parametrize("n,k", SMALL)
def test_nvfp4_small_all_m(n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n + 3 * k)
    x8 = synth.activations(8, k, seed=n + 3 * k)
    pw = qpn.pack_nvfp4(dev(w))
    codes, scales, g = oracle.pack_nvfp4(w)
    for m in range(1, 9):
        log(f"nvfp4 gemm {n}x{k} m={m}")
        y = host(qpn.gemm(pw, dev(x8[:m])))
        parity(y, oracle.gemm_nvfp4(codes, scales, g, x8[:m]), f"nvfp4 {n}x{k} m={m}")


@pytest.mark.parametrize("n,k", SMALL + [(24, 8), (19, 72)])
def test_fp8_small_all_m(n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n + 5 * k)
    x8 = synth.activations(8, k, seed=n + 5 * k)
    pw = qpn.pack_fp8(dev(w))
    codes, rs = oracle.pack_fp8(w)
    for m in range(1, 9):
        log(f"fp8 gemm {n}x{k} m={m}")
        y = host(qpn.gemm(pw, dev(x8[:m])))
        parity(y, oracle.gemm_fp8(codes, rs, x8[:m]), f"fp8 {n}x{k} m={m}")


def test_nvfp4_2048_square_m1_full():
    qpn = need_gpu()
    n = k = 2048
    w = synth.weights(n, k, seed=0)
    x = synth.activations(1, k, seed=0)
    log("nvfp4 2048x2048 m=1 full oracle")
    y = host(qpn.gemm(qpn.pack_nvfp4(dev(w)), dev(x)))
    codes, scales, g = oracle.pack_nvfp4(w)
    parity(y, oracle.gemm_nvfp4(codes, scales, g, x), "2048^2 m=1")


# decoder shapes, then the per-rank shards under 4-way tensor parallelism
# (gate/up N/4, down K/4, lm_head vocabulary N/4; QKV N/4, O K/4)
FULL_NV = [(17408, 5120, (1, 4, 8)), (5120, 17408, (1, 4, 8)), (34816, 5120, (8,)),
           (8704, 5120, (1, 8)), (5120, 4352, (1, 8)), (37984, 5120, (1, 8))]
FULL_F8 = [(6144, 5120, (1, 2, 4)), (5120, 5120, (1, 2, 4, 8)), (7168, 5120, (8,)),
           (1792, 5120, (1, 8)), (5120, 1280, (1, 8))]


@pytest.mark.parametrize("n,k,ms", FULL_NV)
def test_nvfp4_full_size_sampled(n, k, ms):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=0)
    x8 = synth.activations(8, k, seed=0)
    pw = qpn.pack_nvfp4(dev(w))
    rows = _sample_rows(n, 384, seed=n)
    for m in ms:
        log(f"nvfp4 full {n}x{k} m={m}")
        y = host(qpn.gemm(pw, dev(x8[:m])))
        parity(y[:, rows], _oracle_nvfp4_rows(w, rows, x8[:m]), f"nvfp4 {n}x{k} m={m}")
        assert np.isfinite(y).all()


@pytest.mark.parametrize("n,k,ms", FULL_F8)
def test_fp8_full_size_sampled(n, k, ms):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=0)
    x8 = synth.activations(8, k, seed=0)
    pw = qpn.pack_fp8(dev(w))
    rows = _sample_rows(n, 384, seed=n)
    for m in ms:
        log(f"fp8 full {n}x{k} m={m}")
        y = host(qpn.gemm(pw, dev(x8[:m])))
        parity(y[:, rows], _oracle_fp8_rows(w, rows, x8[:m]), f"fp8 {n}x{k} m={m}")
        assert np.isfinite(y).all()


MAX_SIZES = [("nvfp4", 48, 1 << 20), ("fp8", 40, 1 << 20), ("nvfp4", 1 << 24, 16), ("fp8", 1 << 24, 8)]


@pytest.mark.parametrize("fmt,n,k", MAX_SIZES)
def test_documented_maximum_sizes(fmt, n, k):
    """k = 2^20 (the K limit; at M = 8 the activation slice is split over
    hundreds of K ranges) and n = 2^24 (the N limit: 2^20 panels), sampled
    rows against the oracle."""
    qpn = need_gpu()
    w = synth.weights(n, k, seed=5)
    x8 = synth.activations(8, k, seed=5)
    pw = qpn.pack_nvfp4(dev(w)) if fmt == "nvfp4" else qpn.pack_fp8(dev(w))
    rows = _sample_rows(n, 64, seed=1)
    ref8 = (_oracle_nvfp4_rows if fmt == "nvfp4" else _oracle_fp8_rows)(w, rows, x8)
    op = qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8
    del w
    for m in (1, 3, 8):
        pl = qpn.gemm_plan(op, m, n, k)
        log(f"max size {fmt} {n}x{k} m={m} workgroups={pl.workgroups} splits={pl.splits}")
        y = qpn.gemm(pw, dev(x8[:m]))
        yr = host(y[:, torch.from_numpy(rows).cuda()])
        del y
        parity(yr, ref8[:m], f"max size {fmt} {n}x{k} m={m}")


def test_one_hot_activation_pins_layout():
    qpn = need_gpu()
    n, k = 40, 384
    w = synth.weights(n, k, seed=2)
    codes, scales, g = oracle.pack_nvfp4(w)
    wh = oracle.dequant_nvfp4(codes, scales, g)
    c8, rs = oracle.pack_fp8(w)
    wh8 = oracle.dequant_fp8(c8, rs)
    pw, pw8 = qpn.pack_nvfp4(dev(w)), qpn.pack_fp8(dev(w))
    cols = [0, 1, 7, 8, 31, 32, 100, 127, 128, 255, 383]
    x = np.zeros((len(cols[:8]), k), np.float16)
    for i, c in enumerate(cols[:8]):
        x[i, c] = 1.0
    x2 = np.zeros((len(cols[8:]), k), np.float16)
    for i, c in enumerate(cols[8:]):
        x2[i, c] = 1.0
    for xx, cc in ((x, cols[:8]), (x2, cols[8:])):
        y = host(qpn.gemm(pw, dev(xx)))
        y8 = host(qpn.gemm(pw8, dev(xx)))
        for i, c in enumerate(cc):
            # one product per output: only the final FP32 scale and FP16
            # rounding apply (half an ulp, absolute 2^-25 below 2^-14)
            assert np.allclose(y[i].astype(np.float64), wh[:, c], rtol=2 ** -10, atol=2 ** -24), c
            assert np.allclose(y8[i].astype(np.float64), wh8[:, c], rtol=2 ** -10, atol=2 ** -24), c


def test_deterministic_and_row_position_independent():
    qpn = need_gpu()
    n, k = 96, 2048
    w = synth.weights(n, k, seed=4)
    w[70] = w[3]          # duplicate rows in different panels and positions
    w[21] = w[3]
    x = synth.activations(8, k, seed=4)
    for pack in (qpn.pack_nvfp4, qpn.pack_fp8):
        pw = pack(dev(w))
        y1 = host(qpn.gemm(pw, dev(x)))
        y2 = host(qpn.gemm(pw, dev(x)))
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
        assert np.array_equal(y1[:, 70].view(np.uint16), y1[:, 3].view(np.uint16))
        assert np.array_equal(y1[:, 21].view(np.uint16), y1[:, 3].view(np.uint16))


def test_k_zero_and_empty_calls():
    qpn = need_gpu()
    w = np.zeros((20, 0), np.float32)
    for pack in (qpn.pack_nvfp4, qpn.pack_fp8):
        pw = pack(torch.zeros((20, 0), dtype=torch.float32, device="cuda"))
        x = torch.zeros((3, 0), dtype=torch.float16, device="cuda")
        y = torch.full((3, 20), 7.0, dtype=torch.float16, device="cuda")
        qpn.gemm(pw, x, out=y)
        assert not host(y).any()
    pw = qpn.pack_nvfp4(dev(synth.weights(20, 32, seed=1)))
    y = torch.full((0, 20), 7.0, dtype=torch.float16, device="cuda")
    qpn.gemm(pw, torch.zeros((0, 32), dtype=torch.float16, device="cuda"), out=y)


def test_header_mismatch_yields_nan():
    qpn = need_gpu()
    w = synth.weights(32, 64, seed=9)
    x = dev(synth.activations(2, 64, seed=9))
    pw8 = qpn.pack_fp8(dev(w))
    pw4 = qpn.pack_nvfp4(dev(w))
    wrong = qpn.PackedWeight(pw8.blob, 32, 64, qpn.FMT_NVFP4)   # FP8 blob to the NVFP4 GEMM
    assert np.isnan(host(qpn.gemm(wrong, x)).astype(np.float32)).all()
    wrong = qpn.PackedWeight(pw4.blob, 32, 64, qpn.FMT_FP8)     # NVFP4 blob to the FP8 GEMM
    assert np.isnan(host(qpn.gemm(wrong, x)).astype(np.float32)).all()
    wrong = qpn.PackedWeight(pw4.blob, 16, 64, qpn.FMT_NVFP4)   # wrong n
    assert np.isnan(host(qpn.gemm(wrong, x)).astype(np.float32)).all()


# Every compiled launch plan (wavefronts per panel, panels per workgroup,
# prefetch depth) on shapes with a partial last workgroup, a ragged K tail and
# k-step counts that no plan's wavefront count divides.
PLAN_SHAPES = [(37, 80), (300, 2064), (48, 9008), (16, 128)]
PLAN_IDS = plan_ids()


@pytest.mark.parametrize("plan", PLAN_IDS)
def test_every_plan_against_oracle(plan):
    qpn = need_gpu()
    for n, k in PLAN_SHAPES:
        w = synth.weights(n, k, seed=7 * n + k)
        x8 = synth.activations(8, k, seed=7 * n + k)
        pw4, pw8 = qpn.pack_nvfp4(dev(w)), qpn.pack_fp8(dev(w))
        codes, scales, g = oracle.pack_nvfp4(w)
        c8, rs = oracle.pack_fp8(w)
        for m in (1, 2, 3, 4, 5, 8):
            log(f"plan {plan}: {n}x{k} m={m}")
            parity(host(qpn.gemm(pw4, dev(x8[:m]), plan=plan)),
                   oracle.gemm_nvfp4(codes, scales, g, x8[:m]), f"plan {plan} nvfp4 {n}x{k} m={m}")
            parity(host(qpn.gemm(pw8, dev(x8[:m]), plan=plan)), oracle.gemm_fp8(c8, rs, x8[:m]),
                   f"plan {plan} fp8 {n}x{k} m={m}")


@pytest.mark.parametrize("plan", PLAN_IDS)
def test_every_plan_full_size_rows(plan):
    """Full gate/up and down shapes at M=1 and 8 under each plan, sampled rows."""
    qpn = need_gpu()
    for n, k in ((17408, 5120), (5120, 17408)):
        w = synth.weights(n, k, seed=0)
        x8 = synth.activations(8, k, seed=0)
        pw = qpn.pack_nvfp4(dev(w))
        rows = _sample_rows(n, 96, seed=n + plan)
        ref = _oracle_nvfp4_rows(w, rows, x8)
        for m in (1, 8):
            log(f"plan {plan}: full {n}x{k} m={m}")
            y = host(qpn.gemm(pw, dev(x8[:m]), plan=plan))
            parity(y[:, rows], ref[:m], f"plan {plan} nvfp4 {n}x{k} m={m}")


HYBRID = [("nvfp4", 5120, 17408, (1, 2)), ("nvfp4", 4805, 16000, (1, 2)),
          ("fp8", 6144, 5120, (1, 2)), ("fp8", 4600, 9000, (1, 2))]


@pytest.mark.parametrize("fmt,n,k,ms", HYBRID)
def test_balanced_hybrid_launch(fmt, n, k, ms):
    """Shapes with 1-3 panels per CU and a remainder: the launch takes whole
    panels for every CU and splits only the remaining panels in K.  Every row
    of the split panels and sampled whole-panel rows match the oracle."""
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n ^ k)
    x8 = synth.activations(8, k, seed=n ^ k)
    pw = qpn.pack_nvfp4(dev(w)) if fmt == "nvfp4" else qpn.pack_fp8(dev(w))
    op = qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8
    for m in ms:
        pl = qpn.gemm_plan(op, m, n, k)
        whole = pl.workgroups - pl.split_workgroups
        assert whole > 0 and pl.splits > 1, pl
        first_split_row = whole * pl.panels_per_workgroup * 16
        rows = np.union1d(np.arange(first_split_row, n), _sample_rows(first_split_row, 96, seed=m))
        ref = (_oracle_nvfp4_rows if fmt == "nvfp4" else _oracle_fp8_rows)(w, rows, x8[:m])
        log(f"hybrid {fmt} {n}x{k} m={m} workgroups={pl.workgroups} split={pl.split_workgroups}x{pl.splits}")
        ws = torch.zeros(max(qpn.workspace_bytes(op, m, n, k), 256), dtype=torch.uint8, device="cuda")
        y = host(qpn.gemm(pw, dev(x8[:m]), ws=ws))
        parity(y[:, rows], ref, f"hybrid {fmt} {n}x{k} m={m}")
        assert not host(ws).any(), "workspace not left zero-filled"


def test_split_k_workspace_reuse_and_determinism():
    """Split-K plans: the same call repeated on one workspace gives identical
    bits (the arrival counters re-arm themselves), matches the oracle, and a
    call given no workspace (no split) agrees within the parity bar."""
    qpn = need_gpu()
    for fmt, (n, k) in (("nvfp4", (300, 4096)), ("fp8", (200, 8192)), ("nvfp4", (5120, 17408))):
        w = synth.weights(n, k, seed=11)
        x8 = synth.activations(8, k, seed=11)
        pw = qpn.pack_nvfp4(dev(w)) if fmt == "nvfp4" else qpn.pack_fp8(dev(w))
        op = qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8
        for m in (1, 4, 8):
            pl = qpn.gemm_plan(op, m, n, k)
            need = qpn.workspace_bytes(op, m, n, k)
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
            log(f"split-K {fmt} {n}x{k} m={m} splits={pl.splits}")
            ys = [host(qpn.gemm(pw, dev(x8[:m]), ws=ws)) for _ in range(3)]
            for yy in ys[1:]:
                assert np.array_equal(yy.view(np.uint16), ys[0].view(np.uint16))
            assert not host(ws).any(), "workspace not left zero-filled"
            try:
                y0 = host(qpn.gemm(pw, dev(x8[:m]), ws=torch.zeros(0, dtype=torch.uint8, device="cuda")))
            except qpn.QpnError as e:
                # only where one activation slice of the whole K cannot fit in LDS
                assert e.status == 4 and pl.activation_rows * k * 2 > 80 * 1024, e
                y0 = None
            if fmt == "nvfp4":
                rows = np.arange(n) if n <= 300 else _sample_rows(n, 128, seed=3)
                ref = _oracle_nvfp4_rows(w, rows, x8[:m])
            else:
                rows = np.arange(n)
                ref = _oracle_fp8_rows(w, rows, x8[:m])
            parity(ys[0][:, rows], ref, f"split {fmt} {n}x{k} m={m}")
            if y0 is not None:
                parity(y0[:, rows], ref, f"unsplit {fmt} {n}x{k} m={m}")
