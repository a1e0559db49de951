"""Prefill-sized activation blocks (9 <= m <= 256) against the oracle.

Up to 16 rows the call runs the skinny kernel with a 16-row activation tile
(the tiled kernel for large calls at 9-16 rows, and when no workspace is
given and K needs splitting); from 17 rows the tiled MFMA kernel.  Both
paths are covered below.

The same parity bar as the skinny GEMM: per element |err| <= 1e-2 rms(ref)
+ 1e-3 and relative Frobenius error <= 2e-3 against the FP64 oracle product
of the canonical codes.  Shapes span several 128- and 256-channel blocks,
ragged N and M tails, K splits, every activation-tile count (32, 64, 128
rows), the wide tile at 17 to 64 rows and its two 128-row blocks (129 to 256
rows), and the full decoder shapes (sampled output channels).
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu

MS = (9, 12, 16, 17, 31, 33, 64, 100, 128, 129, 200, 256)


def _prefill_one_range(qpn, pw, xd):
    """The call without a workspace: one K range, so every workgroup runs
    all k-steps through many cycles of its prefetch ring."""
    out = torch.empty((xd.shape[0], pw.n), dtype=torch.float16, device="cuda")
    fn = qpn.lib.qpn_gemm_prefill_nvfp4 if pw.fmt == qpn.FMT_NVFP4 else qpn.lib.qpn_gemm_prefill_fp8
    assert fn(pw.blob.data_ptr(), xd.data_ptr(), out.data_ptr(), xd.shape[0], pw.n, pw.k, None, 0, None) == 0
    return out


def _pack(qpn, fmt, w):
    if fmt == "nvfp4":
        codes, scales, g = oracle.pack_nvfp4(w)
        return qpn.pack_nvfp4(dev(w)), lambda x, rows=slice(None): oracle.gemm_nvfp4(codes[rows], scales[rows], g, x)
    codes, rs = oracle.pack_fp8(w)
    return qpn.pack_fp8(dev(w)), lambda x, rows=slice(None): oracle.gemm_fp8(codes[rows], rs[rows], x)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
@pytest.mark.parametrize("n,k", [(200, 1024), (1000, 256), (130, 4096), (16, 64)])
def test_prefill_small(fmt, n, k):
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n + k)
    x = synth.activations(256, k, seed=n + k, m_max=256)
    pw, ref = _pack(qpn, fmt, w)
    op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    for m in MS:
        pl = qpn.gemm_plan(op, m, n, k)
        log(f"prefill {fmt} {n}x{k} m={m}: {pl.activation_rows} rows, {pl.splits} splits")
        xd = dev(x[:m])
        y_ref = ref(x[:m])
        parity(host(qpn.prefill(pw, xd)), y_ref, f"prefill {fmt} {n}x{k} m={m}")
        parity(host(_prefill_one_range(qpn, pw, xd)), y_ref, f"prefill {fmt} {n}x{k} m={m} one K range")


@pytest.mark.parametrize("fmt,n,k,ppw,splits", [("nvfp4", 4100, 1280, 5, 1), ("nvfp4", 4100, 3328, 5, 4),
                                               ("fp8", 4100, 3328, 2, 2), ("fp8", 8704, 1024, 5, 1),
                                               ("fp8", 8200, 3328, 5, 2), ("fp8", 48000, 256, 16, 1)])
def test_prefill_16_rows_multi_panel(fmt, n, k, ppw, splits):
    """9-16 rows through the skinny kernel's shared-slice plans (five NVFP4
    panels; two, five or sixteen FP8 panels per workgroup; the 16-row staging
    order, with and without K splits), ragged N, every output checked."""
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n + 3 * k)
    x = synth.activations(16, k, seed=n + 3 * k, m_max=16)
    pw, ref = _pack(qpn, fmt, w)
    op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    for m in (9, 16):
        pl = qpn.gemm_plan(op, m, n, k)
        assert (pl.activation_rows, pl.panels_per_workgroup, pl.splits) == (16, ppw, splits)
        log(f"prefill 16-row tile {fmt} {n}x{k} m={m}: {pl.workgroups} workgroups")
        parity(host(qpn.prefill(pw, dev(x[:m]))), ref(x[:m]), f"prefill {fmt} {n}x{k} m={m} (16-row tile)")


@pytest.mark.parametrize("fmt,n,k", [("nvfp4", 17408, 5120), ("nvfp4", 5120, 17408),
                                     ("fp8", 6144, 5120), ("fp8", 7168, 5120)])
def test_prefill_full_size_sampled(fmt, n, k):
    """Decoder shapes at the launch configuration the benchmark times; the
    oracle computes 192 sampled output channels (including the last)."""
    qpn = need_gpu()
    log(f"prefill full {fmt} {n}x{k}: drawing weights")
    w = synth.weights(n, k, seed=7)
    x = synth.activations(256, k, seed=7, m_max=256)
    pw, ref = _pack(qpn, fmt, w)
    rows = np.sort(np.concatenate([np.random.default_rng(n).choice(n - 1, 191, replace=False), [n - 1]]))
    for m in (16, 32, 64, 128, 256):
        log(f"prefill full {fmt} {n}x{k} m={m}")
        y = host(qpn.prefill(pw, dev(x[:m])))
        parity(y[:, rows], ref(x[:m], rows), f"prefill full {fmt} {n}x{k} m={m}")
    y = host(_prefill_one_range(qpn, pw, dev(x[:128])))
    parity(y[:, rows], ref(x[:128], rows), f"prefill full {fmt} {n}x{k} m=128 one K range")


@pytest.mark.parametrize("fmt,n,k,ppw", [("nvfp4", 24576, 1024, 16), ("fp8", 1000, 8192, 8)])
def test_prefill_9_16_rows_tiled(fmt, n, k, ppw):
    """9-16 rows of a large call (NVFP4 with 1536 or more panels, FP8 with
    128 or more k-steps of 64) on the tiled kernel, a 32-row tile half of which
    reads zero rows: the 256-channel tile for NVFP4, the 128-channel tile
    for FP8 (ragged N), every output checked."""
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n + 5 * k)
    x = synth.activations(16, k, seed=n + 5 * k, m_max=16)
    pw, ref = _pack(qpn, fmt, w)
    op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    for m in (9, 12, 16):
        pl = qpn.gemm_plan(op, m, n, k)
        assert (pl.activation_rows, pl.panels_per_workgroup) == (32, ppw), (m, pl)
        log(f"prefill tiled {fmt} {n}x{k} m={m}: {pl.workgroups} workgroups, {pl.splits} per tile")
        parity(host(qpn.prefill(pw, dev(x[:m]))), ref(x[:m]), f"prefill tiled {fmt} {n}x{k} m={m}")


@pytest.mark.parametrize("fmt,n,k,m", [("fp8", 33000, 1024, 32), ("nvfp4", 33000, 512, 100)])
def test_prefill_many_tiles_one_round(fmt, n, k, m):
    """More output tiles than CUs (258) whose whole-tile rounds would be half
    empty: one round of 256 equal ranges, every tile but a few cut between
    two workgroups and summed up the pairwise tree; 1024 sampled output
    channels (the last included) against the oracle, and the call without a
    workspace (whole tiles) as well."""
    qpn = need_gpu()
    w = synth.weights(n, k, seed=n + 7 * k)
    x = synth.activations(m, k, seed=n + 7 * k, m_max=m)
    pw, ref = _pack(qpn, fmt, w)
    op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    pl = qpn.gemm_plan(op, m, n, k)
    assert (pl.workgroups, pl.splits, pl.panels_per_workgroup) == (256, 2, 8), pl
    rows = np.sort(np.concatenate([np.random.default_rng(n).choice(n - 1, 1023, replace=False), [n - 1]]))
    y_ref = ref(x, rows)
    log(f"prefill many tiles {fmt} {n}x{k} m={m}")
    parity(host(qpn.prefill(pw, dev(x)))[:, rows], y_ref, f"prefill many tiles {fmt} {n}x{k} m={m}")
    parity(host(_prefill_one_range(qpn, pw, dev(x)))[:, rows], y_ref,
           f"prefill many tiles {fmt} {n}x{k} m={m} whole tiles")


@pytest.mark.parametrize("fmt,m", [("nvfp4", 100), ("fp8", 80)])
def test_prefill_wide_tile_65_128_rows(fmt, m):
    """65-128 rows of a call with more than 128 tiles of 128 channels on the
    256-channel tile (129 tiles of one 128-row block, equal ranges over 256
    workgroups, ragged N and M): 1024 sampled output channels, the last
    included, against the oracle, with and without a workspace."""
    qpn = need_gpu()
    n, k = 33000, 1024
    w = synth.weights(n, k, seed=n + m)
    x = synth.activations(m, k, seed=n + m, m_max=m)
    pw, ref = _pack(qpn, fmt, w)
    op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    pl = qpn.gemm_plan(op, m, n, k)
    assert (pl.panels_per_workgroup, pl.activation_rows, pl.workgroups) == (16, 128, 256), pl
    rows = np.sort(np.concatenate([np.random.default_rng(m).choice(n - 1, 1023, replace=False), [n - 1]]))
    y_ref = ref(x, rows)
    log(f"prefill wide 65-128 {fmt} {n}x{k} m={m}: {pl.splits} per tile")
    parity(host(qpn.prefill(pw, dev(x)))[:, rows], y_ref, f"prefill wide {fmt} {n}x{k} m={m}")
    parity(host(_prefill_one_range(qpn, pw, dev(x)))[:, rows], y_ref, f"prefill wide {fmt} {n}x{k} m={m} one K range")


def test_prefill_wide_tile_small_blocks():
    """17-64 NVFP4 rows on the 256-channel tile (32- and 64-row tiles, taken
    when the call still fills half the CUs): ragged N (33 blocks, the last
    one 8 channels) and M, with and without a workspace, every output."""
    qpn = need_gpu()
    n, k = 8200, 4096
    w = synth.weights(n, k, seed=8200)
    x = synth.activations(64, k, seed=8200, m_max=64)
    pw, ref = _pack(qpn, "nvfp4", w)
    for m in (17, 31, 32, 33, 50, 64):
        pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, m, n, k)
        assert pl.panels_per_workgroup == 16 and pl.splits > 1, (m, pl)
        log(f"prefill wide {n}x{k} m={m}: {pl.workgroups} workgroups, {pl.splits} per tile")
        xd = dev(x[:m])
        y_ref = ref(x[:m])
        parity(host(qpn.prefill(pw, xd)), y_ref, f"prefill wide {n}x{k} m={m}")
        parity(host(_prefill_one_range(qpn, pw, xd)), y_ref, f"prefill wide {n}x{k} m={m} one K range")


def test_prefill_is_deterministic_and_row_independent():
    """Two identical calls give identical bits (the workgroups that share a
    tile are summed in workgroup order, whichever finishes last), and a
    row's result does not depend on the rows around it: the first 150 rows
    of a 200-row block equal a 150-row call bit for bit (same plan, so the
    same K ranges for every tile).  A 20-row call takes the narrow tile,
    whose K ranges differ, so it is held to parity."""
    qpn = need_gpu()
    n, k = 3000, 2048
    w = synth.weights(n, k, seed=9)
    x = synth.activations(200, k, seed=9, m_max=200)
    pw, ref = _pack(qpn, "nvfp4", w)
    p200 = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 200, n, k)
    assert p200.splits > 1  # tiles are cut between workgroups
    y1 = host(qpn.prefill(pw, dev(x)))
    y2 = host(qpn.prefill(pw, dev(x)))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    parity(y1, ref(x), "prefill 200 rows")
    assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 150, n, k) == p200
    y150 = host(qpn.prefill(pw, dev(x[:150])))
    assert np.array_equal(y150.view(np.uint16), y1[:150].view(np.uint16))
    parity(host(qpn.prefill(pw, dev(x[:20]))), ref(x[:20]), "prefill 20 rows")


# (m, n, k): tiles cut between many workgroups and summed in shares (narrow
# 64- and 128-row tiles, wide tiles)
SHARE_CASES = [(96, 640, 8192), (200, 3000, 2048), (128, 1000, 6144), (200, 1500, 4096), (40, 300, 9008)]


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_prefill_shares_without_waiting(fmt):
    """No contributor waits (the path a wait that runs out takes): the last
    to arrive sums every share.  The result must be bit-identical to the
    normal call, the workspace must end all zeros, and both must meet the
    oracle."""
    qpn = need_gpu()
    op = qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    for m, n, k in SHARE_CASES:
        pl = qpn.gemm_plan(op, m, n, k)
        assert pl.splits > 1, (m, n, k, pl)
        w = synth.weights(n, k, seed=m + n)
        x = synth.activations(m, k, seed=m + n, m_max=m)
        pw, ref = _pack(qpn, fmt, w)
        ws = torch.zeros(qpn.workspace_bytes(op, m, n, k), dtype=torch.uint8, device="cuda")
        log(f"prefill {fmt} {m}x{n}x{k}: {pl.workgroups} workgroups, up to {pl.splits} per tile")
        y = host(qpn.prefill(pw, dev(x), ws=ws))
        assert not host(ws).any()
        y_nw = host(qpn.prefill(pw, dev(x), ws=ws, no_wait=True))
        assert not host(ws).any()
        assert np.array_equal(y.view(np.uint16), y_nw.view(np.uint16)), (fmt, m, n, k)
        rows = np.unique(np.linspace(0, n - 1, 96).astype(np.int64))
        parity(y[:, rows], ref(x, rows), f"prefill {fmt} {m}x{n}x{k} shares")


def test_prefill_leaves_workspace_zeroed_and_runs_without_one():
    qpn = need_gpu()
    n, k = 640, 8192
    w = synth.weights(n, k, seed=4)
    x = synth.activations(96, k, seed=4, m_max=96)
    pw, ref = _pack(qpn, "nvfp4", w)
    need = qpn.workspace_bytes(qpn.OP_PREFILL_NVFP4, 96, n, k)
    assert need > 0  # this shape splits K
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y_ref = ref(x)
    for _ in range(2):
        y = host(qpn.prefill(pw, dev(x), ws=ws))
        assert not host(ws).any()
        parity(y, y_ref, "prefill with workspace")
    # no workspace: one K range
    parity(host(_prefill_one_range(qpn, pw, dev(x))), y_ref, "prefill without workspace")


def test_prefill_wrong_blob_gives_nan():
    qpn = need_gpu()
    n, k = 256, 512
    pw8 = qpn.pack_fp8(dev(synth.weights(n, k, seed=2)))
    x = dev(synth.activations(40, k, seed=2, m_max=40))
    bad = qpn.PackedWeight(torch.zeros(qpn.nvfp4_packed_bytes(n, k), dtype=torch.uint8, device="cuda"),
                           n, k, qpn.FMT_NVFP4)
    assert np.all(np.isnan(host(qpn.prefill(bad, x)).astype(np.float32)))
    # an FP8 blob read as NVFP4 of the same shape (its header names FP8)
    blob = torch.zeros(qpn.nvfp4_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
    nb = min(blob.numel(), pw8.nbytes)
    blob[:nb] = pw8.blob[:nb]
    y = host(qpn.prefill(qpn.PackedWeight(blob, n, k, qpn.FMT_NVFP4), x))
    assert np.all(np.isnan(y.astype(np.float32)))
