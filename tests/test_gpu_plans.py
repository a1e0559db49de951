"""Every branch of the automatic launch-plan choice, on a shape that selects
it, against the oracle (every output element).

The branches, both formats unless named:
- one panel per workgroup below 256 panels, at any m;
- at 1-2 rows (up to 256-767 panels with a remainder of 16 or more): the
  remainder split in K over a long K (64 or more k-steps; eight wavefronts
  per panel for NVFP4, four for FP8), and over a short K with 512 or more
  panels and a remainder of 64 or more (four wavefronts); whole panels for
  a short K otherwise;
- at 3-8 rows: two panels per workgroup over fewer than 512 panels when the
  whole activation slice fits the LDS budget; else five panels per
  workgroup (with twice the K splits the LDS budget forces when those still
  fit 256 workgroups); eight NVFP4 panels per workgroup for 2048 or more
  panels when they fill whole rounds of 256 CUs; one workgroup per CU with
  all its 8-16 panels (one wavefront each) when neither the eight- nor the
  five-panel workgroups fill 82% of their rounds;
- NVFP4 at 2 rows: the eight- and sixteen-panel plans as at 3-8 rows;
- FP8 at 9-16 rows (the 16-row prefill tile): two panels per workgroup.
The plan fields reported through the C ABI are asserted first, so each case
covers the branch it names.
"""
import numpy as np
import pytest

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import check_argmax, dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu

# (fmt, n, k, m, waves_per_panel, panels_per_workgroup, whole-panel workgroups present, branch)
CASES = [
    ("nvfp4", 2000, 1024, 1, 4, 1, False, "one panel per workgroup, < 256 panels"),
    ("nvfp4", 2000, 1024, 8, 4, 1, False, "one panel per workgroup, < 256 panels, 8 rows"),
    ("fp8", 2000, 1024, 8, 4, 1, False, "one panel per workgroup, < 256 panels, FP8 8 rows"),
    ("nvfp4", 5120, 8192, 1, 8, 1, True, "remainder split, long K, NVFP4"),
    ("nvfp4", 5120, 8192, 2, 8, 1, True, "remainder split, long K, NVFP4, 2 rows"),
    ("fp8", 5120, 4096, 2, 4, 1, True, "remainder split, long K, FP8"),
    ("nvfp4", 10240, 2048, 1, 4, 1, True, "remainder split, short K, >= 512 panels"),
    ("nvfp4", 8704, 2048, 1, 4, 1, False, "whole panels, short K, remainder under a quarter round"),
    ("nvfp4", 5120, 2048, 1, 4, 1, False, "whole panels, short K, < 512 panels"),
    ("nvfp4", 8200, 2048, 5, 3, 5, False, "five panels per workgroup"),
    ("nvfp4", 4100, 2048, 5, 4, 2, False, "two NVFP4 panels per workgroup, 1-2 panels per CU"),
    ("nvfp4", 4100, 10368, 4, 3, 5, False, "five panels per workgroup, LDS-forced K splits doubled"),
    ("fp8", 4100, 2048, 6, 4, 2, False, "two FP8 panels per workgroup"),
    ("fp8", 4100, 4096, 4, 4, 2, False, "two FP8 panels per workgroup, 4 rows, long K"),
    ("fp8", 8704, 1024, 8, 3, 5, False, "five FP8 panels per workgroup, 512 or more panels"),
    ("fp8", 49152, 256, 4, 1, 16, False, "sixteen FP8 panels per workgroup"),
    ("nvfp4", 17400, 512, 2, 4, 1, False, "one panel per workgroup, 2 rows, 768 or more panels"),
    ("nvfp4", 32768, 512, 2, 2, 8, False, "eight panels per workgroup, 2 rows"),
    ("nvfp4", 32768, 512, 8, 2, 8, False, "eight panels per workgroup, 8 rows"),
    ("nvfp4", 49152, 256, 2, 1, 16, False, "sixteen panels per workgroup, 2 rows"),
    ("nvfp4", 49152, 256, 8, 1, 16, False, "sixteen panels per workgroup, 8 rows"),
]


def _pack(qpn, fmt, w):
    if fmt == "nvfp4":
        codes, scales, g = oracle.pack_nvfp4(w)
        return qpn.pack_nvfp4(dev(w)), lambda x: oracle.gemm_nvfp4(codes, scales, g, x)
    codes, rs = oracle.pack_fp8(w)
    return qpn.pack_fp8(dev(w)), lambda x: oracle.gemm_fp8(codes, rs, x)


@pytest.mark.parametrize("fmt,n,k,m,wpp,ppw,whole,branch", CASES, ids=[c[-1] for c in CASES])
def test_automatic_plan_branch(fmt, n, k, m, wpp, ppw, whole, branch):
    qpn = need_gpu()
    op = qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8
    pl = qpn.gemm_plan(op, m, n, k)
    assert (pl.waves_per_panel, pl.panels_per_workgroup) == (wpp, ppw), (branch, pl)
    assert (pl.workgroups > pl.split_workgroups) == whole, (branch, pl)
    w = synth.weights(n, k, seed=n + k + m)
    x = synth.activations(m, k, seed=n + k + m)
    pw, ref = _pack(qpn, fmt, w)
    if "doubled" in branch:
        assert (pl.workgroups, pl.splits) == (208, 4), pl   # 52 groups of five panels
    log(f"plan branch '{branch}': {fmt} {n}x{k} m={m}, {pl.workgroups} workgroups, {pl.splits} splits")
    parity(host(qpn.gemm(pw, dev(x))), ref(x), f"{branch}: {fmt} {n}x{k} m={m}")


def test_lmhead_eight_panel_plan():
    """The lm_head (argmax fused) through the eight-panel plan: logits within
    the parity bar and the argmax equal to the oracle's on every row (apart
    from rows made ambiguous by FP16 rounding, see gpu_util.check_argmax)."""
    qpn = need_gpu()
    n, k, m = 32768, 512, 8
    pl = qpn.gemm_plan(qpn.OP_LMHEAD_NVFP4, m, n, k)
    assert (pl.waves_per_panel, pl.panels_per_workgroup) == (2, 8)
    w = synth.weights(n, k, seed=11)
    x = synth.activations(m, k, seed=11)
    pw, ref = _pack(qpn, "nvfp4", w)
    lg, am = qpn.lmhead_nvfp4(pw, dev(x))
    lg, am = host(lg), host(am)
    y_ref = ref(x)
    parity(lg, y_ref, "lm_head eight-panel plan")
    check_argmax(am, lg, y_ref, "lm_head eight-panel plan")
