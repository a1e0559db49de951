"""Calls issued on a torch stream other than the current one.

The binding zero-fills the cached workspace and allocates outputs on the
stream a call runs on, so split-K GEMM, prefill with cut tiles and the
lm_head argmax on a side stream give the same bits as on the current stream,
and leave their workspace zero-filled.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import check_argmax, dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    assert np.array_equal(host(a).view(np.uint16), host(b).view(np.uint16)), what


def test_side_stream_calls():
    qpn = need_gpu()
    side = torch.cuda.Stream()  # default priority
    # 65 panels: at m = 8 the automatic plan splits K (GEMM and lm_head alike)
    n, k = 1040, 5120
    w = synth.weights(n, k, seed=31)
    x = synth.activations(64, k, seed=31)
    pw = qpn.pack_nvfp4(dev(w))
    xd = dev(x)
    torch.cuda.synchronize()
    assert qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, n, k).splits > 1
    assert qpn.workspace_bytes(qpn.OP_PREFILL_NVFP4, 64, n, k) > 0  # tiles cut between workgroups
    log(f"side stream: gemm m=8, prefill m=64, lm_head m=8 on {n}x{k}")
    y_cur = qpn.gemm(pw, xd[:8])
    p_cur = qpn.prefill(pw, xd)
    lg_cur, am_cur = qpn.lmhead_nvfp4(pw, xd[:8])
    torch.cuda.synchronize()
    for rep in range(3):
        y_s = qpn.gemm(pw, xd[:8], stream=side)
        p_s = qpn.prefill(pw, xd, stream=side)
        lg_s, am_s = qpn.lmhead_nvfp4(pw, xd[:8], stream=side)
        side.synchronize()
        _same(y_s, y_cur, f"gemm rep {rep}")
        _same(p_s, p_cur, f"prefill rep {rep}")
        _same(lg_s, lg_cur, f"lm_head logits rep {rep}")
        assert np.array_equal(host(am_s), host(am_cur)), f"lm_head argmax rep {rep}"
    # the side stream's cached workspace is zero again after its calls
    key = (torch.cuda.current_device(), side.cuda_stream)
    assert int(qpn._workspaces[key].count_nonzero()) == 0
    codes, scales, g = oracle.pack_nvfp4(w)
    y_ref = oracle.gemm_nvfp4(codes, scales, g, x[:8])
    parity(host(y_s), y_ref, "side-stream gemm")
    parity(host(p_s), oracle.gemm_nvfp4(codes, scales, g, x), "side-stream prefill")
    check_argmax(host(am_s), host(lg_s), y_ref, "side-stream lm_head")
