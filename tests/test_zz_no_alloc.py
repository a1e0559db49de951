"""qpn_gemm_nvfp4_noalloc (the entry point for callers that cannot allocate)
against qpn_gemm_nvfp4 with a caller workspace, through the C ABI.

Two calls in a row on the library's static scratch, the second with a
smaller input: the first splits K four ways at M = 8 (its partials and
counters go through the scratch), the second splits a smaller shape, so it
only gets the right answer if the first left the scratch zero-filled.  Each
output is held to the parity bar against the entry point with a workspace
(and is bit-identical to it, since both run the same launch plan) and
against the oracle on sampled rows.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu

CALLS = [(5120, 17408, 8), (300, 9008, 5)]   # (n, k, m): the second is smaller


def _noalloc(qpn, pw, x, y):
    return qpn.lib.qpn_gemm_nvfp4_noalloc(ctypes.c_void_p(pw.blob.data_ptr()),
                                          ctypes.c_void_p(x.data_ptr()),
                                          ctypes.c_void_p(y.data_ptr()), x.shape[0], pw.n, pw.k,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _with_workspace(qpn, pw, x, y, ws):
    return qpn.lib.qpn_gemm_nvfp4(ctypes.c_void_p(pw.blob.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), x.shape[0], pw.n, pw.k,
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_point():
    qpn = need_gpu()
    for i, (n, k, m) in enumerate(CALLS):
        pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, m, n, k)
        log(f"noalloc call {i}: {n}x{k} m={m}, {pl.splits} K splits")
        assert pl.splits > 1, "the case must go through the scratch"
        w = synth.weights(n, k, seed=31 + i)
        x = dev(synth.activations(8, k, seed=31 + i)[:m])
        pw = qpn.pack_nvfp4(dev(w))
        y0 = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
        y1 = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
        assert _noalloc(qpn, pw, x, y0) == qpn.QPN_OK
        ws = torch.zeros(qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, m, n, k), dtype=torch.uint8,
                         device="cuda")
        assert _with_workspace(qpn, pw, x, y1, ws) == qpn.QPN_OK
        a, b = host(y0), host(y1)
        parity(a, b.astype(np.float64), f"noalloc vs workspace call {i}")
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"call {i}: not bit-identical"
        rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 97)), [n - 1]]))
        g, _ = oracle.nvfp4_tensor_scale(w)
        c, s = oracle.pack_nvfp4_rows(w[rows], g)
        parity(a[:, rows], oracle.gemm_nvfp4(c, s, g, host(x)), f"noalloc vs oracle call {i}")


def test_noalloc_argument_errors():
    qpn = need_gpu()
    v = ctypes.c_void_p
    f = qpn.lib.qpn_gemm_nvfp4_noalloc
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    assert f(v(0), v(p), v(p), 1, 16, 16, None) == 1
    assert f(v(p), v(p), v(p), 9, 16, 16, None) == 2
    assert f(v(p + 16), v(p), v(p), 1, 16, 16, None) == 3
    assert f(v(p), v(p), v(p), 0, 16, 16, None) == 0
    # K = 2^20 at 8 rows over 2^24 rows would need far more than the scratch
    assert f(v(p), v(p), v(p), 8, 1 << 24, 1 << 20, None) == 7
    assert "static scratch" in qpn.status_string(7)
