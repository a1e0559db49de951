"""A bounded soak of the split-K exchange: 1200 calls chained on one stream
and one workspace, every output bit-identical to the first result of its
call.

The calls interleave, in a fixed pseudo-random order: NVFP4 and FP8 GEMMs
whose automatic plans split K 2, 3, 4, 5, 6, 7, 10, 13 and 18 ways; the
balanced hybrid launches (whole panels plus a K-split remainder, four and
six splits); lm_head calls with split K; the 16-row skinny prefill tile and
the tiled prefill kernel with tiles cut between workgroups (narrow and
wide tiles, summed up the pairwise tree and in shares, and more tiles than
CUs in one round of 256 ranges); and the no-allocation GEMM on the
library's own scratch.  Every 40 calls the outputs are compared bit for bit
with the first result of their call, stopping at the first mismatch.  The
first result of each call is checked against the oracle on sampled rows, and
the workspace must be all zeros at the end.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_quantized_skinny_qpn_amd import synth
from gpu_util import dev, host, log, need_gpu, parity

pytestmark = pytest.mark.gpu

CALLS_TOTAL = 1200
CHECK_EVERY = 40

# (kind, fmt, m, n, k, splits the automatic plan takes)
CASES = [
    ("gemm", "nvfp4", 2, 300, 2048, 2), ("gemm", "nvfp4", 2, 1000, 4096, 3),
    ("gemm", "nvfp4", 2, 300, 4096, 4), ("gemm", "nvfp4", 5, 1000, 24576, 5),
    ("gemm", "nvfp4", 2, 300, 6144, 6), ("gemm", "nvfp4", 8, 300, 8192, 7),
    ("gemm", "nvfp4", 8, 160, 10240, 10), ("gemm", "fp8", 2, 2000, 2048, 2),
    ("gemm", "fp8", 2, 1000, 2048, 3), ("gemm", "fp8", 8, 160, 10240, 13),
    ("gemm", "fp8", 4, 100, 10240, 18),
    ("gemm", "nvfp4", 1, 5120, 17408, 4), ("gemm", "nvfp4", 1, 4805, 16000, 6),
    ("lmhead", "nvfp4", 2, 300, 2048, 2), ("lmhead", "nvfp4", 8, 1000, 4096, 3),
    ("prefill", "nvfp4", 16, 300, 9008, 7), ("prefill", "fp8", 9, 300, 4096, 7),
    ("prefill", "nvfp4", 40, 300, 9008, 8), ("prefill", "nvfp4", 200, 1500, 4096, 4),
    ("prefill", "fp8", 128, 1000, 6144, 6), ("prefill", "fp8", 40, 300, 20000, 39),
    ("prefill", "fp8", 32, 33000, 1024, 2),
    ("noalloc", "nvfp4", 8, 300, 8192, 7),
]


def _op(qpn, kind, fmt):
    if kind == "lmhead":
        return qpn.OP_LMHEAD_NVFP4
    if kind == "prefill":
        return qpn.OP_PREFILL_NVFP4 if fmt == "nvfp4" else qpn.OP_PREFILL_FP8
    return qpn.OP_GEMM_NVFP4 if fmt == "nvfp4" else qpn.OP_GEMM_FP8


def test_split_k_soak():
    import ctypes
    qpn = need_gpu()
    runs, need = [], 256
    for i, (kind, fmt, m, n, k, splits) in enumerate(CASES):
        op = _op(qpn, kind, fmt)
        pl = qpn.gemm_plan(op, m, n, k)
        assert pl.splits == splits, (kind, fmt, m, n, k, pl)
        need = max(need, qpn.workspace_bytes(op, m, n, k))
        w = synth.weights(n, k, seed=100 + i)
        x = synth.activations(max(m, 8), k, seed=100 + i, m_max=max(m, 8))[:m]
        pw = qpn.pack_nvfp4(dev(w)) if fmt == "nvfp4" else qpn.pack_fp8(dev(w))
        rows = np.unique(np.linspace(0, n - 1, 64).astype(np.int64))
        if fmt == "nvfp4":
            g, _ = oracle.nvfp4_tensor_scale(w)
            c, s = oracle.pack_nvfp4_rows(w[rows], g)
            ref = oracle.gemm_nvfp4(c, s, g, x)
        else:
            c, rs = oracle.pack_fp8(w[rows])
            ref = oracle.gemm_fp8(c, rs, x)
        runs.append({"case": (kind, fmt, m, n, k), "pw": pw, "x": dev(x), "rows": rows, "ref": ref,
                     "y": torch.empty((m, n), dtype=torch.float16, device="cuda"),
                     "am": torch.empty((m,), dtype=torch.int32, device="cuda"), "first": None})
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(r):
        kind, fmt, m, n, k = r["case"]
        if kind == "gemm":
            qpn.gemm(r["pw"], r["x"], out=r["y"], ws=ws)
        elif kind == "prefill":
            qpn.prefill(r["pw"], r["x"], out=r["y"], ws=ws)
        elif kind == "lmhead":
            qpn.lmhead_nvfp4(r["pw"], r["x"], logits=r["y"], argmax=r["am"], workspace_=ws)
        else:
            qpn.check(qpn.lib.qpn_gemm_nvfp4_noalloc(
                ctypes.c_void_p(r["pw"].blob.data_ptr()), ctypes.c_void_p(r["x"].data_ptr()),
                ctypes.c_void_p(r["y"].data_ptr()), m, n, k, stream))

    # first results, against the oracle
    for r in runs:
        launch(r)
        y = host(r["y"])
        parity(y[:, r["rows"]], r["ref"], f"soak first result {r['case']}")
        r["first"] = r["y"].clone()
        r["first_am"] = r["am"].clone()
        if r["case"][0] == "lmhead":
            assert np.array_equal(host(r["am"]), np.argmax(y, axis=1))
    order = np.random.default_rng(2024).integers(0, len(runs), CALLS_TOTAL)
    pending = []
    for ci, ri in enumerate(order):
        r = runs[int(ri)]
        launch(r)
        # compared on the device, in stream order, before the next call of
        # this case overwrites the output
        diff = (r["y"].view(torch.int16) != r["first"].view(torch.int16)).any()
        if r["case"][0] == "lmhead":
            diff = diff | (r["am"] != r["first_am"]).any()
        pending.append((ci, r["case"], diff))
        if (ci + 1) % CHECK_EVERY == 0 or ci + 1 == CALLS_TOTAL:
            for cj, case, d in pending:
                assert not bool(d.item()), f"call {cj} ({case}): output differs from its first result"
            pending = []
            if (ci + 1) % 400 == 0:
                log(f"soak: {ci + 1} calls bit-identical")
    assert not host(ws).any(), "workspace not left zero-filled"
