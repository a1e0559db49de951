"""Thin ctypes binding of libqpn.so (the C ABI in include/qpn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libqpn.so.  torch supplies device memory and the current stream.
Importing this module loads the library and raises if it is not built; there
is no fallback of any kind.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QPN_SANITIZED_BUILD=1 loads the host-sanitized copy of the library
# (build(sanitize=True), used only by tests/run_sanitized.py on the CPU).
LIB_PATH = (os.path.join(os.path.dirname(_HERE), "_build", "sanitize", "libqpn.so")
            if os.environ.get("QPN_SANITIZED_BUILD") == "1" else os.path.join(_HERE, "libqpn.so"))

QPN_OK = 0
OP_GEMM_NVFP4 = 1
OP_GEMM_FP8 = 2
OP_LMHEAD_NVFP4 = 3
OP_PREFILL_NVFP4 = 4
OP_PREFILL_FP8 = 5

FMT_NVFP4 = "nvfp4"
FMT_FP8 = "fp8"


class QpnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m fp8_quantized_skinny_qpn_amd.build` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    c = ctypes
    vp, i64, sz, i32 = c.c_void_p, c.c_int64, c.c_size_t, c.c_int
    sig = {
        "qpn_status_string": ([i32], c.c_char_p),
        "qpn_layout_version": ([], i32),
        "qpn_nvfp4_packed_bytes": ([i64, i64], sz),
        "qpn_fp8_packed_bytes": ([i64, i64], sz),
        "qpn_workspace_bytes": ([i32, i32, i64, i64], sz),
        "qpn_gemm_plan": ([i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp], i32),
        "qpn_pack_nvfp4": ([vp, i64, i64, vp, sz, vp], i32),
        "qpn_pack_fp8": ([vp, i64, i64, vp, sz, vp], i32),
        "qpn_requant_fp8_to_nvfp4": ([vp, sz, i64, i64, vp, sz, vp], i32),
        "qpn_gemm_nvfp4": ([vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_gemm_fp8": ([vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_gemm_nvfp4_noalloc": ([vp, vp, vp, i32, i64, i64, vp], i32),
        "qpn_gemm_prefill_nvfp4": ([vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_gemm_prefill_fp8": ([vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_lmhead_nvfp4": ([vp, vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_lmhead_verify_nvfp4": ([vp, vp, vp, vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_debug_unpack_nvfp4": ([vp, i64, i64, vp, vp, vp, vp], i32),
        "qpn_debug_unpack_fp8": ([vp, i64, i64, vp, vp, vp], i32),
        "qpn_debug_decode_nvfp4": ([vp, vp, i64, vp, vp], i32),
        "qpn_debug_decode_fp8": ([vp, i64, vp, vp], i32),
        "qpn_debug_read_ceiling": ([vp, sz, vp, vp], i32),
        "qpn_debug_plan": ([i32, i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "qpn_debug_run_plan": ([i32, i32, vp, vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
        "qpn_debug_prefill_no_wait": ([i32, vp, vp, vp, i32, i64, i64, vp, sz, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()

# Symbols the C header declares (the CPU tests check that each one loads).
EXPORTED = ("qpn_status_string", "qpn_layout_version", "qpn_nvfp4_packed_bytes",
            "qpn_fp8_packed_bytes", "qpn_workspace_bytes", "qpn_gemm_plan", "qpn_pack_nvfp4", "qpn_pack_fp8",
            "qpn_requant_fp8_to_nvfp4",
            "qpn_gemm_nvfp4", "qpn_gemm_fp8", "qpn_gemm_nvfp4_noalloc", "qpn_gemm_prefill_nvfp4", "qpn_gemm_prefill_fp8",
            "qpn_lmhead_nvfp4", "qpn_lmhead_verify_nvfp4",
            "qpn_debug_unpack_nvfp4",
            "qpn_debug_unpack_fp8", "qpn_debug_decode_nvfp4", "qpn_debug_decode_fp8",
            "qpn_debug_read_ceiling", "qpn_debug_plan", "qpn_debug_run_plan",
            "qpn_debug_prefill_no_wait")


def status_string(rc: int) -> str:
    return lib.qpn_status_string(int(rc)).decode()


def check(rc: int):
    if rc != QPN_OK:
        raise QpnError(rc, status_string(rc))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch_stream(stream=None):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream=None):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _empty(ts, shape, dtype, device):
    # allocated on the stream the kernel runs on, so the caching allocator
    # never hands out a block that work queued on another stream still uses
    with torch.cuda.stream(ts):
        return torch.empty(shape, dtype=dtype, device=device)


def nvfp4_packed_bytes(n: int, k: int) -> int:
    return int(lib.qpn_nvfp4_packed_bytes(n, k))


def fp8_packed_bytes(n: int, k: int) -> int:
    return int(lib.qpn_fp8_packed_bytes(n, k))


def workspace_bytes(op: int, m: int, n: int, k: int, plan: int = 0) -> int:
    """Workspace a call uses; `plan` > 0 asks for a forced (diagnostic) plan."""
    if plan == 0:
        return int(lib.qpn_workspace_bytes(op, m, n, k))
    out = ctypes.c_size_t()
    check(lib.qpn_debug_plan(op, plan, m, n, k, *([None] * 8), ctypes.byref(out)))
    return int(out.value)


@dataclass(frozen=True)
class Plan:
    """Launch plan of one call, as the library reports it."""
    workgroups: int
    waves_per_panel: int
    panels_per_workgroup: int
    prefetch_depth: int
    splits: int
    activation_rows: int
    split_workgroups: int   # workgroups on K ranges; the rest take whole panels
    valu_dot: int = 0       # 1: VALU dot products instead of MFMA (diagnostic plans)

    @property
    def waves_per_workgroup(self) -> int:
        return self.waves_per_panel * self.panels_per_workgroup


def gemm_plan(op: int, m: int, n: int, k: int, plan: int = 0) -> Plan:
    """The launch plan the library uses for a call of kind `op` (given the
    workspace qpn_workspace_bytes asks for); `plan` > 0 reports a forced
    (diagnostic) plan through qpn_debug_plan."""
    wg = ctypes.c_int64()
    swg = ctypes.c_int64()
    outs = [ctypes.c_int() for _ in range(5)]
    vd = ctypes.c_int()
    refs = [ctypes.byref(o) for o in outs]
    if plan == 0:
        check(lib.qpn_gemm_plan(op, m, n, k, ctypes.byref(wg), *refs, ctypes.byref(swg)))
    else:
        check(lib.qpn_debug_plan(op, plan, m, n, k, ctypes.byref(wg), *refs, ctypes.byref(swg),
                                 ctypes.byref(vd), None))
    return Plan(wg.value, *[o.value for o in outs], swg.value, vd.value)


def plan_ids():
    """Every compiled launch plan id (probed through qpn_debug_plan)."""
    ids = []
    for i in range(1, 65):
        if lib.qpn_debug_plan(OP_GEMM_NVFP4, i, 1, 16, 16, *([None] * 9)) == QPN_OK:
            ids.append(i)
    return ids


def kernel_name(fmt: str, m: int, n: int, k: int, lmhead: bool = False, plan: int = 0) -> str:
    """Demangled name (template part) of the GEMM kernel a call launches."""
    op = OP_LMHEAD_NVFP4 if lmhead else (OP_GEMM_NVFP4 if fmt == FMT_NVFP4 else OP_GEMM_FP8)
    pl = gemm_plan(op, m, n, k, plan)
    f = 1 if fmt == FMT_NVFP4 else 2
    return (f"qpn::skinny_gemm_kernel<{f}u, {pl.waves_per_panel}, {pl.panels_per_workgroup}, "
            f"{pl.prefetch_depth}, {pl.activation_rows}, {'true' if lmhead else 'false'}, "
            f"{'true' if pl.valu_dot else 'false'}>")


# Zero-initialised workspaces, one per (device, stream): the library leaves a
# workspace's split-K counters at zero after every call, so a workspace is
# zeroed once, when it is allocated, and then reused by calls on its stream.
# It is allocated and zeroed on that stream, so the zero-fill is ordered
# before every kernel that uses it, and a replaced buffer is kept alive
# until the work already queued on the stream is done.
_workspaces = {}


def workspace(nbytes: int, device, stream) -> torch.Tensor:
    """The cached zero-filled workspace of at least nbytes for `stream` (a
    torch stream) on `device`."""
    key = (torch.device(device).index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            new = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        if ws is not None:
            ws.record_stream(stream)
        _workspaces[key] = ws = new
    return ws


@dataclass
class PackedWeight:
    """A packed weight blob on the device plus the shape it was packed for."""
    blob: torch.Tensor  # uint8, device
    n: int
    k: int
    fmt: str

    @property
    def nbytes(self) -> int:
        return self.blob.numel()

    def clone(self) -> "PackedWeight":
        return PackedWeight(self.blob.clone(), self.n, self.k, self.fmt)


def _dev_f32(w):
    if not (w.is_cuda and w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous()):
        raise ValueError("weights must be a contiguous 2-D float32 CUDA tensor")


def pack_nvfp4(w: torch.Tensor, stream=None) -> PackedWeight:
    _dev_f32(w)
    n, k = w.shape
    nb = nvfp4_packed_bytes(n, k)
    if nb == 0:
        raise QpnError(2, status_string(2))
    blob = _empty(_torch_stream(stream), (nb,), torch.uint8, w.device)
    check(lib.qpn_pack_nvfp4(_ptr(w), n, k, _ptr(blob), nb, _stream(stream)))
    return PackedWeight(blob, n, k, FMT_NVFP4)


def pack_fp8(w: torch.Tensor, stream=None) -> PackedWeight:
    _dev_f32(w)
    n, k = w.shape
    nb = fp8_packed_bytes(n, k)
    if nb == 0:
        raise QpnError(2, status_string(2))
    blob = _empty(_torch_stream(stream), (nb,), torch.uint8, w.device)
    check(lib.qpn_pack_fp8(_ptr(w), n, k, _ptr(blob), nb, _stream(stream)))
    return PackedWeight(blob, n, k, FMT_FP8)


def requant_fp8_to_nvfp4(pw: PackedWeight, stream=None) -> PackedWeight:
    """The NVFP4 blob converted from an FP8 blob through qpn_requant_fp8_to_nvfp4."""
    if pw.fmt != FMT_FP8:
        raise ValueError("the source must be an FP8 blob")
    nb = nvfp4_packed_bytes(pw.n, pw.k)
    if nb == 0:
        raise QpnError(2, status_string(2))
    blob = _empty(_torch_stream(stream), (nb,), torch.uint8, pw.blob.device)
    check(lib.qpn_requant_fp8_to_nvfp4(_ptr(pw.blob), pw.nbytes, pw.n, pw.k, _ptr(blob), nb,
                                       _stream(stream)))
    return PackedWeight(blob, pw.n, pw.k, FMT_NVFP4)


def _x_check(x, k):
    if not (x.is_cuda and x.dtype == torch.float16 and x.dim() == 2 and x.is_contiguous()):
        raise ValueError("activations must be a contiguous 2-D float16 CUDA tensor")
    if x.shape[1] != k:
        raise ValueError(f"activation K {x.shape[1]} does not match the packed K {k}")


def gemm(pw: PackedWeight, x: torch.Tensor, out: torch.Tensor = None, stream=None,
         ws: torch.Tensor = None, plan: int = 0) -> torch.Tensor:
    """Y = X * What^T through qpn_gemm_nvfp4 / qpn_gemm_fp8 (through
    qpn_debug_run_plan with a forced plan when `plan` > 0).  `ws` (zero-filled
    before its first use) defaults to a cached per-stream workspace."""
    _x_check(x, pw.k)
    m = x.shape[0]
    ts = _torch_stream(stream)
    st = _stream(ts)
    if out is None:
        out = _empty(ts, (m, pw.n), torch.float16, x.device)
    op = OP_GEMM_NVFP4 if pw.fmt == FMT_NVFP4 else OP_GEMM_FP8
    need = workspace_bytes(op, m, pw.n, pw.k, plan) if m > 0 else 0
    if ws is None and need > 0:
        ws = workspace(need, x.device, ts)
    wp, wn = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    if plan == 0:
        fn = lib.qpn_gemm_nvfp4 if pw.fmt == FMT_NVFP4 else lib.qpn_gemm_fp8
        check(fn(_ptr(pw.blob), _ptr(x), _ptr(out), m, pw.n, pw.k, wp, wn, st))
    else:
        check(lib.qpn_debug_run_plan(op, plan, _ptr(pw.blob), _ptr(x), _ptr(out), None, m, pw.n,
                                     pw.k, wp, wn, st))
    return out


def prefill(pw: PackedWeight, x: torch.Tensor, out: torch.Tensor = None, stream=None,
            ws: torch.Tensor = None, no_wait: bool = False) -> torch.Tensor:
    """Y = X * What^T for 0 <= m <= 256 activation rows through
    qpn_gemm_prefill_nvfp4 / qpn_gemm_prefill_fp8 (qpn_debug_prefill_no_wait
    when `no_wait`).  `ws` (zero-filled before its first use) defaults to a
    cached per-stream workspace."""
    _x_check(x, pw.k)
    m = x.shape[0]
    ts = _torch_stream(stream)
    st = _stream(ts)
    if out is None:
        out = _empty(ts, (m, pw.n), torch.float16, x.device)
    op = OP_PREFILL_NVFP4 if pw.fmt == FMT_NVFP4 else OP_PREFILL_FP8
    fn = lib.qpn_gemm_prefill_nvfp4 if pw.fmt == FMT_NVFP4 else lib.qpn_gemm_prefill_fp8
    need = workspace_bytes(op, m, pw.n, pw.k) if m > 0 else 0
    if ws is None and need > 0:
        ws = workspace(need, x.device, ts)
    wsp, wsn = (_ptr(ws), ws.numel()) if ws is not None else (None, 0)
    if no_wait:
        check(lib.qpn_debug_prefill_no_wait(op, _ptr(pw.blob), _ptr(x), _ptr(out), m, pw.n, pw.k,
                                            wsp, wsn, st))
    else:
        check(fn(_ptr(pw.blob), _ptr(x), _ptr(out), m, pw.n, pw.k, wsp, wsn, st))
    return out


def lmhead_nvfp4(pw: PackedWeight, x: torch.Tensor, logits=None, argmax=None, workspace_=None,
                 stream=None, plan: int = 0):
    """(logits fp16 [m, n], argmax int32 [m]) through qpn_lmhead_nvfp4 (through
    qpn_debug_run_plan with a forced plan when `plan` > 0)."""
    if pw.fmt != FMT_NVFP4:
        raise ValueError("lm_head needs an NVFP4 blob")
    _x_check(x, pw.k)
    m = x.shape[0]
    ts = _torch_stream(stream)
    st = _stream(ts)
    if logits is None:
        logits = _empty(ts, (m, pw.n), torch.float16, x.device)
    if argmax is None:
        argmax = _empty(ts, (m,), torch.int32, x.device)
    need = workspace_bytes(OP_LMHEAD_NVFP4, m, pw.n, pw.k, plan)
    ws = workspace_ if workspace_ is not None else workspace(max(need, 8), x.device, ts)
    if plan == 0:
        check(lib.qpn_lmhead_nvfp4(_ptr(pw.blob), _ptr(x), _ptr(logits), _ptr(argmax), m, pw.n,
                                   pw.k, _ptr(ws), ws.numel(), st))
    else:
        check(lib.qpn_debug_run_plan(OP_LMHEAD_NVFP4, plan, _ptr(pw.blob), _ptr(x), _ptr(logits),
                                     _ptr(argmax), m, pw.n, pw.k, _ptr(ws), ws.numel(), st))
    return logits, argmax


def lmhead_verify_nvfp4(pw: PackedWeight, x: torch.Tensor, draft: torch.Tensor, logits=None,
                        argmax=None, result=None, workspace_=None, stream=None):
    """(logits, argmax, result int32 [2] = (accepted drafts, next token)) through
    qpn_lmhead_verify_nvfp4; draft: int32 [m - 1] on the device."""
    if pw.fmt != FMT_NVFP4:
        raise ValueError("lm_head needs an NVFP4 blob")
    _x_check(x, pw.k)
    m = x.shape[0]
    if draft.dtype != torch.int32 or draft.dim() != 1 or draft.numel() != max(m - 1, 0):
        raise ValueError("draft must be int32 [m - 1]")
    if draft.numel() and (draft.device != x.device or not draft.is_contiguous()):
        raise ValueError("draft must be contiguous on the activation's device")
    ts = _torch_stream(stream)
    st = _stream(ts)
    if logits is None:
        logits = _empty(ts, (m, pw.n), torch.float16, x.device)
    if argmax is None:
        argmax = _empty(ts, (m,), torch.int32, x.device)
    if result is None:
        result = _empty(ts, (2,), torch.int32, x.device)
    need = workspace_bytes(OP_LMHEAD_NVFP4, m, pw.n, pw.k)
    ws = workspace_ if workspace_ is not None else workspace(max(need, 8), x.device, ts)
    check(lib.qpn_lmhead_verify_nvfp4(_ptr(pw.blob), _ptr(x), _ptr(logits), _ptr(argmax),
                                      _ptr(draft) if draft.numel() else None, _ptr(result), m,
                                      pw.n, pw.k, _ptr(ws), ws.numel(), st))
    return logits, argmax, result


def debug_unpack_nvfp4(pw: PackedWeight, stream=None):
    """Canonical (codes [n, k/2], scales [n, k/16], g) read back from the blob."""
    dev, ts = pw.blob.device, _torch_stream(stream)
    codes = _empty(ts, (pw.n, pw.k // 2), torch.uint8, dev)
    scales = _empty(ts, (pw.n, pw.k // 16), torch.uint8, dev)
    g = _empty(ts, (1,), torch.float32, dev)
    check(lib.qpn_debug_unpack_nvfp4(_ptr(pw.blob), pw.n, pw.k, _ptr(codes), _ptr(scales), _ptr(g),
                                     _stream(stream)))
    return codes, scales, g


def debug_unpack_fp8(pw: PackedWeight, stream=None):
    """Canonical (codes [n, k], row_scale [n]) read back from the blob."""
    dev, ts = pw.blob.device, _torch_stream(stream)
    codes = _empty(ts, (pw.n, pw.k), torch.uint8, dev)
    rs = _empty(ts, (pw.n,), torch.float32, dev)
    check(lib.qpn_debug_unpack_fp8(_ptr(pw.blob), pw.n, pw.k, _ptr(codes), _ptr(rs),
                                   _stream(stream)))
    return codes, rs


def debug_decode_nvfp4(codes16: torch.Tensor, scales2: torch.Tensor, stream=None) -> torch.Tensor:
    f = codes16.shape[0]
    out = _empty(_torch_stream(stream), (f, 32), torch.float16, codes16.device)
    check(lib.qpn_debug_decode_nvfp4(_ptr(codes16), _ptr(scales2), f, _ptr(out), _stream(stream)))
    return out


def debug_decode_fp8(codes16: torch.Tensor, stream=None) -> torch.Tensor:
    f = codes16.shape[0]
    out = _empty(_torch_stream(stream), (f, 16), torch.float16, codes16.device)
    check(lib.qpn_debug_decode_fp8(_ptr(codes16), f, _ptr(out), _stream(stream)))
    return out


def debug_read_ceiling(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """One streaming read of `buf` (the measured read ceiling kernel)."""
    check(lib.qpn_debug_read_ceiling(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                     _stream(stream)))
