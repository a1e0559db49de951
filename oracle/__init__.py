"""The CPU oracle for the QPN skinny GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It wraps oracle/qpn_oracle.c (plain C, FP64) with
ctypes and numpy; it shares nothing with the HIP library.

What each function computes, and where it comes from, is documented in
qpn_oracle.c next to the C function of the same name.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def lib():
    """Load the oracle library, compiling it first if it is not built."""
    global _LIB
    if _LIB is None:
        # QPN_SANITIZED_BUILD=1: the ASan/UBSan copy (tests/run_sanitized.py)
        path = _build.SANITIZED_LIB if os.environ.get("QPN_SANITIZED_BUILD") == "1" else _build.LIB
        if not os.path.exists(path):
            _build.build(sanitize=path != _build.LIB)
        L = ctypes.CDLL(path)
        c = ctypes
        L.qpn_oracle_e2m1_value.argtypes = [c.c_int]
        L.qpn_oracle_e2m1_value.restype = c.c_double
        L.qpn_oracle_e4m3_value.argtypes = [c.c_int]
        L.qpn_oracle_e4m3_value.restype = c.c_double
        L.qpn_oracle_ue4m3_value.argtypes = [c.c_int, c.POINTER(c.c_double)]
        L.qpn_oracle_ue4m3_value.restype = c.c_int
        L.qpn_oracle_f16_value.argtypes = [c.c_uint16]
        L.qpn_oracle_f16_value.restype = c.c_double
        L.qpn_oracle_f16_round.argtypes = [c.c_double]
        L.qpn_oracle_f16_round.restype = c.c_uint16
        L.qpn_oracle_quant_e2m1.argtypes = [c.c_float]
        L.qpn_oracle_quant_e2m1.restype = c.c_int
        L.qpn_oracle_quant_e4m3.argtypes = [c.c_float]
        L.qpn_oracle_quant_e4m3.restype = c.c_int
        L.qpn_oracle_nvfp4_tensor_scale.argtypes = [c.c_void_p, c.c_int64, c.POINTER(c.c_float)]
        L.qpn_oracle_nvfp4_tensor_scale.restype = c.c_float
        L.qpn_oracle_pack_nvfp4_rows.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_float,
                                                 c.c_void_p, c.c_void_p]
        L.qpn_oracle_pack_nvfp4_rows.restype = c.c_int
        L.qpn_oracle_pack_fp8_rows.argtypes = [c.c_void_p, c.c_int64, c.c_int64, c.c_void_p,
                                               c.c_void_p]
        L.qpn_oracle_pack_fp8_rows.restype = c.c_int
        L.qpn_oracle_dequant_nvfp4.argtypes = [c.c_void_p, c.c_void_p, c.c_float, c.c_int64,
                                               c.c_int64, c.c_void_p]
        L.qpn_oracle_dequant_nvfp4.restype = c.c_int
        L.qpn_oracle_dequant_fp8.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64,
                                             c.c_void_p]
        L.qpn_oracle_dequant_fp8.restype = None
        L.qpn_oracle_gemm_f64.argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int64, c.c_int64,
                                          c.c_void_p]
        L.qpn_oracle_gemm_f64.restype = None
        L.qpn_oracle_gemm_nvfp4.argtypes = [c.c_void_p, c.c_void_p, c.c_float, c.c_void_p,
                                            c.c_int, c.c_int64, c.c_int64, c.c_void_p]
        L.qpn_oracle_gemm_nvfp4.restype = c.c_int
        L.qpn_oracle_gemm_fp8.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int, c.c_int64,
                                          c.c_int64, c.c_void_p]
        L.qpn_oracle_gemm_fp8.restype = None
        L.qpn_oracle_argmax_f16.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_void_p]
        L.qpn_oracle_argmax_f16.restype = None
        L.qpn_oracle_round_f16_array.argtypes = [c.c_void_p, c.c_int64, c.c_void_p]
        L.qpn_oracle_round_f16_array.restype = None
        L.qpn_oracle_threads.argtypes = []
        L.qpn_oracle_threads.restype = c.c_int
        L.qpn_oracle_set_threads.argtypes = [c.c_int]
        L.qpn_oracle_set_threads.restype = None
        _LIB = L
    return _LIB


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().qpn_oracle_threads())


def set_threads(n: int) -> None:
    """Threads of later parallel loops (results do not depend on it)."""
    lib().qpn_oracle_set_threads(int(n))


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


# -- element formats --------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().qpn_oracle_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().qpn_oracle_e4m3_value(int(code))


def ue4m3_value(byte: int):
    """Value of a UE4M3 scale byte, or None when the byte is not a valid scale."""
    out = ctypes.c_double()
    rc = lib().qpn_oracle_ue4m3_value(int(byte), ctypes.byref(out))
    return None if rc != 0 else out.value


def f16_value(bits: int) -> float:
    return lib().qpn_oracle_f16_value(int(bits) & 0xFFFF)


def f16_round(v: float) -> int:
    return int(lib().qpn_oracle_f16_round(float(v)))


def quant_e2m1(t) -> int:
    return lib().qpn_oracle_quant_e2m1(float(np.float32(t)))


def quant_e4m3(t) -> int:
    return lib().qpn_oracle_quant_e4m3(float(np.float32(t)))


# -- pack ---------------------------------------------------------------------

def nvfp4_tensor_scale(w):
    """(g, amax) for an fp32 weight tensor of any shape."""
    w = _c(w, np.float32)
    amax = ctypes.c_float()
    g = lib().qpn_oracle_nvfp4_tensor_scale(_p(w), w.size, ctypes.byref(amax))
    return np.float32(g), np.float32(amax.value)


def pack_nvfp4_rows(w_rows, g):
    """Canonical NVFP4 pack of rows [r, k] with tensor scale g.

    Returns (codes uint8 [r, k/2], scales uint8 [r, k/16])."""
    w = _c(w_rows, np.float32)
    r, k = w.shape
    codes = np.zeros((r, k // 2), np.uint8)
    scales = np.zeros((r, k // 16), np.uint8)
    rc = lib().qpn_oracle_pack_nvfp4_rows(_p(w), r, k, float(np.float32(g)), _p(codes), _p(scales))
    if rc != 0:
        raise ValueError("oracle NVFP4 pack rejected the shape")
    return codes, scales


def pack_nvfp4(w):
    """Whole-tensor NVFP4 pack: (codes, scales, g)."""
    g, _ = nvfp4_tensor_scale(w)
    codes, scales = pack_nvfp4_rows(w, g)
    return codes, scales, g


def pack_fp8(w):
    """FP8 pack: (codes uint8 [n, k], row_scale float32 [n])."""
    w = _c(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    rs = np.zeros((n,), np.float32)
    rc = lib().qpn_oracle_pack_fp8_rows(_p(w), n, k, _p(codes), _p(rs))
    if rc != 0:
        raise ValueError("oracle FP8 pack rejected the shape")
    return codes, rs


# -- dequant and GEMM ---------------------------------------------------------

def dequant_nvfp4(codes, scales, g):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    r, k2 = codes.shape
    k = k2 * 2
    out = np.zeros((r, k), np.float64)
    if lib().qpn_oracle_dequant_nvfp4(_p(codes), _p(scales), float(np.float32(g)), r, k, _p(out)):
        raise ValueError("invalid UE4M3 scale byte")
    return out


def dequant_fp8(codes, row_scale):
    codes = _c(codes, np.uint8)
    rs = _c(row_scale, np.float32)
    r, k = codes.shape
    out = np.zeros((r, k), np.float64)
    lib().qpn_oracle_dequant_fp8(_p(codes), _p(rs), r, k, _p(out))
    return out


def requant_fp8_to_nvfp4(codes, row_scale):
    """FP8 -> NVFP4 conversion of one weight (taozi.news page, section
    "v1.1 的关键改进": before FP8 regions had their own path they were turned
    into NVFP4, serving a derived checkpoint; aiwitness.kr page, section
    "내가 실제로 만든 것", same account).  The pages do not give the recipe;
    the plainest reading: decode each FP8 weight to its value E4M3(code) * s_r
    (exact in FP64, then one rounding to FP32, the precision the pack works
    in), and quantise that tensor with the NVFP4 recipe used for the FP4
    regions.  Codes must not be the NaN codes.  Returns (codes, scales, g)."""
    w = dequant_fp8(codes, row_scale)
    if not np.all(np.isfinite(w)):
        raise ValueError("FP8 NaN code in the weight")
    return pack_nvfp4(w.astype(np.float32))


def _x_bits(x):
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    return _c(x, np.uint16)


def gemm_f64(w_hat, x):
    """y[m, n] = x[m, :] . w_hat[n, :] in FP64, x given as float16."""
    w_hat = _c(w_hat, np.float64)
    xb = _x_bits(x)
    m, k = xb.shape
    n = w_hat.shape[0]
    y = np.zeros((m, n), np.float64)
    lib().qpn_oracle_gemm_f64(_p(w_hat), _p(xb), m, n, k, _p(y))
    return y


def gemm_nvfp4(codes, scales, g, x):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    xb = _x_bits(x)
    m, k = xb.shape
    n = codes.shape[0]
    y = np.zeros((m, n), np.float64)
    if lib().qpn_oracle_gemm_nvfp4(_p(codes), _p(scales), float(np.float32(g)), _p(xb), m, n, k,
                                   _p(y)):
        raise ValueError("invalid UE4M3 scale byte")
    return y


def gemm_fp8(codes, row_scale, x):
    codes = _c(codes, np.uint8)
    rs = _c(row_scale, np.float32)
    xb = _x_bits(x)
    m, k = xb.shape
    n = codes.shape[0]
    y = np.zeros((m, n), np.float64)
    lib().qpn_oracle_gemm_fp8(_p(codes), _p(rs), _p(xb), m, n, k, _p(y))
    return y


def round_f16(y):
    """FP64 array -> float16 array (bit-exact RNE, the oracle's own rounding)."""
    y = _c(y, np.float64)
    out = np.zeros(y.shape, np.uint16)
    lib().qpn_oracle_round_f16_array(_p(y), y.size, _p(out))
    return out.view(np.float16)


def argmax_f16(logits):
    """Lowest index of the row maximum of float16 logits [m, n]."""
    lb = _x_bits(logits)
    m, n = lb.shape
    out = np.zeros((m,), np.int32)
    lib().qpn_oracle_argmax_f16(_p(lb), m, n, _p(out))
    return out


def lmhead_nvfp4(codes, scales, g, x):
    """(y_ref FP64 [m, n], argmax int32 [m]) -- argmax of the FP16-rounded y."""
    y = gemm_nvfp4(codes, scales, g, x)
    return y, argmax_f16(round_f16(y))


def greedy_verify(argmax, draft):
    """Greedy speculative verification of one round (taozi.news page: section
    "自研 QPN 内核" maps a k = 7 verify round onto the M = 8 path; the opening
    comparison counts tokens committed per round; section
    "一些工程细节与长上下文发现" has the drafter propose by greedy / local
    argmax).  Row i of the verified block holds the target's greedy token for
    position i + 1, and draft[i] is the drafter's token for that position.
    The pages do not spell out the rule; the plainest reading is the greedy
    one: accept drafts while each equals the target's token, then commit the
    target's token at the first position not accepted.
    Returns (accepted, next_token): accepted = the length of the longest
    prefix of draft equal to argmax[:len(draft)], next_token =
    argmax[accepted]; the round commits accepted + 1 tokens."""
    argmax = [int(a) for a in argmax]
    draft = [int(d) for d in draft]
    if len(draft) != len(argmax) - 1:
        raise ValueError("a round verifies m - 1 drafts with m rows")
    accepted = 0
    for proposed, target in zip(draft, argmax):
        if proposed != target:
            break
        accepted += 1
    return accepted, argmax[accepted]

