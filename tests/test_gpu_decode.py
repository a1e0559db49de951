"""The GEMM's own register decode, exhaustively, against the oracle's decoders.

Bit-exact: every E2M1 code in every byte position under every valid UE4M3
scale, and every E4M3 byte in every position."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import dev, host, log, need_gpu

pytestmark = pytest.mark.gpu


def _f16_bits(v):
    return int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])


def test_nvfp4_decode_exhaustive():
    qpn = need_gpu()
    # fragment f: 16 code bytes and 2 scale bytes.  Cover all 256 byte values
    # in all 16 positions (rotate), with both scale slots running over all
    # valid UE4M3 bytes 0x00..0x7E.
    frags = []
    scales = []
    for s in range(0x7F):
        for rot in range(16):
            base = (np.arange(16) * 16 + rot * 17 + s) % 256
            frags.append(base.astype(np.uint8))
            scales.append([s, (0x7E - s)])
    codes16 = np.array(frags, np.uint8)
    sc2 = np.array(scales, np.uint8)
    log(f"nvfp4 decode: {codes16.shape[0]} fragments")
    out = host(qpn.debug_decode_nvfp4(dev(codes16), dev(sc2))).view(np.uint16)
    e2 = [oracle.e2m1_value(c) for c in range(16)]
    sv = [oracle.ue4m3_value(b) for b in range(0x7F)]
    exp = np.zeros_like(out)
    for f in range(codes16.shape[0]):
        for e in range(32):
            b = int(codes16[f, e // 2])
            c = (b & 0xF) if e % 2 == 0 else (b >> 4)
            S = sv[int(sc2[f, e // 16])]
            exp[f, e] = _f16_bits(e2[c] * S)  # exact: <= 6 significant bits
    bad = np.argwhere(out != exp)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:4]}"


def test_fp8_decode_exhaustive():
    qpn = need_gpu()
    codes16 = np.array([(np.arange(16) + 16 * r + rot) % 256 for r in range(16) for rot in range(16)],
                       np.uint8)
    out = host(qpn.debug_decode_fp8(dev(codes16))).view(np.uint16)
    for f in range(codes16.shape[0]):
        for e in range(16):
            c = int(codes16[f, e])
            v = oracle.e4m3_value(c)
            got = out[f, e]
            if math.isnan(v):
                assert np.isnan(np.array([got], np.uint16).view(np.float16)[0])
            else:
                assert got == _f16_bits(v), (hex(c), hex(got))
