"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and its host-side size queries and argument checks behave as
include/qpn.h documents.  No kernel is launched by any test here."""
import ctypes
import dataclasses
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qpn.h")


@pytest.fixture(scope="module")
def qpn():
    from fp8_quantized_skinny_qpn_amd import qpn as q
    return q


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"QPN_API\s+[\w\s\*]*?\b(qpn_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(qpn):
    names = _declared()
    assert len(names) == 24
    lib = ctypes.CDLL(qpn.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(qpn.EXPORTED) == names


def test_status_strings(qpn):
    for rc in range(7):
        s = qpn.status_string(rc)
        assert s.startswith("QPN_")
    assert "unknown" in qpn.status_string(99)
    assert qpn.lib.qpn_layout_version() == 2


def test_packed_sizes(qpn):
    # header 256 B + ceil(n/16) panels * ceil(k/128) k-steps * 1152 B
    assert qpn.nvfp4_packed_bytes(5120, 17408) == 256 + 320 * 136 * 1152
    assert qpn.nvfp4_packed_bytes(17408, 5120) == 256 + 1088 * 40 * 1152
    assert qpn.nvfp4_packed_bytes(151936, 5120) == 256 + 9496 * 40 * 1152
    # the algorithmic bytes of the format (codes + scales + g) fit exactly
    # when n % 16 == 0 and k % 128 == 0
    for n, k in [(2048, 2048), (5120, 17408), (17408, 5120), (151936, 5120)]:
        assert qpn.nvfp4_packed_bytes(n, k) - 256 == n * k // 2 + n * k // 16
    assert qpn.nvfp4_packed_bytes(17, 16) == 256 + 2 * 1 * 1152
    assert qpn.nvfp4_packed_bytes(0, 0) == 256
    assert qpn.nvfp4_packed_bytes(16, 8) == 0       # k % 16 != 0
    assert qpn.nvfp4_packed_bytes(-1, 16) == 0
    assert qpn.nvfp4_packed_bytes(1 << 25, 16) == 0  # n too large
    # FP8: header + 256-aligned row scales + ceil(n/16) * ceil(k/64) * 1024
    assert qpn.fp8_packed_bytes(6144, 5120) == 256 + 6144 * 4 + 384 * 80 * 1024
    assert qpn.fp8_packed_bytes(20, 8) == 256 + 256 + 2 * 1 * 1024
    assert qpn.fp8_packed_bytes(16, 12) == 0


def test_gemm_plan(qpn):
    # workgroups cover the 16-row panels once per K split; a pure function of the shape
    for op, m, n, k in [(1, 1, 17408, 5120), (1, 8, 17408, 5120), (1, 4, 5120, 17408),
                        (1, 8, 5120, 17408), (2, 2, 6144, 5120), (3, 8, 151936, 5120),
                        (1, 3, 17, 16), (2, 7, 24, 8), (1, 8, 64, 1 << 20)]:
        pl = qpn.gemm_plan(op, m, n, k)
        panels = -(-n // 16)
        ks = 128 if op != 2 else 64
        J = -(-k // ks)
        assert 1 <= pl.split_workgroups <= pl.workgroups
        assert pl.split_workgroups % pl.splits == 0
        groups = pl.split_workgroups // pl.splits
        whole = pl.workgroups - pl.split_workgroups
        # the split segment's groups and the whole-panel workgroups cover every
        # panel, at most panels_per_workgroup per workgroup
        assert (groups + whole) * pl.panels_per_workgroup >= panels
        assert 1 <= groups <= max(panels, 1)
        assert pl.waves_per_panel in (1, 2, 3, 4, 8) and pl.panels_per_workgroup >= 1
        assert 1 <= pl.waves_per_workgroup <= 16
        assert pl.prefetch_depth >= 1 and pl.splits >= 1
        assert pl.activation_rows in (1, 2, 4, 8) and pl.activation_rows >= m
        assert pl.activation_rows < 2 * m or m == 0
        # the activation slice a workgroup stages fits in LDS (whole-panel
        # workgroups stage all of K)
        steps = J if whole else -(-J // pl.splits)
        assert steps * ks * pl.activation_rows * 2 <= 160 * 1024
        assert pl == qpn.gemm_plan(op, m, n, k)
        ws = qpn.workspace_bytes(op, m, n, k)
        if op != 3:
            assert (ws == 0) == (pl.splits == 1)
        name = qpn.kernel_name(qpn.FMT_NVFP4 if op != 2 else qpn.FMT_FP8, m, n, k, lmhead=op == 3)
        assert name.startswith("qpn::skinny_gemm_kernel<") and name.endswith(", false>")
        assert pl.valu_dot == 0                               # automatic plans use the MFMA
        # plan 0 of the diagnostic query is the automatic choice
        assert qpn.gemm_plan(op, m, n, k, plan=0) == pl
        assert qpn.workspace_bytes(op, m, n, k, plan=0) == ws
    # 320 panels on 256 CUs: 256 whole panels plus the last 64 split four ways
    pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 1, 5120, 17408)
    assert (pl.workgroups, pl.split_workgroups, pl.splits) == (512, 256, 4)
    # the LDS budget splits 5120x17408 at M = 4 in two; twice that over
    # 64 groups of five panels still fits one workgroup per CU: 4 splits, 256
    pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 4, 5120, 17408)
    assert (pl.workgroups, pl.panels_per_workgroup, pl.splits) == (256, 5, 4)
    # 3072 panels: 615 five-panel (80% of 3 rounds) or 384 eight-panel
    # workgroups (75% of 2) fill their rounds poorly; 256 of 12 panels each
    for m in (2, 4, 8):
        pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, m, 49152, 5120)
        assert (pl.workgroups, pl.waves_per_panel, pl.panels_per_workgroup) == (256, 1, 16)
    # 2176 panels (436 five-panel workgroups, 85%) keep the five-panel plan
    pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 34816, 5120)
    assert (pl.workgroups, pl.panels_per_workgroup) == (436, 5)
    # FP8 at 3-8 rows over 384 panels and 80 k-steps (slice fits): two panels
    # per workgroup; at 1-2 rows one; with 1088 panels, or a slice that must
    # be split (5120x17408), five; 3072 panels, sixteen
    for m in (3, 4, 8):
        assert qpn.gemm_plan(qpn.OP_GEMM_FP8, m, 6144, 5120).panels_per_workgroup == 2
        assert qpn.gemm_plan(qpn.OP_GEMM_FP8, m, 17408, 5120).panels_per_workgroup == 5
        assert qpn.gemm_plan(qpn.OP_GEMM_FP8, m, 5120, 17408).panels_per_workgroup == 5
        assert qpn.gemm_plan(qpn.OP_GEMM_FP8, m, 49152, 5120).panels_per_workgroup == 16
    assert qpn.gemm_plan(qpn.OP_GEMM_FP8, 2, 6144, 5120).panels_per_workgroup == 1
    # NVFP4 at 1-2 rows over 768 or more panels: one panel per workgroup
    for m in (1, 2):
        assert qpn.gemm_plan(qpn.OP_GEMM_NVFP4, m, 17408, 5120).panels_per_workgroup == 1
        assert qpn.gemm_plan(qpn.OP_GEMM_NVFP4, m, 37984, 5120).panels_per_workgroup == 1
    # NVFP4 at 3-8 rows over fewer than 512 panels whose whole slice fits the
    # LDS budget: two panels per workgroup; 4352x8192 at 8 rows would need a
    # split slice and keeps five
    for n, k in ((5120, 5120), (7168, 5120), (5120, 4352)):
        for m in (4, 8):
            assert qpn.gemm_plan(qpn.OP_GEMM_NVFP4, m, n, k).panels_per_workgroup == 2
    assert qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 4352, 8192).panels_per_workgroup == 5
    # a short K splits the remainder panels only from a quarter round (64) on
    pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 1, 8704, 5120)          # 544 panels
    assert pl.workgroups == pl.split_workgroups == 544
    pl = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 1, 9216, 5120)          # 576 panels
    assert pl.workgroups > pl.split_workgroups
    # the VALU-dot diagnostic plans repeat plans 2 and 1 with the other contraction
    auto = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 17408, 5120)
    for vd, base in ((11, 2), (12, 1)):
        a = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 17408, 5120, plan=base)
        b = qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 17408, 5120, plan=vd)
        assert (a.valu_dot, b.valu_dot) == (0, 1)
        assert dataclasses.replace(a, valu_dot=1) == b
        assert qpn.kernel_name(qpn.FMT_NVFP4, 8, 17408, 5120, plan=vd).endswith("false, true>")
        assert qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, 8, 17408, 5120, plan=vd) == \
            qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, 8, 17408, 5120, plan=base)
    # asking about a forced plan changes nothing for later calls
    assert qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 17408, 5120) == auto
    # K = 2^20 at M = 8 cannot be staged whole: it is split
    assert qpn.gemm_plan(1, 8, 64, 1 << 20).splits > 1
    with pytest.raises(qpn.QpnError):
        qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 8, 16, 24)
    with pytest.raises(qpn.QpnError):
        qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 9, 16, 32)


def test_forced_plans_reject_unknown_ids(qpn):
    v = ctypes.c_void_p
    assert qpn.plan_ids() == list(range(1, 15))
    for bad in (10 ** 6, -1, 15):
        with pytest.raises(qpn.QpnError):
            qpn.gemm_plan(qpn.OP_GEMM_NVFP4, 1, 16, 16, plan=bad)
        # the run entry point checks the plan before anything else
        assert qpn.lib.qpn_debug_run_plan(qpn.OP_GEMM_NVFP4, bad, v(A256), v(A16), v(A16), None,
                                          1, 16, 16, None, 0, None) == 2
    # prefill ops have no forced plans; unknown ops are rejected
    with pytest.raises(qpn.QpnError):
        qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 32, 16, 16, plan=1)
    assert qpn.lib.qpn_debug_run_plan(qpn.OP_PREFILL_NVFP4, 1, v(A256), v(A16), v(A16), None,
                                      1, 16, 16, None, 0, None) == 2
    # argument checks of the entry point a forced plan runs
    assert qpn.lib.qpn_debug_run_plan(qpn.OP_GEMM_FP8, 3, v(0), v(A16), v(A16), None,
                                      1, 16, 16, None, 0, None) == 1
    assert qpn.lib.qpn_debug_run_plan(qpn.OP_LMHEAD_NVFP4, 13, v(A256), v(A16), v(A16), v(0),
                                      1, 16, 16, v(A16), 4096, None) == 1


def test_workspace_stays_below_2_31(qpn):
    """Split-K partials are addressed with 32-bit offsets: no plan asks for
    2^31 bytes or more, down to the documented maximum sizes."""
    big = ctypes.c_size_t(-1).value
    for op in (qpn.OP_GEMM_NVFP4, qpn.OP_GEMM_FP8, qpn.OP_LMHEAD_NVFP4, qpn.OP_PREFILL_NVFP4,
               qpn.OP_PREFILL_FP8):
        ms = (1, 2, 4, 8) if op <= 3 else (1, 8, 9, 16, 17, 64, 256)
        for m in ms:
            for n, k in [(1 << 24, 1 << 20), (524288, 524288), (1 << 24, 16), (48, 1 << 20),
                         (151936, 5120), (5120, 17408), (262144, 1 << 20)]:
                ws = qpn.workspace_bytes(op, m, n, k)
                assert ws == big or ws < (1 << 31), (op, m, n, k, ws)
                for plan in (qpn.plan_ids() if op <= 3 else ()):
                    try:
                        wsp = qpn.workspace_bytes(op, m, n, k, plan=plan)
                    except qpn.QpnError:   # that plan cannot run this shape at all
                        continue
                    assert wsp < (1 << 31), (op, m, n, k, plan, wsp)


def _tree_nodes(s):
    """Nodes of the pairwise tree that sums s split partials."""
    nodes, width = 0, s
    while width > 1:
        nodes += (width + 1) // 2
        width = (width + 1) // 2
    return nodes


def _split_ws(pl):
    """One 1 KiB exchange tile per panel per node of the split tree."""
    groups = pl.split_workgroups // pl.splits
    return 0 if pl.splits == 1 else _tree_nodes(pl.splits) * groups * pl.panels_per_workgroup * 1024


def test_split_tree_nodes():
    assert [_tree_nodes(s) for s in (1, 2, 3, 4, 5, 7, 8)] == [0, 1, 3, 3, 6, 7, 7]


def test_workspace_sizes(qpn):
    for op, m, n, k in [(1, 8, 5120, 17408), (1, 1, 5120, 17408), (2, 4, 5120, 5120), (1, 1, 2048, 2048),
                        (1, 8, 17408, 5120), (2, 8, 7168, 5120)]:
        assert qpn.workspace_bytes(op, m, n, k) == _split_ws(qpn.gemm_plan(op, m, n, k))
    assert qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, 1, 17408, 5120) == 0
    assert qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, 8, 5120, 17408) > 0   # K is split
    assert qpn.workspace_bytes(qpn.OP_LMHEAD_NVFP4, 8, 151936, 5120) == 8 * 8 * 256
    assert qpn.workspace_bytes(qpn.OP_LMHEAD_NVFP4, 1, 17, 16) == 8 * 256
    assert qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, 0, 16, 16) == 0
    big = ctypes.c_size_t(-1).value
    assert qpn.workspace_bytes(99, 1, 16, 16) == big
    assert qpn.workspace_bytes(qpn.OP_GEMM_NVFP4, 9, 16, 16) == big


# Argument checks.  Pointers are plain integers the library never dereferences
# because every call below fails a host-side check first.
A256 = 0x10000
A16 = 0x10010
ODD = 0x10001


def _gemm(qpn, fn, packed, x, y, m, n, k):
    return fn(ctypes.c_void_p(packed), ctypes.c_void_p(x), ctypes.c_void_p(y), m, n, k, None, 0,
              None)


@pytest.mark.parametrize("fname", ["qpn_gemm_nvfp4", "qpn_gemm_fp8"])
def test_gemm_argument_errors(qpn, fname):
    fn = getattr(qpn.lib, fname)
    assert _gemm(qpn, fn, 0, A16, A16, 1, 16, 16) == 1          # null packed
    assert _gemm(qpn, fn, A256, 0, A16, 1, 16, 16) == 1         # null x
    assert _gemm(qpn, fn, A256, A16, 0, 1, 16, 16) == 1         # null y
    assert _gemm(qpn, fn, A256, A16, A16, 9, 16, 16) == 2       # m > 8
    assert _gemm(qpn, fn, A256, A16, A16, -1, 16, 16) == 2
    assert _gemm(qpn, fn, A256, A16, A16, 1, 16, 12) == 2       # k not a multiple of 16 / 8
    assert _gemm(qpn, fn, A256, A16, A16, 1, -3, 16) == 2
    assert _gemm(qpn, fn, A256, A16, A16, 1, 1 << 25, 16) == 2
    assert _gemm(qpn, fn, A256, A16, A16, 1, 16, 1 << 21) == 2
    assert _gemm(qpn, fn, A16, A16, A16, 1, 16, 16) == 3        # packed not 256-aligned
    assert _gemm(qpn, fn, A256, A16 + 8, A16, 1, 16, 16) == 3   # x not 16-aligned
    assert _gemm(qpn, fn, A256, A16, ODD, 1, 16, 16) == 3       # y not 2-aligned
    # empty calls succeed without launching anything
    assert _gemm(qpn, fn, A256, A16, A16, 0, 16, 16) == 0
    assert _gemm(qpn, fn, A256, A16, A16, 3, 0, 16) == 0


def test_lmhead_argument_errors(qpn):
    L = qpn.lib
    v = ctypes.c_void_p

    def call(packed=A256, x=A16, lg=A16, am=A16, m=1, n=16, k=16, ws=A16, wsb=64):
        return L.qpn_lmhead_nvfp4(v(packed), v(x), v(lg), v(am), m, n, k, v(ws), wsb, None)

    assert call(am=0) == 1
    assert call(ws=0) == 1
    assert call(n=0) == 2
    assert call(am=A16 + 2) == 3
    assert call(ws=A16 + 4) == 3
    assert call(wsb=8 * 1 * 256 - 1) == 4                      # workspace too small
    assert call(m=8, n=160, wsb=8 * 8 * 256 - 8) == 4
    assert call(m=0) == 0


def test_lmhead_verify_argument_errors(qpn):
    L = qpn.lib
    v = ctypes.c_void_p

    def call(dr=A16, res=A16, m=2, n=16, k=16, am=A16, ws=A16, wsb=8 * 8 * 256):
        return L.qpn_lmhead_verify_nvfp4(v(A256), v(A16), v(A16), v(am), v(dr), v(res), m, n, k,
                                         v(ws), wsb, None)

    assert call(res=0) == 1                                   # result is required
    assert call(dr=0) == 1                                    # drafts are required for m >= 2
    assert call(res=A16 + 2) == 3
    assert call(dr=A16 + 1) == 3
    assert call(am=0) == 1                                    # the lm_head's own checks follow
    assert call(n=0) == 2
    assert call(wsb=8 * 2 * 256 - 1) == 4
    assert call(m=0, dr=0, res=0) == 0                        # nothing to do
    assert call(m=9) == 2


def test_requant_argument_errors(qpn):
    L = qpn.lib
    v = ctypes.c_void_p
    n8, n4 = qpn.fp8_packed_bytes(32, 64), qpn.nvfp4_packed_bytes(32, 64)
    far = A256 + (1 << 20)

    def call(src=A256, sb=n8, n=32, k=64, dst=far, db=n4):
        return L.qpn_requant_fp8_to_nvfp4(v(src), sb, n, k, v(dst), db, None)

    assert call(src=0) == 1
    assert call(dst=0) == 1
    assert call(k=40) == 2                                    # NVFP4 needs k % 16 == 0
    assert call(n=-1) == 2
    assert call(src=A256 + 16) == 3
    assert call(dst=far + 128) == 3
    assert call(sb=n8 - 1) == 4
    assert call(db=n4 - 1) == 4
    assert call(dst=A256 + 256) == 4                          # overlapping blobs


def test_prefill_queries(qpn):
    for op in (qpn.OP_PREFILL_NVFP4, qpn.OP_PREFILL_FP8):
        for m, n, k in [(9, 17408, 5120), (16, 5120, 17408), (17, 17408, 5120), (64, 5120, 17408),
                        (32, 5120, 17408), (64, 17408, 5120), (128, 5120, 17408), (128, 6144, 5120),
                        (128, 5120, 4096), (256, 17408, 5120), (256, 5120, 17408), (130, 200, 1024),
                        (1, 16, 64), (256, 6144, 5120), (256, 5120, 5120), (100, 40000, 1024),
                        (32, 6144, 5120), (40, 300, 9008), (40, 300, 20000), (64, 5120, 4096),
                        (16, 25600, 5120), (9, 20480, 17408), (12, 65536, 5120), (16, 16384, 1024),
                        (16, 24576, 512), (9, 1024, 8192), (8, 65536, 5120), (16, 34816, 5120),
                        (128, 34816, 5120), (256, 34816, 5120), (128, 151936, 5120), (32, 33000, 1024),
                        (100, 33000, 512), (200, 102400, 64), (128, 65536, 5120), (80, 16400, 1024),
                        (128, 16384, 1024), (100, 37984, 5120)]:
            pl = qpn.gemm_plan(op, m, n, k)
            ws = qpn.workspace_bytes(op, m, n, k)
            P = -(-n // 16)
            if op == qpn.OP_PREFILL_NVFP4:
                J = -(-k // 128)
                tiled = P >= 1536 or (P >= 1024 and J >= 64)
            else:
                J = -(-k // 64)
                tiled = J >= 128 or P >= 3072
            if m <= 8 or (m <= 16 and not tiled):
                # the skinny kernel (a 16-row tile above 8 rows): up to 8 rows,
                # and at 9-16 rows unless the call is large (many panels, or a
                # long K: with 1024 or more panels for NVFP4)
                assert pl.activation_rows in (1, 2, 4, 8, 16)
                assert m <= pl.activation_rows < 2 * max(m, 1)
                assert pl.split_workgroups % pl.splits == 0 and pl.split_workgroups <= pl.workgroups
                assert (ws == 0) == (pl.splits == 1)
                continue
            ks = 128 if op == qpn.OP_PREFILL_NVFP4 else 64
            J = -(-k // ks)
            # a workgroup's rows: 32, 64 or 128 (the fewest that hold m), at
            # most 128 per row block; 128 channels (narrow) or 256 (wide)
            rows = 32 if m <= 32 else 64 if m <= 64 else 128

            def launch(wide):
                chans = 256 if wide else 128
                tiles = -(-n // chans) * -(-m // rows)
                U = tiles * max(J, 1)

                def pieces_of(g):
                    owner = lambda u: ((u + 1) * g + U - 1) // U - 1
                    return max(owner(t * J + J - 1) - owner(t * J) + 1 for t in range(tiles)) if g != tiles else 1
                # stream-K: the (tile, k-step) units cut into equal contiguous
                # ranges, one per workgroup, at least 512 of K each, up to 256
                # workgroups; from 256 tiles on, whole tiles, unless their
                # rounds of 256 are less than 85% full: then one round of 256
                G = tiles if (J == 0 or tiles >= 256) else max(tiles, min(256, U // (512 // ks)))
                rounds = -(-tiles // 256)
                if J > 0 and tiles > 256 and tiles % 256 and U // 256 >= 512 // ks and tiles < 0.85 * 256 * rounds:
                    G = 256
                shares = False
                if J > 0 and tiles < 256:
                    # tiles summed in shares go through 1 KiB-per-contributor LDS
                    # stages: four per workgroup, shared by two of its eight
                    # wavefronts (four wavefronts for FP8 32-row tiles: one each)
                    waves = 4 if (op == qpn.OP_PREFILL_FP8 and not wide and rows == 32) else 8
                    stage_kib = (4 if op == qpn.OP_PREFILL_NVFP4 else 2) * rows // 16 // (waves // 4)
                    # whole pieces: a multiple of the tiles, each piece 1024 to 4096 of K
                    # (32-row tiles of 128 channels: at most three pieces)
                    c = min(256 // tiles, stage_kib if wide or rows > 32 else min(stage_kib, 3),
                            max(1, J * ks // 1024))
                    if c >= 2 and J * ks <= c * 4096:
                        G, shares = tiles * c, True
                    elif (wide or rows == 128) and pieces_of(G) > stage_kib:
                        G = max(tiles, tiles * (stage_kib - 1))
                return chans, tiles, G, pieces_of(G)
            wide = m > 128
            if op == qpn.OP_PREFILL_NVFP4 and m <= 64 and launch(True)[2] >= 128:
                wide = True   # up to 64 NVFP4 rows: 256 channels when that still fills half the CUs
            if 64 < m <= 128 and launch(False)[1] > 128 and launch(True)[2] >= 192:
                wide = True   # 65-128 rows: 256 channels with more than 128 narrow tiles, on 192+ workgroups
            chans, tiles, G, pieces = launch(wide)
            assert (pl.waves_per_panel, pl.panels_per_workgroup) == ((1, 16) if wide else (2, 8))
            assert pl.activation_rows == rows
            assert pl.workgroups == G == pl.split_workgroups
            assert pl.splits == pieces
            if G == tiles:
                assert ws == 0
            else:          # per cut tile 2 + pieces state words, then two FP32 partial tiles per workgroup
                cnt = -(-tiles * (2 + pieces) * 4 // 256) * 256
                assert ws == cnt + 2 * G * chans * pl.activation_rows * 4
        assert qpn.workspace_bytes(op, 0, 64, 64) == 0
        assert qpn.workspace_bytes(op, 257, 64, 64) == 2 ** 64 - 1
        with pytest.raises(qpn.QpnError):
            qpn.gemm_plan(op, 257, 64, 64)
    # 5120x17408 at 256 rows: 40 tiles, each cut into six whole pieces (one per workgroup)
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 256, 5120, 17408)
    assert (pl.workgroups, pl.splits) == (240, 6)
    # 17408x5120 at 32 rows: 68 tiles of 256 channels, three pieces each
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 32, 17408, 5120)
    assert (pl.workgroups, pl.splits, pl.panels_per_workgroup) == (204, 3, 16)
    # 5120x17408 at 32 rows: the wide tile would leave 80 workgroups, and four
    # whole pieces of 4352 K each are too long: equal ranges over 256 workgroups
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 32, 5120, 17408)
    assert (pl.workgroups, pl.panels_per_workgroup) == (256, 8)
    # FP8 7168x5120 at 32 rows: 56 tiles of 32 rows in three whole pieces
    pl = qpn.gemm_plan(qpn.OP_PREFILL_FP8, 32, 7168, 5120)
    assert (pl.workgroups, pl.splits) == (168, 3)
    # FP8 5120x5120 at 64 rows: 40 tiles in four whole pieces of 1280 K
    pl = qpn.gemm_plan(qpn.OP_PREFILL_FP8, 64, 5120, 5120)
    assert (pl.workgroups, pl.splits) == (160, 4)
    # more tiles than CUs: 34816x5120 at 256 rows (272 tiles) in one round of
    # 256 equal ranges; 151936x5120 at 256 rows (1188 tiles, rounds 93% full)
    # in whole tiles
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 256, 34816, 5120)
    assert (pl.workgroups, pl.splits) == (256, 2)
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 256, 151936, 5120)
    assert (pl.workgroups, pl.splits) == (1188, 1)
    # 65-128 rows with more than 128 narrow tiles: the 256-channel tile
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 128, 34816, 5120)
    assert (pl.panels_per_workgroup, pl.workgroups, pl.splits) == (16, 256, 3)
    assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 128, 17408, 5120).panels_per_workgroup == 16
    assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 128, 5120, 17408).panels_per_workgroup == 8
    assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 128, 16400, 1024).panels_per_workgroup == 8  # 130 wide workgroups
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 128, 151936, 5120)
    assert (pl.panels_per_workgroup, pl.workgroups, pl.splits) == (16, 256, 2)
    pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, 128, 65536, 5120)
    assert (pl.panels_per_workgroup, pl.workgroups, pl.splits) == (16, 256, 1)
    # 9-16 rows: the skinny kernel on the decoder shapes, the tiled one on
    # large calls
    for m in (9, 16):
        assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, m, 17408, 5120).activation_rows == 16
        assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, m, 5120, 17408).activation_rows == 16
        pl = qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, m, 25600, 5120)
        assert (pl.activation_rows, pl.panels_per_workgroup) == (32, 16)
        assert qpn.gemm_plan(qpn.OP_PREFILL_NVFP4, m, 20480, 17408).activation_rows == 32
        assert qpn.gemm_plan(qpn.OP_PREFILL_FP8, m, 5120, 17408).activation_rows == 32
        assert qpn.gemm_plan(qpn.OP_PREFILL_FP8, m, 65536, 5120).activation_rows == 32
        # FP8 on the skinny kernel: two panels per workgroup below 512
        # panels, five from 512
        pl = qpn.gemm_plan(qpn.OP_PREFILL_FP8, m, 6144, 5120)
        assert (pl.activation_rows, pl.panels_per_workgroup) == (16, 2)
        pl = qpn.gemm_plan(qpn.OP_PREFILL_FP8, m, 34816, 5120)
        assert (pl.activation_rows, pl.panels_per_workgroup) == (16, 5)


def test_prefill_argument_errors(qpn):
    L = qpn.lib
    v = ctypes.c_void_p
    for fn in (L.qpn_gemm_prefill_nvfp4, L.qpn_gemm_prefill_fp8):
        def call(packed=A256, x=A16, y=A16, m=16, n=32, k=64, ws=0, wsb=0):
            return fn(v(packed), v(x), v(y), m, n, k, v(ws), wsb, None)
        assert call(m=257) == 2
        assert call(m=-1) == 2
        assert call(k=12) == 2
        assert call(packed=0) == 1
        assert call(y=0) == 1
        assert call(x=A16 + 8) == 3
        assert call(packed=A256 + 16) == 3
        assert call(y=A16 + 1) == 3
        assert call(ws=A16 + 4, wsb=1024) == 3
        assert call(m=0) == 0 and call(n=0) == 0


def test_pack_argument_errors(qpn):
    L = qpn.lib
    v = ctypes.c_void_p
    need = qpn.nvfp4_packed_bytes(32, 64)
    assert L.qpn_pack_nvfp4(v(A16), 32, 64, v(0), need, None) == 1
    assert L.qpn_pack_nvfp4(v(0), 32, 64, v(A256), need, None) == 1
    assert L.qpn_pack_nvfp4(v(A16), 32, 40, v(A256), need, None) == 2
    assert L.qpn_pack_nvfp4(v(A16 + 4), 32, 64, v(A256), need, None) == 3
    assert L.qpn_pack_nvfp4(v(A16), 32, 64, v(A256 + 128), need, None) == 3
    assert L.qpn_pack_nvfp4(v(A16), 32, 64, v(A256), need - 1, None) == 4
    need8 = qpn.fp8_packed_bytes(32, 64)
    assert L.qpn_pack_fp8(v(A16), 32, 64, v(A256), need8 - 1, None) == 4
    assert L.qpn_pack_fp8(v(A16), 32, 60, v(A256), need8, None) == 2


def test_debug_argument_errors(qpn):
    L = qpn.lib
    v = ctypes.c_void_p
    assert L.qpn_debug_decode_nvfp4(v(0), v(A16), 4, v(A16), None) == 1
    assert L.qpn_debug_decode_nvfp4(v(A16), v(A16), -1, v(A16), None) == 2
    assert L.qpn_debug_decode_fp8(v(A16), 0, v(A16), None) == 0
    assert L.qpn_debug_unpack_nvfp4(v(A256), 16, 24, v(A16), v(A16), v(A16), None) == 2
    assert L.qpn_debug_unpack_fp8(v(A16), 16, 16, v(A16), v(A16), None) == 3
    assert L.qpn_debug_read_ceiling(v(A16), 24, v(A16), None) == 2
    assert L.qpn_debug_read_ceiling(v(A16 + 4), 32, v(A16), None) == 3
    assert L.qpn_debug_decode_fp8(v(A16), 4, v(A16 + 2), None) == 3


def test_valid_call_without_gpu_reports_device_error(qpn):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    fn = qpn.lib.qpn_gemm_nvfp4
    assert _gemm(qpn, fn, A256, A16, A16, 1, 16, 16) == 5
