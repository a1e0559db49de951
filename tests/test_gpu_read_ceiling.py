"""The read-ceiling diagnostic reads every 16-byte unit of its buffer.

The kernel folds each thread's loads with XOR and writes the sink only when a
thread's fold equals 0x9E3779B9.  A buffer of zeros with one unit whose four
words fold to that value therefore sets the sink exactly when the unit was
read; placing it first, last and in the middle of ragged sizes (partial last
pass of the grid, sizes above one grid window, and above the 2^24 units up to
which the grid is capped) checks that no unit is skipped.
"""
import numpy as np
import pytest
import torch

from gpu_util import log, need_gpu

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("units", [1, 7, 2048, 2049, 1 << 21, (1 << 21) + 13, 5 * (1 << 20) + 3,
                                   (1 << 24) + 5])
def test_every_unit_is_read(units):
    qpn = need_gpu()
    buf = torch.zeros(units * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for pos in sorted({0, units // 2, units - 1}):
        log(f"read ceiling: {units} units, marked unit {pos}")
        buf.zero_()
        sink.zero_()
        qpn.debug_read_ceiling(buf, sink)
        torch.cuda.synchronize()
        assert int(sink[0].item()) == 0, "a zero buffer must leave the sink untouched"
        word = np.array([MAGIC], dtype=np.uint32).view(np.int32)[0]
        buf[4 * pos] = int(word)
        qpn.debug_read_ceiling(buf, sink)
        torch.cuda.synchronize()
        assert int(sink[0].item()) == int(word), f"unit {pos} of {units} was not read"
