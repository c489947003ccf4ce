"""Peak device memory, tiled vs naive (exercise 3 of the S12 chapter): the
library call needs no device memory beyond its inputs and output at any n
(neither torch's allocator nor the device's free memory, hipMemGetInfo, moves
during it), while evaluating S and P in full needs at least the n x n float32
score matrix, so its extra memory grows with n^2."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

pytestmark = pytest.mark.gpu


def test_peak_memory_scaling():
    import bench
    from tiled_online_softmax_04_amd import fa
    rows = bench.peak_memory(fa)
    for r in rows:
        print(r, flush=True)
        assert r["flash_extra_bytes"] == 0, "the tiled call must allocate nothing"
        assert r["flash_device_free_drop_bytes"] == 0, "device free memory fell during the call"
        assert r["naive_extra_bytes"] >= r["n2_float32_bytes"]
    # quadratic growth: 16x the extra memory per 4x in n (within allocator rounding)
    for a, b in zip(rows, rows[1:]):
        ratio = b["naive_extra_bytes"] / a["naive_extra_bytes"]
        assert 12.0 <= ratio <= 20.0, ratio
