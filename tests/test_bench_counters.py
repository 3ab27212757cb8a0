"""The bench's reading of rocprofv3 counter files (CPU only): the roofline's
HBM traffic is the median over dispatches of FETCH_SIZE / WRITE_SIZE summed
per dispatch, with tiny dispatches of a same-named kernel left out."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import bench  # noqa: E402

HEADER = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"


def write(tmp_path, rows, name="p_counter_collection.csv"):
    p = tmp_path / name
    p.write_text(HEADER + "".join("%s,%s,%s,%s\n" % r for r in rows))
    return str(p)


def test_sums_per_dispatch_and_takes_the_median(tmp_path):
    k = '"void fp4q::gemm_fp4_persistent_kernel<1, 0, 0>(int, int)"'
    rows = []
    for d, (a, b) in enumerate([(10.0, 5.0), (10.0, 6.0), (10.0, 9.0)]):  # two rows each
        rows += [(d, k, "FETCH_SIZE", a), (d, k, "FETCH_SIZE", b)]
    rows.append((9, k, "WRITE_SIZE", 1000.0))          # another counter
    rows.append((10, '"other_kernel"', "FETCH_SIZE", 1000.0))  # another kernel
    f = write(tmp_path, rows)
    assert bench.counter_median([f], "gemm_fp4_persistent_kernel<1, 0, 0>", "FETCH_SIZE",
                                1.0) == 16.0


def test_small_dispatches_dropped_and_too_few_is_none(tmp_path):
    rows = [(0, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 4.0)]
    rows += [(d, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 131083.5) for d in range(1, 6)]
    f = write(tmp_path, rows)
    assert bench.counter_median([f], "copyBuffer", "FETCH_SIZE", 1024.0) == 131083.5
    g = write(tmp_path, rows[:3], "q.csv")
    assert bench.counter_median([g], "copyBuffer", "FETCH_SIZE", 1024.0) is None
    assert bench.counter_median([], "copyBuffer", "FETCH_SIZE", 1024.0) is None
