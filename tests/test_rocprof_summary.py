"""The profile summariser that turns rocprofv3 CSVs into the committed
per-stage traffic lines: calibration against the encoder launches, stage
attribution by launch order, and the checks that refuse a trace that is not
made of whole steps.  Synthetic CSVs; no GPU."""
import csv

import pytest

import bench
from fp8_packed_reduced_amd import rocprof_summary as rs


def _write_csv(path, rows, counter):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


def _kernel_name(stage):
    return f"void fpr::{rs.KERNEL_OF_STAGE[stage]}<x>(args)"


def test_traffic_lines_scale_by_the_calibration_and_average_per_stage(tmp_path):
    order = rs.step_order("step_64k")
    calib_kib = bench.CALIB_FLOATS * 4 / 1024 / 2.0    # a counter reading half the bytes
    rows = [("void fpr::encode_kernel<false>(args)", calib_kib)] * 3
    for step in range(2):
        for k, stage in enumerate(order):
            rows.append((_kernel_name(stage), 100.0 * (k + 1) + step))
    f = tmp_path / "fetch.csv"
    _write_csv(f, rows, "FETCH_SIZE")
    got, factor = rs._per_stage(str(f), "FETCH_SIZE", 4.0 * bench.CALIB_FLOATS, order)
    assert factor == pytest.approx(2.0)
    for k, stage in enumerate(order):
        assert got[stage] == pytest.approx((100.0 * (k + 1) + 0.5) * 1024 * 2.0)


def test_a_trace_of_partial_steps_or_wrong_kernels_is_refused(tmp_path):
    order = rs.step_order("step_64k")
    calib = [("void fpr::encode_kernel<false>(args)", 1.0)]
    f = tmp_path / "a.csv"
    _write_csv(f, calib + [(_kernel_name(s), 1.0) for s in order[:-1]], "WRITE_SIZE")
    with pytest.raises(SystemExit, match="whole"):
        rs._per_stage(str(f), "WRITE_SIZE", 1.0, order)
    swapped = [_kernel_name(s) for s in order]
    swapped[4], swapped[5] = swapped[5], swapped[4]     # GEMM and norm/RoPE exchanged
    _write_csv(f, calib + [(n, 1.0) for n in swapped], "WRITE_SIZE")
    with pytest.raises(SystemExit, match="expected"):
        rs._per_stage(str(f), "WRITE_SIZE", 1.0, order)


def test_step_orders_match_the_library_stage_names():
    assert rs.step_order("step_64k") == rs.QKV_ORDER
    assert rs.step_order("mlp_64k") == rs.MLP_ORDER
    assert rs.step_order("block_64k") == rs.QKV_ORDER + rs.MLP_ORDER
    names = open("include/fpr.h").read()
    for stage in set(rs.QKV_ORDER + rs.MLP_ORDER):
        assert stage in names, stage
        assert stage in bench.STAGE_SOURCES, stage
