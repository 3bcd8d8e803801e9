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
    sep = rs.step_order("step_64k", separate_pack=True)
    assert sep[:5] == ["amax_w", "quantize_w", "amax_x", "quantize_x", "gemm_fwd"]
    assert sep[5:] == rs.QKV_ORDER[3:]
    assert rs.QKV_ORDER_UNFUSED == rs.QKV_ORDER[:3] + ["norm_rope_fwd"] + rs.QKV_ORDER[3:]
    msep = rs.step_order("mlp_64k", separate_pack=True)
    assert msep[:7] == rs.MLP_PACK_SEPARATE + ["mlp_gemm_up"] and msep[6:] == rs.MLP_ORDER[2:]
    assert rs.step_order("block_64k", separate_pack=True) == sep + msep
    names = open("include/fpr.h").read()
    for stage in set(rs.QKV_ORDER + sep + rs.MLP_ORDER + msep):
        assert stage in names, stage
        assert stage in bench.STAGE_SOURCES, stage


def test_mfma_rows_count_flop_and_fit_the_clock(tmp_path):
    """Three counters per dispatch with timestamps; the GEMM stages carry
    exactly 2MNK / 131072 instructions and the active cycles follow a 2.0 GHz
    clock plus a fixed window, which the fit must recover."""
    order = rs.step_order("step_64k")
    flop = rs.gemm_flop("step_64k")
    xcc, simds = 8, 1024
    f = tmp_path / "c.csv"
    with open(f, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        d, t0 = 0, 10**9
        for step in range(2):
            for k, stage in enumerate(order):
                ns = 1000 * (k + 3) + 7 * step
                inst = flop[stage] // rs.MFMA_FLOP if stage in flop else 0
                vals = {"SQ_INSTS_VALU_MFMA_F8": inst, "SQ_VALU_MFMA_BUSY_CYCLES": 64 * inst,
                        "GRBM_GUI_ACTIVE": xcc * (20000 + 2.0 * ns)}
                for c, v in vals.items():
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": _kernel_name(stage),
                                "Counter_Name": c, "Counter_Value": v,
                                "Start_Timestamp": t0, "End_Timestamp": t0 + ns})
                d, t0 = d + 1, t0 + ns + 500
    rows, clock = rs.mfma_rows(str(f), xcc, simds, "step_64k")
    assert clock == pytest.approx(2.0)
    assert set(rows) == {"gemm_fwd", "gemm_dx", "gemm_dw"}
    for s, r in rows.items():
        assert r["flop_ratio"] == pytest.approx(1.0) and r["busy_per_inst"] == 64
        assert r["launches"] == 2
        k = order.index(s)
        t = 1000 * (k + 3) + 3.5
        assert r["busy_frac"] == pytest.approx(64 * r["inst"] / (simds * 2.0 * t))
        assert r["util"] == pytest.approx(64 * r["inst"] / ((20000 + 2.0 * t) * simds))


def test_stats_carries_the_live_average_of_the_same_run(tmp_path):
    f = tmp_path / "stats.csv"
    with open(f, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs",
                                           "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void fpr::gemm_bf16out_kernel<x>(args)", "Calls": 3,
                    "AverageNs": 97000, "MinNs": 96000, "MaxNs": 99000, "Percentage": 17.0})
    log = tmp_path / "bench.log"
    log.write_text('rocprofv3 noise\n{"ms_per_step": 0.59, "roofline": {"kernel": "gemm_fwd", '
                   '"avg_us": 96.9, "launches": 30, "achieved": 1995.0, "unit": "TFLOP/s", '
                   '"frac": 0.399, "peak": 5000.0}}\nmore noise\n')
    out = rs.stats(str(f), "t", "cmd", str(log))
    assert "| `fpr::gemm_bf16out_kernel<x>` | 3 | 97.00 |" in out
    assert "`gemm_fwd` 96.9 µs average over 30 launches" in out and "0.399 of 5000.0" in out
    log.write_text("no json here\n")
    with pytest.raises(SystemExit, match="no bench.py JSON"):
        rs.stats(str(f), "t", "cmd", str(log))


def test_counter_lines_are_keyed_to_kernel_code_not_comments(tmp_path, monkeypatch):
    """A stage's counter line stays valid across comment edits of its kernel
    source and is dropped once a line of code changes."""
    src = tmp_path / "fp8_packed_reduced_amd" / "csrc"
    src.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    f = src / bench.STAGE_SOURCES["gemm_fwd"]
    f.write_text("// a kernel\nint f(int x) { return x + 1; }  /* done */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash("gemm_fwd")
    (tmp_path / "profiles" / "traffic_w.txt").write_text(
        "# header\n" f"gemm_fwd 1000 24 {h}\n")
    assert bench.read_traffic("w", "gemm_fwd") == 1024
    f.write_text("/* the kernel,\n   reworded */\nint f(int x) {\n  return x + 1;\n}\n")
    assert bench.source_hash("gemm_fwd") == h
    assert bench.read_traffic("w", "gemm_fwd") == 1024
    f.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash("gemm_fwd") != h
    assert bench.read_traffic("w", "gemm_fwd") is None


def test_two_pass_backward_work_accounting():
    """With two backward passes the norm/RoPE stage reads the forward's rows
    and writes nothing, and the gradient-code stage reads them again with dv
    and writes the codes; every other stage keeps its work."""
    w = dict(n_seq=1, seq_len=65536, d_model=768, n_heads=6, d_qk=96, d_v=128)
    T, H, dqk, dv = 65536, 6, 96, 128
    N, qk = H * (2 * dqk + dv), 2 * H * dqk
    one, two = bench.stage_work(w, 5), bench.stage_work(w, 5, two_pass=True)
    rows = 2 * T * qk * 2 + 4 * T * 2 * H
    assert one["norm_rope_bwd"] == ("hbm", rows + 2 * T * qk)
    assert two["norm_rope_bwd"] == ("hbm", rows)
    assert two["quantize_g"] == ("hbm", rows + 2 * T * H * dv + T * N)
    assert {k: v for k, v in one.items() if k not in ("norm_rope_bwd", "quantize_g")} == \
        {k: v for k, v in two.items() if k not in ("norm_rope_bwd", "quantize_g")}


def test_combined_pack_forward_work_accounting():
    """qkv_pack_forward's two launches carry exactly the work of the four
    separate quantiser launches: W's and x's amax, then both quantisers;
    mlp_pack_forward's that of its six (two per weight, two for x)."""
    w = dict(n_seq=1, seq_len=65536, d_model=768, n_heads=6, d_qk=96, d_v=128)
    work = bench.stage_work(w, 5)
    assert work["amax_wx"] == ("hbm", work["amax_w"][1] + work["amax_x"][1])
    assert work["quantize_wx"] == ("hbm", work["quantize_w"][1] + work["quantize_x"][1])
    m = bench.mlp_stage_work(dict(n_seq=1, seq_len=65536, d_model=768, d_ff=3072), (7, 7))
    assert m["mlp_amax_wx"] == ("hbm", 2 * m["mlp_amax_w"][1] + m["mlp_amax_x"][1])
    assert m["mlp_quantize_wx"] == ("hbm", 2 * m["mlp_quantize_w"][1] + m["mlp_quantize_x"][1])


def test_stage_times_split_a_trace_by_launch_order(tmp_path):
    """Per-stage means from a kernel trace: torch's and the probes' launches
    are skipped, stages that launch twice per step average both, and a
    forward-only trace follows the forward's order."""
    def write(order, steps):
        f = tmp_path / "run_kernel_trace.csv"
        with open(f, "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            t = 1000
            w.writerow({"Kernel_Name": "void fpr::probe_copy_kernel(args)",
                        "Start_Timestamp": t, "End_Timestamp": t + 5000})
            for step in range(steps):
                for k, stage in enumerate(order):
                    t += 10000
                    w.writerow({"Kernel_Name": _kernel_name(stage), "Start_Timestamp": t,
                                "End_Timestamp": t + 1000 * (k + 1) + 100 * step})
            w.writerow({"Kernel_Name": "at::native::fill(args)", "Start_Timestamp": t + 20000,
                        "End_Timestamp": t + 90000})
        return str(f)

    order = rs.step_order("mlp_64k", separate_pack=True)
    got = rs.stage_times(write(order, 2), "mlp_64k", separate_pack=True)
    assert got["mlp_gemm_up"] == (2, pytest.approx(order.index("mlp_gemm_up") + 1.05))
    k1, k2 = 1, 3  # mlp_quantize_w launches once per weight
    assert order[k1] == order[k2] == "mlp_quantize_w"
    assert got["mlp_quantize_w"] == (4, pytest.approx((k1 + 1 + k2 + 1) / 2 + 0.05))
    fwd = rs.step_order("fwd_16k", forward_only=True)
    assert fwd == ["amax_wx", "quantize_wx", "gemm_fwd"]
    got = rs.stage_times(write(fwd, 3), "fwd_16k", forward_only=True)
    assert got["gemm_fwd"] == (3, pytest.approx(3.1))
