"""Turn rocprofv3 output of ``bench.py`` into the short text summaries kept
under ``profiles/``.

    python -m fp8_packed_reduced_amd.rocprof_summary stats KERNEL_STATS_CSV TITLE CMD [BENCH_OUT [WORKLOAD]]
        -> markdown table of per-kernel durations (``--kernel-trace --stats``);
           with BENCH_OUT (what the profiled bench.py printed), also the
           roofline kernel's HIP-event average that bench.py measured live in
           the same run; with WORKLOAD, also every stage's mean duration from
           the kernel trace beside the statistics (run_kernel_trace.csv), the
           launches attributed to stages by launch order

    python -m fp8_packed_reduced_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV WORKLOAD CMD...
        -> per-launch HBM bytes of every stage of the step, from two ``--pmc``
           runs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch)

    python -m fp8_packed_reduced_amd.rocprof_summary mfma COUNTER_CSV AGENT_CSV WORKLOAD CMD...
        -> matrix-core use of every GEMM stage, from one ``--pmc`` run of
           SQ_INSTS_VALU_MFMA_F8, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE

Byte counters are calibrated against the encoder launches bench.py makes
before its first step (known traffic: 4 bytes read and 1 byte written per
element): factor = known bytes / counter reading, per counter.  A stage's
line carries the hash of its kernel source, and bench.py ignores the line
once that source has changed.
"""
from __future__ import annotations

import csv
import statistics
import sys

# Launch order of one step of each part (a stage may launch more than once).
# The QKV step packs the weights and runs the forward in one qkv_pack_forward
# call (two shared quantiser launches), or, with bench.py --pack-forward
# separate, in pack_quantize_weights and qkv_forward (four launches); the
# MLP step likewise in mlp_pack_forward (two) or in its two calls (six).  Head
# widths 64, 96 and 128 run the norm/RoPE inside the forward GEMM
# (gemm_qkv_fwd_kernel); other widths launch norm_rope_fwd after it.
QKV_PACK_COMBINED = ["amax_wx", "quantize_wx"]
QKV_PACK_SEPARATE = ["amax_w", "quantize_w", "amax_x", "quantize_x"]
QKV_BWD = ["amax_dv", "norm_rope_bwd", "quantize_g", "gemm_dx", "gemm_dw", "dw_reduce"]
QKV_ORDER = QKV_PACK_COMBINED + ["gemm_fwd"] + QKV_BWD
QKV_ORDER_UNFUSED = QKV_PACK_COMBINED + ["gemm_fwd", "norm_rope_fwd"] + QKV_BWD
FUSED_WIDTHS = (64, 96, 128)
SEPARATE_FLAG = "--pack-forward separate"
MLP_PACK_COMBINED = ["mlp_amax_wx", "mlp_quantize_wx"]
MLP_PACK_SEPARATE = ["mlp_amax_w", "mlp_quantize_w", "mlp_amax_w", "mlp_quantize_w",
                     "mlp_amax_x", "mlp_quantize_x"]
MLP_REST = ["mlp_gemm_up", "mlp_quantize_h", "mlp_gemm_down", "mlp_amax_dy",
            "mlp_quantize_dy", "mlp_gemm_dh", "mlp_quantize_dpre", "mlp_gemm_dx",
            "mlp_gemm_dw1", "mlp_dw1_reduce", "mlp_gemm_dw2", "mlp_dw2_reduce"]
MLP_ORDER = MLP_PACK_COMBINED + MLP_REST
KERNEL_OF_STAGE = {
    "amax_w": "amax_w_kernel", "quantize_w": "quantize_w_kernel",
    "amax_x": "amax_bf16_kernel", "quantize_x": "quantize_act_kernel",
    "amax_wx": "amax_wx_kernel", "quantize_wx": "quantize_wx_kernel",
    "gemm_fwd": "gemm_", "norm_rope_fwd": "norm_rope_fwd",
    "norm_rope_bwd": "norm_rope_bwd", "amax_dv": "amax_bf16_kernel",
    "quantize_g": "quantize_act_kernel",
    "gemm_dx": "gemm_bf16out_kernel", "gemm_dw": "gemm_dw_part_kernel",
    "dw_reduce": "dw_reduce_kernel",
    "mlp_amax_w": "amax_w_kernel", "mlp_quantize_w": "quantize_w_kernel",
    "mlp_amax_x": "amax_bf16_kernel", "mlp_quantize_x": "quantize_act_kernel",
    "mlp_amax_wx": "amax_wx_kernel", "mlp_quantize_wx": "quantize_wx_kernel",
    "mlp_gemm_up": "EpiRelu2", "mlp_quantize_h": "quantize_act_kernel",
    "mlp_gemm_down": "EpiDx", "mlp_amax_dy": "amax_bf16_kernel",
    "mlp_quantize_dy": "quantize_act_kernel", "mlp_gemm_dh": "EpiDpre",
    "mlp_quantize_dpre": "quantize_act_kernel", "mlp_gemm_dx": "EpiDx",
    "mlp_gemm_dw1": "gemm_dw_part_kernel", "mlp_dw1_reduce": "dw_reduce_kernel",
    "mlp_gemm_dw2": "gemm_dw_part_kernel", "mlp_dw2_reduce": "dw_reduce_kernel",
}


def step_order(workload: str, separate_pack: bool = False,
               forward_only: bool = False) -> list[str]:
    import bench
    from fp8_packed_reduced_amd import inputs
    qkv, mlp = bench.BENCH_WORKLOADS.get(workload, (workload, None))
    order = []
    if qkv:
        fused = inputs.WORKLOADS[qkv]["d_qk"] in FUSED_WIDTHS
        order += QKV_ORDER if fused else QKV_ORDER_UNFUSED
        if separate_pack:
            order = QKV_PACK_SEPARATE + order[len(QKV_PACK_COMBINED):]
        if forward_only:  # bench.py --forward-only: pack and forward
            order = order[:order.index("amax_dv")]
    if mlp:
        order += (MLP_PACK_SEPARATE if separate_pack else MLP_PACK_COMBINED) + MLP_REST
    return order
CALIB_KERNEL = "encode_kernel"


def short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def _bench_line(path: str) -> dict:
    """The JSON line bench.py printed (its last line starting with '{')."""
    import json
    lines = [ln for ln in open(path) if ln.startswith("{")]
    if not lines:
        raise SystemExit(f"{path}: no bench.py JSON line")
    return json.loads(lines[-1])


def stage_times(trace_csv: str, workload: str, separate_pack: bool = False,
                forward_only: bool = False) -> dict:
    """Stage -> (launches, mean µs) from a kernel trace of whole steps."""
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ds = [(i, short(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
          for i, r in enumerate(rows)]
    per = _by_stage(trace_csv, ds, step_order(workload, separate_pack, forward_only))
    return {s: (len(v), statistics.mean(us for _, us in v)) for s, v in per.items()}


def stats(path: str, title: str, cmd: str, bench_out: str | None = None,
          workload: str | None = None) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}\n", "Command (run from /tmp with TMPDIR=/tmp, repository at $R):\n",
           "```\n" + cmd + "\n```\n",
           "| kernel | calls | avg µs | min µs | max µs | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    if workload:
        import os
        trace = os.path.join(os.path.dirname(path), "run_kernel_trace.csv")
        out += ["\nPer stage, from the kernel trace of the same run (launches attributed by "
                "launch order):\n", "| stage | launches | avg µs |", "|---|---:|---:|"]
        for st, (n, us) in stage_times(trace, workload, SEPARATE_FLAG in cmd,
                                       "--forward-only" in cmd).items():
            out.append(f"| `{st}` | {n} | {us:.2f} |")
    if bench_out:
        b = _bench_line(bench_out)
        rf = b["roofline"]
        out.append(f"\nbench.py in the same run: {b['ms_per_step']} ms per step; roofline kernel "
                   f"`{rf['kernel']}` {rf['avg_us']} µs average over {rf['launches']} launches "
                   f"(HIP events on its stream), {rf['achieved']} {rf['unit']} = "
                   f"{rf['frac']} of {rf['peak']}.")
    return "\n".join(out) + "\n"


def _dispatches(path: str, counter: str):
    """(dispatch id, kernel name, value) in dispatch order."""
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(int(r["Dispatch_Id"]), short(r["Kernel_Name"]), float(r["Counter_Value"]))
            for r in rows]


def _by_stage(path: str, ds, order: list[str]):
    """Stage -> [(dispatch id, value)] of the step launches (calibration,
    ceiling probes and torch's own launches left out), refusing anything but
    whole steps in the library's launch order."""
    step_kernels = [(d, n, v) for d, n, v in ds
                    if "fpr::" in n and CALIB_KERNEL not in n and "probe_" not in n]
    if len(step_kernels) % len(order):
        raise SystemExit(f"{path}: {len(step_kernels)} library dispatches is not a whole "
                         f"number of {len(order)}-kernel steps")
    per = {s: [] for s in order}
    for i, (d, n, v) in enumerate(step_kernels):
        stage = order[i % len(order)]
        if KERNEL_OF_STAGE[stage] not in n:
            raise SystemExit(f"{path}: dispatch {i} is {n}, expected {stage}")
        per[stage].append((d, v))
    return per


def _per_stage(path: str, counter: str, known_bytes: float, order: list[str]):
    ds = _dispatches(path, counter)
    calib = [v for _, n, v in ds if CALIB_KERNEL in n]
    if not calib:
        raise SystemExit(f"{path}: no calibration launch ({CALIB_KERNEL}) found")
    factor = known_bytes / (statistics.median(calib) * 1024.0)
    per = _by_stage(path, ds, order)
    return {s: statistics.mean(v * 1024.0 * factor for _, v in dv)
            for s, dv in per.items()}, factor


def traffic(fetch_csv: str, write_csv: str, workload: str, cmd: str) -> str:
    sys.path.insert(0, ".")
    import bench  # the stage -> source mapping and the calibration size
    n = bench.CALIB_FLOATS
    order = step_order(workload, SEPARATE_FLAG in cmd)
    fetch, ff = _per_stage(fetch_csv, "FETCH_SIZE", 4.0 * n, order)
    write, wf = _per_stage(write_csv, "WRITE_SIZE", 1.0 * n, order)
    out = [f"# HBM traffic per launch, {workload}: stage fetch_bytes write_bytes source_sha12",
           f"# from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of: {cmd}",
           f"# calibration (encoder, {4 * n} B read / {n} B written): fetch x{ff:.4f}, "
           f"write x{wf:.4f}"]
    for s in dict.fromkeys(order):
        out.append(f"{s} {fetch[s]:.0f} {write[s]:.0f} {bench.source_hash(s)}")
    return "\n".join(out) + "\n"


# FLOP of one v_mfma_scale_f32_32x32x64_f8f6f4 (every GEMM here uses only it)
MFMA_FLOP = 2 * 32 * 32 * 64


def gemm_flop(workload: str) -> dict:
    """Algorithmic 2*M*N*K of each GEMM stage of the workload."""
    import bench
    from fp8_packed_reduced_amd import inputs
    qkv, mlp = bench.BENCH_WORKLOADS.get(workload, (workload, None))
    work = {}
    if qkv:
        work.update(bench.stage_work(inputs.WORKLOADS[qkv], 1))
    if mlp:
        work.update(bench.mlp_stage_work(inputs.MLP_WORKLOADS[mlp], (1, 1)))
    return {s: v for s, (kind, v) in work.items() if kind == "mfma"}


def mfma_rows(counter_csv: str, xcc: int, simds: int, workload: str,
              separate_pack: bool = False) -> tuple[dict, float]:
    """Per GEMM stage: mean MFMA F8 instructions, busy cycles, active cycles
    per XCD and duration of a launch; and the shader clock fitted over every
    step launch (active cycles per XCD against duration, least squares: the
    slope is the clock, the intercept the counter window's fixed overhead)."""
    order = step_order(workload, separate_pack)
    flop = gemm_flop(workload)
    ns = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
          for r in csv.DictReader(open(counter_csv))}
    per = {c: _by_stage(counter_csv, _dispatches(counter_csv, c), order)
           for c in ("SQ_INSTS_VALU_MFMA_F8", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
    gui = [(ns[d], v / xcc) for dv in per["GRBM_GUI_ACTIVE"].values() for d, v in dv]
    clock_ghz = statistics.linear_regression([t for t, _ in gui], [c for _, c in gui]).slope
    rows = {}
    for s in dict.fromkeys(order):
        if s not in flop:
            continue
        inst = statistics.mean(v for _, v in per["SQ_INSTS_VALU_MFMA_F8"][s])
        busy = statistics.mean(v for _, v in per["SQ_VALU_MFMA_BUSY_CYCLES"][s])
        act = statistics.mean(v / xcc for _, v in per["GRBM_GUI_ACTIVE"][s])
        t = statistics.mean(ns[d] for d, _ in per["GRBM_GUI_ACTIVE"][s])
        rows[s] = dict(launches=len(per["GRBM_GUI_ACTIVE"][s]), inst=inst,
                       flop_ratio=inst * MFMA_FLOP / flop[s], busy_per_inst=busy / inst,
                       us=t / 1e3, util=busy / (act * simds),
                       busy_frac=busy / (simds * clock_ghz * t))
    return rows, clock_ghz


def mfma(counter_csv: str, agent_csv: str, workload: str, cmd: str) -> str:
    gpu = [r for r in csv.DictReader(open(agent_csv)) if r["Agent_Type"] == "GPU"][0]
    xcc, simds = int(gpu["Num_Xcc"]), int(gpu["Simd_Count"])
    rows, clock = mfma_rows(counter_csv, xcc, simds, workload, SEPARATE_FLAG in cmd)
    out = [f"# Matrix-core use of the GEMMs, {workload}\n",
           "Command (run from /tmp with TMPDIR=/tmp, repository at $R):\n",
           "```\n" + cmd + "\n```\n",
           f"{xcc} XCDs, {simds} SIMDs. Shader clock fitted over every step launch "
           f"(active cycles per XCD against duration): {clock:.2f} GHz.\n",
           "| stage | launches | MFMA F8 instr / launch | instr x 131072 / 2MNK | busy cycles / instr "
           "| µs | MfmaUtil | busy at fitted clock |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for s, r in rows.items():
        out.append(f"| `{s}` | {r['launches']} | {r['inst']:.0f} | {r['flop_ratio']:.4f} | "
                   f"{r['busy_per_inst']:.2f} | {r['us']:.1f} | {100 * r['util']:.1f}% | "
                   f"{100 * r['busy_frac']:.1f}% |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        sys.stdout.write(stats(sys.argv[2], sys.argv[3], sys.argv[4],
                               sys.argv[5] if len(sys.argv) > 5 else None,
                               sys.argv[6] if len(sys.argv) > 6 else None))
    elif mode == "traffic":
        sys.stdout.write(traffic(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:])))
    elif mode == "mfma":
        sys.stdout.write(mfma(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:])))
    else:
        raise SystemExit(__doc__)
