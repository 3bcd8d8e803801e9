#!/usr/bin/env python3
"""Benchmark of the packed FP8 QKV projection (reduced-width Q/K) on one MI355X.

One step = the weight pack (the weight cache is rebuilt every step) and
the forward, in one qkv_pack_forward call, + qkv_backward at D=768, 6 heads,
d_qk=96, d_v=128 (packed N=1920), T=65536 tokens in one sequence, all
through the C interface of libfpr.so (--pack-forward separate: the pack and
the forward as pack_quantize_weights + qkv_forward).  Inputs are synthetic (seeded normals of the shapes the pages
train on) and resident in HBM before timing starts.

Prints one JSON line: whole-step tokens/s, TFLOP/s of the FP8 GEMMs
against the FP8 dense peak, the live roofline of the dominant kernel (timed
with HIP events on its launch stream inside the timed region), and the CPU
oracle timed on a bounded sample on this host.

Other workloads (--workload): the QKV shapes of ``inputs.WORKLOADS``; the
FP8 ReLU^2 MLP alone (``mlp_64k``: mlp_pack_forward + mlp_backward at
D=768, d_ff=3072, T=65536); and the block's projection set
(``block_64k``: the QKV step of ``step_64k`` followed by the MLP step of
``mlp_64k``).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed FP8 QKV fwd+bwd tokens/s and TFLOP/s (% FP8 peak) at D=768,H=6,T=65536"
METRIC_MLP = "FP8 ReLU^2 MLP fwd+bwd tokens/s and TFLOP/s (% FP8 peak) at D=768,d_ff=3072,T=65536"
METRIC_BLOCK = ("packed FP8 QKV + FP8 ReLU^2 MLP fwd+bwd tokens/s and TFLOP/s (% FP8 peak) at "
                "D=768,H=6,d_ff=3072,T=65536")
# workload -> (QKV shapes or None, MLP shapes or None)
BENCH_WORKLOADS = {"mlp_64k": (None, "mlp_64k"), "block_64k": ("step_64k", "mlp_64k")}
PEAK_FP8_FLOPS = 5.0e15   # MI355X dense FP8 MFMA
PEAK_HBM_BYTES = 8.0e12   # MI355X HBM3E
CALIB_FLOATS = 64 << 20   # counter calibration: encoder over 256 MiB of fp32
STAGE_SOURCES = {
    "amax_w": "quantize.hip", "quantize_w": "quantize.hip",
    "amax_x": "quantize.hip", "quantize_x": "quantize.hip", "quantize_g": "quantize.hip",
    "amax_dv": "quantize.hip", "amax_wx": "quantize.hip", "quantize_wx": "quantize.hip",
    "gemm_fwd": "gemm.hip", "gemm_dx": "gemm.hip", "gemm_dw": "gemm.hip",
    "dw_reduce": "gemm.hip", "norm_rope_fwd": "epilogue.hip", "norm_rope_bwd": "epilogue.hip",
    "mlp_amax_w": "quantize.hip", "mlp_quantize_w": "quantize.hip",
    "mlp_amax_x": "quantize.hip", "mlp_quantize_x": "quantize.hip",
    "mlp_amax_wx": "quantize.hip", "mlp_quantize_wx": "quantize.hip",
    "mlp_quantize_h": "quantize.hip", "mlp_amax_dy": "quantize.hip",
    "mlp_quantize_dy": "quantize.hip", "mlp_quantize_dpre": "quantize.hip",
    "mlp_gemm_up": "gemm.hip", "mlp_gemm_down": "gemm.hip", "mlp_gemm_dh": "gemm.hip",
    "mlp_gemm_dx": "gemm.hip", "mlp_gemm_dw1": "gemm.hip", "mlp_gemm_dw2": "gemm.hip",
    "mlp_dw1_reduce": "gemm.hip", "mlp_dw2_reduce": "gemm.hip",
}


TRACE_STEPS = 10


def stage_work(w: dict, dw_splits: int, two_pass: bool = False) -> dict:
    """Algorithmic work per launch: ("mfma", FLOP) or ("hbm", bytes).  With
    the two-pass backward, norm_rope_bwd is its amax pass (the forward's rows
    in, nothing out) and quantize_g its second pass (the same rows and dv in,
    the gradient codes out)."""
    T = w["n_seq"] * w["seq_len"]
    D, H, dqk, dv = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    N = H * (2 * dqk + dv)
    qk, vv = 2 * H * dqk, H * dv
    gemm = 2 * T * D * N
    fwd_rows = 2 * T * qk * 2 + 4 * T * 2 * H  # dq, dk, q, k and the 1/rms of each row
    two = {"norm_rope_bwd": ("hbm", fwd_rows),
           "quantize_g": ("hbm", fwd_rows + 2 * T * vv + T * N)} if two_pass else {}
    return {
        "amax_w": ("hbm", 4 * D * N),
        "quantize_w": ("hbm", 4 * D * N + 2 * D * N),            # fp32 in, two e4m3 layouts out
        "amax_x": ("hbm", 2 * T * D),
        "quantize_x": ("hbm", 2 * T * D + T * D),                # bf16 in, e4m3 out
        # qkv_pack_forward: the two above pairs, each in one launch
        "amax_wx": ("hbm", 4 * D * N + 2 * T * D),
        "quantize_wx": ("hbm", 6 * D * N + 3 * T * D),
        "gemm_fwd": ("mfma", gemm),   # with the norm/RoPE in its epilogue at d_qk 64/96/128
        "norm_rope_fwd": ("hbm", 2 * T * qk + 2 * T * qk),       # other widths: pre-norm in, q|k out
        # dq, dk, q, k and the 1/rms of each Q/K head row in; dQK out
        "norm_rope_bwd": ("hbm", 2 * T * qk * 2 + 2 * T * qk + 4 * T * 2 * H),
        "amax_dv": ("hbm", 2 * T * vv),
        "quantize_g": ("hbm", 2 * T * N + T * N),
        "gemm_dx": ("mfma", gemm),
        "gemm_dw": ("mfma", gemm),
        "dw_reduce": ("hbm", dw_splits * 4 * D * N + 4 * D * N),
        **two,
    }


def mlp_stage_work(w: dict, dw_splits: tuple[int, int]) -> dict:
    """Algorithmic work per launch of the MLP's stages."""
    T = w["n_seq"] * w["seq_len"]
    D, F = w["d_model"], w["d_ff"]
    gemm = ("mfma", 2 * T * D * F)
    return {
        "mlp_amax_w": ("hbm", 4 * D * F),                  # one launch per weight
        "mlp_quantize_w": ("hbm", 4 * D * F + 2 * D * F),
        "mlp_amax_x": ("hbm", 2 * T * D),
        "mlp_quantize_x": ("hbm", 3 * T * D),
        # mlp_pack_forward: both weights' pairs and x's, each kind in one launch
        "mlp_amax_wx": ("hbm", 2 * 4 * D * F + 2 * T * D),
        "mlp_quantize_wx": ("hbm", 2 * (4 * D * F + 2 * D * F) + 3 * T * D),
        "mlp_gemm_up": gemm,
        "mlp_quantize_h": ("hbm", 3 * T * F),
        "mlp_gemm_down": gemm,
        "mlp_amax_dy": ("hbm", 2 * T * D),
        "mlp_quantize_dy": ("hbm", 3 * T * D),
        "mlp_gemm_dh": gemm,
        "mlp_quantize_dpre": ("hbm", 3 * T * F),
        "mlp_gemm_dx": gemm,
        "mlp_gemm_dw1": gemm,
        "mlp_dw1_reduce": ("hbm", dw_splits[0] * 4 * D * F + 4 * D * F),
        "mlp_gemm_dw2": gemm,
        "mlp_dw2_reduce": ("hbm", dw_splits[1] * 4 * D * F + 4 * D * F),
    }


def measured_ceilings(B, dev, reps: int = 5) -> dict:
    """The device's practical ceilings, taken in this run with the library's
    probe kernels and HIP events: a streaming copy and a streaming read of
    1 GiB (four times the last-level cache), and the bare FP8 MFMA loop
    (2 waves per SIMD, 4 independent accumulators each).  Medians of reps."""
    import torch
    stream = torch.cuda.current_stream(dev)

    def timed(launch) -> float:
        ts = []
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            ts.append(e0.elapsed_time(e1) / 1e3)
        return sorted(ts[1:])[reps // 2]

    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    words = torch.empty(8192, dtype=torch.int32, device=dev)
    blocks = 64 * torch.cuda.get_device_properties(dev).multi_processor_count
    t_copy = timed(lambda: B.probe_copy(src, dst, blocks))
    t_read = timed(lambda: B.probe_read(src, words, blocks))
    del src, dst
    mb, iters = 4 * torch.cuda.get_device_properties(dev).multi_processor_count, 2000
    sink = torch.empty(mb * 8, dtype=torch.float32, device=dev)
    flop = B.probe_mfma(mb, iters, sink)
    t_mfma = timed(lambda: B.probe_mfma(mb, iters, sink))
    return {"copy_GBps": round(2 * nbytes / t_copy / 1e9, 1),
            "read_GBps": round(nbytes / t_read / 1e9, 1),
            "mfma_TFLOPs": round(flop / t_mfma / 1e12, 1),
            "how": "library probe kernels in this run: streaming copy and read of 1 GiB "
                   "(non-temporal 16-byte loads, four in flight per thread, 64 blocks per CU) "
                   "(cold: 4x the last-level cache; a kernel whose inputs partly hit that "
                   "cache can exceed them), bare FP8 32x32x64 MFMA loop; HIP events, "
                   "median of 5"}


def ceiling_of(stage: str, kind: str, ceil: dict) -> float:
    """The measured ceiling a stage is held to: the MFMA loop for the GEMMs,
    the streaming read for the read-only amax passes, the copy otherwise."""
    if kind == "mfma":
        return ceil["mfma_TFLOPs"] * 1e12
    if "amax" in stage:
        return ceil["read_GBps"] * 1e9
    return ceil["copy_GBps"] * 1e9


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def source_hash(stage: str) -> str:
    """Hash of the code of a stage's kernel source: comments and blank space
    dropped, so that a comment edit keeps its counter lines valid."""
    path = os.path.join(ROOT, "fp8_packed_reduced_amd", "csrc", STAGE_SOURCES[stage])
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:12]


def read_traffic(workload: str, stage: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        if len(f) >= 4 and f[0] == stage:
            if f[3] != source_hash(stage):
                return None
            return int(float(f[1])) + int(float(f[2]))
    return None


def _oracle_step(w: dict, seed: int, tokens: int, backward: bool = True) -> float:
    """Seconds the oracle takes for pack + forward (+ backward) of the first
    `tokens` tokens of the workload (as one sequence)."""
    import oracle
    from fp8_packed_reduced_amd import inputs
    wl = dict(w, n_seq=1, seq_len=tokens)
    x = inputs.make_x(wl, seed)
    W = inputs.make_w(wl, seed + 1)
    dq, dk, dv = inputs.make_dy(wl, seed + 2)
    dims = inputs.dims_of(wl)
    nqk2 = 2 * w["n_heads"] * w["d_qk"]
    oracle.lib()
    t0 = time.perf_counter()
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    of = oracle.qkv_forward(dims, 1, tokens, x, wp, s_w)
    if backward:
        oracle.qkv_backward(dims, 1, tokens, dq, dk, dv, of["x8"], of["s_x"],
                            of["y_bits"][:, :nqk2], wp, s_w)
    return time.perf_counter() - t0


def _oracle_mlp_step(w: dict, seed: int, tokens: int) -> float:
    """Seconds the oracle takes for the MLP's pack + forward + backward of the
    first `tokens` tokens of the workload."""
    import oracle
    from fp8_packed_reduced_amd import inputs
    wl = dict(w, n_seq=1, seq_len=tokens)
    x = inputs.make_x(wl, seed)
    w1, w2 = inputs.make_mlp_w(wl, seed + 1)
    dy = inputs.make_mlp_dy(wl, seed + 2)
    oracle.lib()
    t0 = time.perf_counter()
    wq = oracle.mlp_quantize_weights(w1, w2)
    fw = oracle.mlp_forward(x, wq)
    oracle.mlp_backward(dy, fw["x8"], fw["s_x"], fw["h8"], fw["s_h"], wq)
    return time.perf_counter() - t0


def cpu_baseline(T: int, oracle_step, seed: int, target_s: float, c1_step=None,
                 what: str = "pack + forward + backward") -> dict:
    """The oracle, untouched, timed on a bounded prefix of the workload whose
    length is chosen (in multiples of 4096 tokens, at most the whole
    workload) from a 4096-token probe so that it takes about target_s; when
    the whole workload takes less, it is run repeatedly for about target_s.
    oracle_step(seed, tokens) returns the seconds one step of that prefix
    takes.  c1_step(seed), if given, is timed once more on one thread (the
    tiny configuration's step)."""
    probe = min(4096, T)
    t_probe = oracle_step(seed, probe)
    tokens = int(min(T, max(probe, probe * round(target_s / max(t_probe, 1e-3)))))
    dt = oracle_step(seed, tokens)
    reps = max(1, int(round(target_s / max(dt, 1e-3)))) if tokens == T else 1
    for _ in range(reps - 1):
        dt += oracle_step(seed, tokens)
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info())
    except Exception:
        cores = os.cpu_count()
    runs = f", {reps} runs" if reps > 1 else ""
    single = None
    if c1_step is not None:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                single = round(c1_step(seed), 3)
        except Exception:
            single = None
    return {"value": round(reps * tokens / dt, 1), "unit": "tokens/s", "cores": cores,
            "cpu_model": cpu_model(), "c1_single_thread_s": single,
            "kind": "oracle",
            "sample": f"{what} of the first {tokens} tokens (one sequence, "
                      f"positions 0..{tokens - 1}) of the same workload and seed{runs}; "
                      f"{dt:.2f} s"}


# A weight large enough for the weight quantiser to stream (4096 x 10240 fp32,
# 168 MB: 32 heads of the pages' widths at D = 4096): at the benchmark's
# 5.9 MB the two pack kernels are launch-latency bound.
WIDE_PACK = dict(n_seq=1, seq_len=256, d_model=4096, n_heads=32, d_qk=96, d_v=128)


def pack_streaming(B, inputs, dev, seed: int, reps: int = 20) -> dict:
    import torch
    w = WIDE_PACK
    D, H, dqk, dv = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    N, nq = H * (2 * dqk + dv), H * dqk
    dims = B.make_dims(D, H, dqk, dv, inputs.EPS, inputs.ROPE_BASE)
    W = torch.from_numpy(inputs.make_w(w, seed + 1)).to(dev)
    cache = B.WeightCache(dims, dev)
    ws = torch.empty(B.workspace_bytes(dims, 0, B.FPR_CALL_PACK), dtype=torch.uint8, device=dev)
    args = (dims, W[:, :nq], W[:, nq:2 * nq], W[:, 2 * nq:], cache)
    B.pack_quantize_weights(*args, workspace=ws)
    torch.cuda.synchronize()
    with B.KernelTrace(2 * reps, device=dev) as tr:
        for _ in range(reps):
            B.pack_quantize_weights(*args, workspace=ws)
    torch.cuda.synchronize()
    t = {}
    for name, ms in tr.records():
        t[name] = t.get(name, 0.0) + ms / reps
    work = {"amax_w": 4 * D * N, "quantize_w": 6 * D * N}
    out = {"workload": f"W [{D}][{N}] fp32 ({4 * D * N / 1e6:.0f} MB)"}
    for name, b in work.items():
        rate = b / (t[name] / 1e3)
        out[name] = {"us": round(t[name] * 1e3, 2), "GB/s": round(rate / 1e9, 1),
                     "frac": round(rate / PEAK_HBM_BYTES, 4)}
    del W, cache, ws
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="step_64k")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the step replayed from a captured HIP graph")
    ap.add_argument("--forward-only", action="store_true",
                    help="time pack + forward only (the 16k-token forward configuration)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the step-time percentiles and the large-weight quantiser "
                         "measurement (profiling runs, whose dispatches must be whole steps)")
    ap.add_argument("--bwd-passes", type=int, choices=[1, 2], default=1,
                    help="2: the backward in two passes that never write dQK")
    ap.add_argument("--pack-forward", choices=["combined", "separate"], default="combined",
                    help="combined: the weight pack and the forward in one call "
                         "(qkv_pack_forward, mlp_pack_forward), whose quantiser launches serve "
                         "the weights and x together; separate: the pack call, then the "
                         "forward call")
    ap.add_argument("--grad-format", choices=["e4m3", "e5m2"], default="e4m3",
                    help="FP8 format of the backward's gradient codes (QKV and MLP)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X and has no "
              "multi-GPU mode (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp8_packed_reduced_amd import binding as B
    from fp8_packed_reduced_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qkv_name, mlp_name = BENCH_WORKLOADS.get(args.workload, (args.workload, None))
    w = inputs.WORKLOADS[qkv_name] if qkv_name else None
    wm = inputs.MLP_WORKLOADS[mlp_name] if mlp_name else None
    T = (w or wm)["n_seq"] * (w or wm)["seq_len"]

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    steps, work, gemm_flop, config, oracle_steps = [], {}, 0, {"workload": args.workload,
                                                               "tokens": T}, []
    if w is not None:
        n_seq, S = w["n_seq"], w["seq_len"]
        D, H, dqk, dvw = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
        N, nq = H * (2 * dqk + dvw), H * dqk
        gfmt = B.FORMAT_E5M2 if args.grad_format == "e5m2" else B.FORMAT_E4M3
        dims = B.make_dims(D, H, dqk, dvw, inputs.EPS, inputs.ROPE_BASE, grad_format=gfmt,
                           bwd_passes=args.bwd_passes)
        x = bf16(inputs.make_x(w, args.seed))
        W = torch.from_numpy(inputs.make_w(w, args.seed + 1)).to(dev)
        dq, dk, dv = (bf16(a) for a in inputs.make_dy(w, args.seed + 2))
        wq, wk, wv = W[:, :nq], W[:, nq:2 * nq], W[:, 2 * nq:]
        cache = B.WeightCache(dims, dev)
        ws_p = torch.empty(B.workspace_bytes(dims, 0, B.FPR_CALL_PACK), dtype=torch.uint8,
                           device=dev)
        ws_f = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_FORWARD), dtype=torch.uint8,
                           device=dev)
        ws_b = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_BACKWARD), dtype=torch.uint8,
                           device=dev)
        saved = torch.empty(B.saved_bytes(dims, T), dtype=torch.uint8, device=dev)
        q = torch.empty((n_seq, H, S, dqk), dtype=torch.bfloat16, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((n_seq, H, S, dvw), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((D, N), dtype=torch.float32, device=dev)

        combined = args.pack_forward == "combined"
        if combined:
            ws_f = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_PACK_FORWARD),
                               dtype=torch.uint8, device=dev)

        def qkv_step():
            if combined:
                B.qkv_pack_forward(dims, wq, wk, wv, cache, n_seq, S, x, q, k, v, saved, ws_f)
            else:
                B.pack_quantize_weights(dims, wq, wk, wv, cache, workspace=ws_p)
                B.qkv_forward(dims, n_seq, S, x, cache, q, k, v, saved, ws_f)
            if not args.forward_only:
                B.qkv_backward(dims, n_seq, S, q, k, dq, dk, dv, saved, cache, dx, dw, ws_b)

        steps.append(qkv_step)
        work.update(stage_work(w, B.layout(dims, T).dw_splits, args.bwd_passes == 2))
        gemm_flop += (1 if args.forward_only else 3) * 2 * T * D * N
        config.update(n_seq=n_seq, seq_len=S, d_model=D, n_heads=H, d_qk=dqk, d_v=dvw,
                      packed_n=N)
        if args.grad_format != "e4m3":
            config["grad_format"] = args.grad_format
        if args.bwd_passes == 2:
            config["bwd_passes"] = 2
        if not combined:
            config["pack_forward"] = "separate"
        oracle_steps.append(
            lambda seed, tokens: _oracle_step(w, seed, tokens, not args.forward_only))
    if wm is not None:
        Dm, F = wm["d_model"], wm["d_ff"]
        mdims = B.MlpDims(Dm, F, B.FORMAT_E5M2 if args.grad_format == "e5m2" else B.FORMAT_E4M3)
        mx = bf16(inputs.make_x(wm, args.seed))
        w1, w2 = (torch.from_numpy(a).to(dev) for a in inputs.make_mlp_w(wm, args.seed + 1))
        mdy = bf16(inputs.make_mlp_dy(wm, args.seed + 2))
        mcache = B.MlpCache(mdims, dev)
        mws_p = torch.empty(B.mlp_workspace_bytes(mdims, 0, B.FPR_CALL_PACK), dtype=torch.uint8,
                            device=dev)
        mcombined = args.pack_forward == "combined"
        mws_f = torch.empty(B.mlp_workspace_bytes(mdims, T, B.FPR_CALL_PACK_FORWARD if mcombined
                                                  else B.FPR_CALL_FORWARD),
                            dtype=torch.uint8, device=dev)
        mws_b = torch.empty(B.mlp_workspace_bytes(mdims, T, B.FPR_CALL_BACKWARD),
                            dtype=torch.uint8, device=dev)
        msaved = torch.empty(B.mlp_saved_bytes(mdims, T), dtype=torch.uint8, device=dev)
        my = torch.empty((T, Dm), dtype=torch.bfloat16, device=dev)
        mdx = torch.empty((T, Dm), dtype=torch.bfloat16, device=dev)
        dw1 = torch.empty((Dm, F), dtype=torch.float32, device=dev)
        dw2 = torch.empty((F, Dm), dtype=torch.float32, device=dev)

        def mlp_step():
            if mcombined:
                B.mlp_pack_forward(mdims, w1, w2, mcache, mx, my, msaved, mws_f)
            else:
                B.mlp_pack_quantize_weights(mdims, w1, w2, mcache, workspace=mws_p)
                B.mlp_forward(mdims, mx, mcache, my, msaved, mws_f)
            B.mlp_backward(mdims, mdy, msaved, mcache, mdx, dw1, dw2, mws_b)

        steps.append(mlp_step)
        ml = B.mlp_layout(mdims, T)
        work.update(mlp_stage_work(wm, (ml.dw1_splits, ml.dw2_splits)))
        gemm_flop += 6 * 2 * T * Dm * F
        config.update(d_model=Dm, d_ff=F)
        if args.grad_format != "e4m3":
            config["grad_format"] = args.grad_format
        if args.bwd_passes == 2:
            config["bwd_passes"] = 2
        if not mcombined:
            config["pack_forward"] = "separate"
        oracle_steps.append(lambda seed, tokens: _oracle_mlp_step(wm, seed, tokens))
    qkv_calls = ("qkv_pack_forward" if args.pack_forward == "combined" else
                 "pack_quantize_weights + qkv_forward")
    config["step"] = " + ".join(
        ([qkv_calls + ("" if args.forward_only else " + qkv_backward")]
         if w is not None else []) +
        ([("mlp_pack_forward" if args.pack_forward == "combined" else
           "mlp_pack_quantize_weights + mlp_forward") + " + mlp_backward"]
         if wm is not None else []))
    config["seed"] = args.seed
    metric = METRIC if wm is None else METRIC_MLP if w is None else METRIC_BLOCK
    if w is not None and (D, H, T, dqk) != (768, 6, 65536, 96):  # another QKV shape
        metric = (f"packed FP8 QKV fwd+bwd tokens/s and TFLOP/s (% FP8 peak) at "
                  f"D={D},H={H},d_qk={dqk},T={T}")
    if args.forward_only:
        if wm is not None:
            raise SystemExit("--forward-only applies to the QKV workloads")
        metric = metric.replace("fwd+bwd", "forward (pack + forward)")

    def eager_step():
        for f in steps:
            f()

    step = eager_step

    # A streaming kernel of known traffic (the e4m3 encoder: 256 MiB of fp32
    # read, 64 MiB of codes written), so that rocprofv3 byte counters taken on
    # this same command can be calibrated.  Not timed, not part of a step.
    calib = torch.zeros(CALIB_FLOATS, dtype=torch.float32, device=dev)
    for _ in range(3):
        B.e4m3_encode(calib)
    torch.cuda.synchronize()
    del calib

    ceil = measured_ceilings(B, dev)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    if args.graph:  # the same kernels, launched by one graph replay per step
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()
        step = graph.replay
        step()
        torch.cuda.synchronize()
    # Per-stage times: the mean over TRACE_STEPS traced steps (the sum of a
    # stage's launches in a step; a single step is too noisy to rank by).
    with B.KernelTrace(32 * TRACE_STEPS, device=dev) as tr:
        for _ in range(TRACE_STEPS):
            eager_step()
    torch.cuda.synchronize()
    per_stage, launches = {}, {}
    for name, ms in tr.records():
        per_stage[name] = per_stage.get(name, 0.0) + ms / TRACE_STEPS
        launches[name] = launches.get(name, 0) + 1
    dominant = max(per_stage, key=per_stage.get)

    K = args.steps
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # The dominant kernel is timed inside the timed region; a graph replay
    # makes no library calls, so in that mode it is timed over K eager steps.
    dom = B.KernelTrace(K * launches[dominant] // TRACE_STEPS, only=dominant, device=dev)
    with (contextlib.nullcontext() if args.graph else dom):
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
    if args.graph:
        with dom:
            for _ in range(K):
                eager_step()
        torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / K
    dom_ms = [ms for _, ms in dom.records()]
    dom_avg_s = sum(dom_ms) / len(dom_ms) / 1e3
    kind, amount = work[dominant]
    if kind == "mfma":
        achieved, peak, unit = amount / dom_avg_s / 1e12, PEAK_FP8_FLOPS / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = amount / dom_avg_s / 1e9, PEAK_HBM_BYTES / 1e9, "GB/s"
    traffic = read_traffic(args.workload, dominant)

    tflops = gemm_flop / (ms_step / 1e3) / 1e12
    tokens_per_s = T / (ms_step / 1e3)
    kernels = {}
    for name, ms in per_stage.items():
        kd, amt = work[name]
        n_launch = launches[name] // TRACE_STEPS
        rate = n_launch * amt / (ms / 1e3)
        kernels[name] = {"us": round(ms * 1e3, 2),
                         ("TFLOP/s" if kd == "mfma" else "GB/s"):
                             round(rate / (1e12 if kd == "mfma" else 1e9), 1),
                         "frac": round(rate / (PEAK_FP8_FLOPS if kd == "mfma" else PEAK_HBM_BYTES), 4),
                         "frac_measured": round(rate / ceiling_of(name, kd, ceil), 4)}
        if n_launch > 1:
            kernels[name]["launches"] = n_launch

    out = {
        "metric": metric,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": config,
        "tflops": round(tflops, 1),
        "pct_fp8_peak": round(100 * tflops * 1e12 / PEAK_FP8_FLOPS, 2),
        "wall_ms_per_step": round(t_wall * 1e3 / K, 4),
        "launch": "hip graph replay" if args.graph else "eager",
        "device": f"{torch.cuda.get_device_name(dev)} "
                  f"({getattr(torch.cuda.get_device_properties(dev), 'gcnArchName', '?')}, "
                  f"{torch.cuda.get_device_properties(dev).multi_processor_count} CUs)",
        "roofline": {"kernel": dominant, "bound": kind, "achieved": round(achieved, 1),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "launches": len(dom_ms),
                     "avg_us": round(dom_avg_s * 1e6, 2),
                     "measured_ceiling": round(ceiling_of(dominant, kind, ceil) /
                                               (1e12 if kind == "mfma" else 1e9), 1),
                     "frac_measured": round(amount / dom_avg_s / ceiling_of(dominant, kind, ceil),
                                            4)},
        "measured_ceilings": ceil,
        "kernels": kernels,
    }
    if not args.no_extras:
        # Per-step distribution: one event per step boundary over another K steps.
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(K):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(K))
        out["step_ms_p10_p50_p90"] = [round(per[int(0.1 * (K - 1))], 4),
                                      round(per[(K - 1) // 2], 4),
                                      round(per[int(0.9 * (K - 1))], 4)]
        # Cold: 512 MB written between steps evicts the 256 MB last-level
        # cache; each step is timed on its own, the flush outside the events.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for i in range(min(K, 20)):
            flush.fill_(i & 0xFF)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        del flush
        out["cold_ms_per_step"] = round(sum(cold) / len(cold), 4)
        if w is not None:
            out["weight_quantiser_streaming"] = pack_streaming(B, inputs, dev, args.seed)
    if not args.no_cpu_baseline:
        tiny = inputs.WORKLOADS["tiny"]
        c1 = (lambda seed: _oracle_step(tiny, seed, tiny["seq_len"])) if w is not None else None
        out["cpu_baseline"] = cpu_baseline(
            T, lambda seed, tokens: sum(f(seed, tokens) for f in oracle_steps), args.seed,
            args.cpu_seconds, c1,
            "pack + forward" if args.forward_only else "pack + forward + backward")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
