#!/usr/bin/env python3
"""Benchmark of the packed FP8 QKV projection (reduced-width Q/K) on one MI355X.

One step = pack_quantize_weights (the weight cache is rebuilt every step) +
qkv_forward + qkv_backward at D=768, 6 heads, d_qk=96, d_v=128 (packed
N=1920), T=65536 tokens in one sequence, all through the C interface of
libfpr.so.  Inputs are synthetic (seeded normals of the shapes the pages
train on) and resident in HBM before timing starts.

Prints one JSON line: whole-step tokens/s, TFLOP/s of the three FP8 GEMMs
against the FP8 dense peak, the live roofline of the dominant kernel (timed
with HIP events on its launch stream inside the timed region), and the CPU
oracle timed on a bounded sample on this host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed FP8 QKV fwd+bwd tokens/s and TFLOP/s (% FP8 peak) at D=768,H=6,T=65536"
PEAK_FP8_FLOPS = 5.0e15   # MI355X dense FP8 MFMA
PEAK_HBM_BYTES = 8.0e12   # MI355X HBM3E
CALIB_FLOATS = 64 << 20   # counter calibration: encoder over 256 MiB of fp32
STAGE_SOURCES = {
    "amax_w": "quantize.hip", "quantize_w": "quantize.hip",
    "amax_x": "quantize.hip", "quantize_x": "quantize.hip", "quantize_g": "quantize.hip",
    "gemm_fwd": "gemm.hip", "gemm_dx": "gemm.hip", "gemm_dw": "gemm.hip",
    "dw_reduce": "gemm.hip", "norm_rope_fwd": "epilogue.hip", "norm_rope_bwd": "epilogue.hip",
}


TRACE_STEPS = 10


def stage_work(w: dict, dw_splits: int) -> dict:
    """Algorithmic work per launch: ("mfma", FLOP) or ("hbm", bytes)."""
    T = w["n_seq"] * w["seq_len"]
    D, H, dqk, dv = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    N = H * (2 * dqk + dv)
    qk, vv = 2 * H * dqk, H * dv
    gemm = 2 * T * D * N
    return {
        "amax_w": ("hbm", 4 * D * N),
        "quantize_w": ("hbm", 4 * D * N + 2 * D * N),            # fp32 in, two e4m3 layouts out
        "amax_x": ("hbm", 2 * T * D),
        "quantize_x": ("hbm", 2 * T * D + T * D),                # bf16 in, e4m3 out
        "gemm_fwd": ("mfma", gemm),
        "norm_rope_fwd": ("hbm", 2 * T * qk + 2 * T * qk),       # pre-norm Q|K in, q|k out
        "norm_rope_bwd": ("hbm", 2 * T * qk * 2 + 2 * T * vv + 2 * T * qk),  # dq,dk,pre, dv in; dQK out
        "quantize_g": ("hbm", 2 * T * N + T * N),
        "gemm_dx": ("mfma", gemm),
        "gemm_dw": ("mfma", gemm),
        "dw_reduce": ("hbm", dw_splits * 4 * D * N + 4 * D * N),
    }


def source_hash(stage: str) -> str:
    path = os.path.join(ROOT, "fp8_packed_reduced_amd", "csrc", STAGE_SOURCES[stage])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:12]


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


def _oracle_step(w: dict, seed: int, tokens: int) -> float:
    """Seconds the oracle takes for pack + forward + backward of the first
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
    oracle.qkv_backward(dims, 1, tokens, dq, dk, dv, of["x8"], of["s_x"],
                        of["y_bits"][:, :nqk2], wp, s_w)
    return time.perf_counter() - t0


def cpu_baseline(w: dict, seed: int, target_s: float) -> dict:
    """The oracle, untouched, timed on a bounded prefix of the workload whose
    length is chosen (in multiples of 4096 tokens, at most the whole
    workload) from a 4096-token probe so that it takes about target_s; when
    the whole workload takes less, it is run repeatedly for about target_s."""
    T = w["n_seq"] * w["seq_len"]
    probe = min(4096, T)
    t_probe = _oracle_step(w, seed, probe)
    tokens = int(min(T, max(probe, probe * round(target_s / max(t_probe, 1e-3)))))
    dt = _oracle_step(w, seed, tokens)
    reps = max(1, int(round(target_s / max(dt, 1e-3)))) if tokens == T else 1
    for _ in range(reps - 1):
        dt += _oracle_step(w, seed, tokens)
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info())
    except Exception:
        cores = os.cpu_count()
    runs = f", {reps} runs" if reps > 1 else ""
    return {"value": round(reps * tokens / dt, 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"pack + forward + backward of the first {tokens} tokens (one sequence, "
                      f"positions 0..{tokens - 1}) of the same workload and seed{runs}; "
                      f"{dt:.2f} s"}


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
    w = inputs.WORKLOADS[args.workload]
    n_seq, S = w["n_seq"], w["seq_len"]
    T = n_seq * S
    D, H, dqk, dvw = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    N, nq = H * (2 * dqk + dvw), H * dqk
    dims = B.make_dims(D, H, dqk, dvw, inputs.EPS, inputs.ROPE_BASE)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x = bf16(inputs.make_x(w, args.seed))
    W = torch.from_numpy(inputs.make_w(w, args.seed + 1)).to(dev)
    dq, dk, dv = (bf16(a) for a in inputs.make_dy(w, args.seed + 2))
    wq, wk, wv = W[:, :nq], W[:, nq:2 * nq], W[:, 2 * nq:]
    cache = B.WeightCache(dims, dev)
    ws_p = torch.empty(B.workspace_bytes(dims, 0, B.FPR_CALL_PACK), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_FORWARD), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_BACKWARD), dtype=torch.uint8, device=dev)
    saved = torch.empty(B.saved_bytes(dims, T), dtype=torch.uint8, device=dev)
    q = torch.empty((n_seq, H, S, dqk), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((n_seq, H, S, dvw), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((D, N), dtype=torch.float32, device=dev)

    def step():
        B.pack_quantize_weights(dims, wq, wk, wv, cache, workspace=ws_p)
        B.qkv_forward(dims, n_seq, S, x, cache, q, k, v, saved, ws_f)
        B.qkv_backward(dims, n_seq, S, dq, dk, dv, saved, cache, dx, dw, ws_b)

    # A streaming kernel of known traffic (the e4m3 encoder: 256 MiB of fp32
    # read, 64 MiB of codes written), so that rocprofv3 byte counters taken on
    # this same command can be calibrated.  Not timed, not part of a step.
    calib = torch.zeros(CALIB_FLOATS, dtype=torch.float32, device=dev)
    for _ in range(3):
        B.e4m3_encode(calib)
    torch.cuda.synchronize()
    del calib

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    # Per-stage times: the mean over TRACE_STEPS traced steps (one sample per
    # stage and step; a single step is too noisy to rank the stages by).
    with B.KernelTrace(16 * TRACE_STEPS, device=dev) as tr:
        for _ in range(TRACE_STEPS):
            step()
    torch.cuda.synchronize()
    per_stage = {}
    for name, ms in tr.records():
        per_stage[name] = per_stage.get(name, 0.0) + ms / TRACE_STEPS
    dw_splits = B.layout(dims, T).dw_splits
    work = stage_work(w, dw_splits)
    dominant = max(per_stage, key=per_stage.get)

    K = args.steps
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with B.KernelTrace(K, only=dominant, device=dev) as dom:
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        e0.record(stream)
        for _ in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
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

    gemm_flop = 3 * 2 * T * D * N
    tflops = gemm_flop / (ms_step / 1e3) / 1e12
    tokens_per_s = T / (ms_step / 1e3)
    kernels = {}
    for name, ms in per_stage.items():
        kd, amt = work[name]
        rate = amt / (ms / 1e3)
        kernels[name] = {"us": round(ms * 1e3, 2),
                         ("TFLOP/s" if kd == "mfma" else "GB/s"):
                             round(rate / (1e12 if kd == "mfma" else 1e9), 1),
                         "frac": round(rate / (PEAK_FP8_FLOPS if kd == "mfma" else PEAK_HBM_BYTES), 4)}

    out = {
        "metric": METRIC,
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
        "config": {"workload": args.workload, "tokens": T, "n_seq": n_seq, "seq_len": S,
                   "d_model": D, "n_heads": H, "d_qk": dqk, "d_v": dvw, "packed_n": N,
                   "step": "pack_quantize_weights + qkv_forward + qkv_backward",
                   "seed": args.seed},
        "tflops": round(tflops, 1),
        "pct_fp8_peak": round(100 * tflops * 1e12 / PEAK_FP8_FLOPS, 2),
        "wall_ms_per_step": round(t_wall * 1e3 / K, 4),
        "roofline": {"kernel": dominant, "bound": kind, "achieved": round(achieved, 1),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "launches": len(dom_ms),
                     "avg_us": round(dom_avg_s * 1e6, 2)},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.seed, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
