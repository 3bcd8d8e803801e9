"""Seeded synthetic inputs and workload shapes.

This module is shared by the GPU path's tests/benchmark and by the CPU
oracle's tests.  It holds none of the method's arithmetic: it only draws
normal samples with numpy's PCG64 generator and casts them to the input
dtypes (bf16 through torch's round-to-nearest-even cast).

Workloads (the pages train a GPT on token streams that are not available
here; these shapes and distributions stand in for them):

* ``tiny``     : one sequence of 256 tokens, D=128, one head (W_packed 128x320)
* ``fwd_16k``  : D=768, 6 heads, 8 sequences x 2048 tokens, forward only
* ``step_64k`` : D=768, 6 heads, one sequence of 65536 tokens, forward+backward
* ``sweep_64`` / ``sweep_128``: ``step_64k`` with d_qk = 64 or 128

FP8 ReLU^2 MLP workloads (``MLP_WORKLOADS``): ``mlp_tiny`` (256 tokens,
D=128, d_ff=512) and ``mlp_64k`` (65536 tokens, D=768, d_ff=3072, the MLP
of the block whose attention projection is ``step_64k``).  W1 [D][d_ff] ~
N(0, 1/D), W2 [d_ff][D] ~ N(0, 1/d_ff) (fan-in), both from seed base+1 in
that order; dy [T][D] ~ N(0, 1e-2) as bf16.

x ~ N(0, 1) as bf16; W ~ N(0, 1/D) as fp32 (one draw of the whole [D][N]
packed matrix, handed over as three strided column blocks); the upstream
gradients dq, dk, dv ~ N(0, 1e-2) (variance 1e-2, std 0.1) as bf16.
Per tensor the seed is base+0 (x), base+1 (W), base+2 (gradients).
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "tiny": dict(n_seq=1, seq_len=256, d_model=128, n_heads=1, d_qk=96, d_v=128),
    "fwd_16k": dict(n_seq=8, seq_len=2048, d_model=768, n_heads=6, d_qk=96, d_v=128),
    "step_64k": dict(n_seq=1, seq_len=65536, d_model=768, n_heads=6, d_qk=96, d_v=128),
    "sweep_64": dict(n_seq=1, seq_len=65536, d_model=768, n_heads=6, d_qk=64, d_v=128),
    "sweep_128": dict(n_seq=1, seq_len=65536, d_model=768, n_heads=6, d_qk=128, d_v=128),
}

MLP_WORKLOADS = {
    "mlp_tiny": dict(n_seq=1, seq_len=256, d_model=128, d_ff=512),
    "mlp_64k": dict(n_seq=1, seq_len=65536, d_model=768, d_ff=3072),
}

EPS = 1e-6
ROPE_BASE = 10000.0


def dims_of(w: dict, eps: float = EPS, rope_base: float = ROPE_BASE) -> dict:
    return dict(d_model=w["d_model"], n_heads=w["n_heads"], d_qk=w["d_qk"],
                d_v=w["d_v"], eps=eps, rope_base=rope_base)


def packed_width(w: dict) -> int:
    return w["n_heads"] * (2 * w["d_qk"] + w["d_v"])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns through torch's cast (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def make_x(w: dict, seed: int, tokens: int | None = None) -> np.ndarray:
    T = w["n_seq"] * w["seq_len"] if tokens is None else tokens
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, w["d_model"]), dtype=np.float32)
    return f32_to_bf16_bits(x)


def make_w(w: dict, seed: int) -> np.ndarray:
    """[D][N] fp32 packed weight, N(0, 1/D)."""
    D = w["d_model"]
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((D, packed_width(w)), dtype=np.float32)
    return (W * np.float32(1.0 / np.sqrt(D))).astype(np.float32)


def split_w(w: dict, W: np.ndarray):
    """Three strided views [D][H*d_qk], [D][H*d_qk], [D][H*d_v] of W."""
    nq = w["n_heads"] * w["d_qk"]
    return W[:, :nq], W[:, nq:2 * nq], W[:, 2 * nq:]


def make_dy(w: dict, seed: int):
    """Upstream gradients in head-major layout, bf16 patterns."""
    n, H, S = w["n_seq"], w["n_heads"], w["seq_len"]
    rng = np.random.default_rng(seed)
    std = np.float32(0.1)
    dq = rng.standard_normal((n, H, S, w["d_qk"]), dtype=np.float32) * std
    dk = rng.standard_normal((n, H, S, w["d_qk"]), dtype=np.float32) * std
    dv = rng.standard_normal((n, H, S, w["d_v"]), dtype=np.float32) * std
    return f32_to_bf16_bits(dq), f32_to_bf16_bits(dk), f32_to_bf16_bits(dv)


def make_all(w: dict, seed: int = 42):
    return dict(x=make_x(w, seed), W=make_w(w, seed + 1), dy=make_dy(w, seed + 2))


def make_mlp_w(w: dict, seed: int):
    """W1 [D][d_ff] ~ N(0, 1/D) and W2 [d_ff][D] ~ N(0, 1/d_ff), fp32."""
    D, F = w["d_model"], w["d_ff"]
    rng = np.random.default_rng(seed)
    w1 = rng.standard_normal((D, F), dtype=np.float32) * np.float32(1.0 / np.sqrt(D))
    w2 = rng.standard_normal((F, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(F))
    return w1.astype(np.float32), w2.astype(np.float32)


def make_mlp_dy(w: dict, seed: int, tokens: int | None = None) -> np.ndarray:
    """Upstream gradient of the MLP output, [T][D] bf16 patterns, std 0.1."""
    T = w["n_seq"] * w["seq_len"] if tokens is None else tokens
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((T, w["d_model"]), dtype=np.float32) * np.float32(0.1)
    return f32_to_bf16_bits(dy)
