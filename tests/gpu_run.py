"""Helpers for the GPU parity tests: run the HIP path through the C interface
on seeded inputs and return every stage's output as numpy arrays (bf16 as
uint16 bit patterns), plus tolerance helpers.  Imports no oracle code."""
from __future__ import annotations

import sys

import numpy as np
import torch

from fp8_packed_reduced_amd import binding as B
from fp8_packed_reduced_amd import inputs

EPS = inputs.EPS
BASE = inputs.ROPE_BASE


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dims_for(w: dict, qk_stride: int = 0, grad_format: int = 0, bwd_passes: int = 0):
    return B.make_dims(w["d_model"], w["n_heads"], w["d_qk"], w["d_v"], EPS, BASE, qk_stride,
                       grad_format, bwd_passes)


def pad_rows(a: np.ndarray, width: int, fill: int) -> np.ndarray:
    """bf16 bit rows widened to `width` columns of `fill` bits."""
    out = np.full(a.shape[:-1] + (width,), fill, dtype=np.uint16)
    out[..., :a.shape[-1]] = a
    return out


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def unblock_rows(buf, off: int, rows: int, cols: int, lay) -> np.ndarray:
    """[rows_pad][cols_pad] bytes from the row-blocked FP8 layout: blocks of
    act_block_rows x k_block bytes, ceil(cols / k_block) blocks per block row."""
    R, KB = lay.act_block_rows, lay.k_block
    nb, kc = _ceil(rows, R), _ceil(cols, KB)
    a = B.view_bytes(buf, off, (nb, kc, R, KB), torch.uint8).cpu().numpy()
    return a.transpose(0, 2, 1, 3).reshape(nb * R, kc * KB)


def run(w: dict, seed: int = 42, x_bits=None, W=None, dy=None, backward: bool = True,
        qk_stride: int = 0, grad_format: int = 0, bwd_passes: int = 0,
        pack_forward: bool = False):
    """Pack, forward (and backward) on the GPU; returns a dict of numpy arrays.

    With qk_stride > d_qk, q and k come back with their padded rows (the
    output buffers start filled with NaN bits, so the padding seen is what
    the kernels wrote) and dq, dk (given or drawn at d_qk) go in padded with
    NaN bits, which the backward must never read.  grad_format 1 quantises the
    packed gradient to e5m2.  bwd_passes 2 runs the two-pass backward, which
    never writes dQK (then "dqkv" is None).  pack_forward packs the weights
    and runs the forward in one qkv_pack_forward call, on a cache whose
    status word starts with every bit set (the call must clear it); its
    pre-norm rows are not returned ("qk_pre" is None)."""
    n_seq, S = w["n_seq"], w["seq_len"]
    T = n_seq * S
    D, H, dqk, dv = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    N = inputs.packed_width(w)
    dims = dims_for(w, qk_stride, grad_format, bwd_passes)
    qs = qk_stride or dqk
    say(f"[gpu] run n_seq={n_seq} S={S} D={D} H={H} d_qk={dqk} d_v={dv} stride={qs} "
        f"grad_format={grad_format} bwd_passes={bwd_passes} pack_forward={pack_forward} "
        f"seed={seed}")
    if x_bits is None:
        x_bits = inputs.make_x(w, seed)
    if W is None:
        W = inputs.make_w(w, seed + 1)
    Wd = torch.from_numpy(np.ascontiguousarray(W)).cuda()
    nq = H * dqk
    wq, wk, wv = Wd[:, :nq], Wd[:, nq:2 * nq], Wd[:, 2 * nq:]
    cache = B.WeightCache(dims)
    x = bits_to_dev(x_bits)
    qo = ko = None
    if qs != dqk:
        qo, ko = (torch.full((n_seq, H, S, qs), -1, dtype=torch.int16, device="cuda")
                  .view(torch.bfloat16) for _ in range(2))
    if pack_forward:
        cache.status.fill_(-1)
        ws_f = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_PACK_FORWARD),
                           dtype=torch.uint8, device="cuda")
        q, k, v, saved = B.qkv_pack_forward(dims, wq, wk, wv, cache, n_seq, S, x, q=qo, k=ko,
                                            workspace=ws_f)
    else:
        B.pack_quantize_weights(dims, wq, wk, wv, cache)
        ws_f = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_FORWARD), dtype=torch.uint8,
                           device="cuda")
        q, k, v, saved = B.qkv_forward(dims, n_seq, S, x, cache, q=qo, k=ko, workspace=ws_f)
    lay = B.layout(dims, T)
    Tp = lay.tokens_padded
    out = dict(T=T, N=N, Tp=Tp, x_bits=x_bits, W=W)
    torch.cuda.synchronize()
    out["w_packed"] = cache.w_packed.cpu().numpy()
    out["w_packed_t"] = cache.w_packed_t.cpu().numpy()
    out["w_scales"] = cache.scales.cpu().numpy()
    x8 = unblock_rows(saved, lay.saved_x8, T, D, lay)
    # x8_tail: the zero token rows T .. Tp - 1 that the dW GEMM reads as its K tail
    out["x8"], out["x8_kpad"], out["x8_tail"] = x8[:T, :D], x8[:T, D:], x8[T:Tp]
    out["x_scales"] = B.view_bytes(saved, lay.saved_x_scales, (2,), torch.float32).cpu().numpy()
    # 1/rms of every q, then every k head row: [2][n_seq][H][S]
    out["rho"] = B.view_bytes(saved, lay.saved_rho, (2, n_seq, H, S), torch.float32).cpu().numpy()
    # the pre-norm Q|K rows exist only where the norm/RoPE is not fused into
    # the forward GEMM (then in the forward workspace)
    out["fused"] = lay.fused_forward
    out["qk_pre"] = None if lay.fused_forward or pack_forward else dev_to_bits(
        B.view_bytes(ws_f, lay.fwd_qk_pre, (T, 2 * nq), torch.bfloat16))
    out["q"], out["k"], out["v"] = dev_to_bits(q), dev_to_bits(k), dev_to_bits(v)
    if backward:
        if dy is None:
            dy = inputs.make_dy(w, seed + 2)
        dqd, dkd, dvd = (bits_to_dev(pad_rows(a, qs, 0xFFFF) if i < 2 and qs != dqk else a)
                         for i, a in enumerate(dy))
        ws_b = torch.empty(B.workspace_bytes(dims, T, B.FPR_CALL_BACKWARD), dtype=torch.uint8,
                           device="cuda")
        dx, dw = B.qkv_backward(dims, n_seq, S, q, k, dqd, dkd, dvd, saved, cache,
                                workspace=ws_b)
        torch.cuda.synchronize()
        out["dy"] = dy
        # the packed gradient: its Q|K part from the workspace, its V part is
        # dv itself (the gradient quantiser reads it head-major)
        out["dqkv"] = None
        if lay.bwd_dqkv != B.NOT_PRESENT:
            gqk = dev_to_bits(B.view_bytes(ws_b, lay.bwd_dqkv, (T, 2 * nq), torch.bfloat16))
            dvt = np.ascontiguousarray(np.asarray(dy[2]).transpose(0, 2, 1, 3)).reshape(T, H * dv)
            out["dqkv"] = np.concatenate([gqk, dvt], axis=1)
        out["g_scales"] = B.view_bytes(ws_b, lay.bwd_g_scales, (2,), torch.float32).cpu().numpy()
        g8 = unblock_rows(ws_b, lay.bwd_g8, T, N, lay)
        out["g8"], out["g8_kpad"], out["g8_tail"] = g8[:T, :N], g8[:T, N:], g8[T:Tp]
        out["dx"] = dev_to_bits(dx)
        out["dw"] = dw.cpu().numpy()
    out["status"] = int(cache.status.cpu().item())
    say("[gpu] done")
    return out


def rho_rows(rho: np.ndarray) -> np.ndarray:
    """[2][n_seq][H][S] (q rows, then k rows) -> [T][2H] in packed head order."""
    two, n_seq, H, S = rho.shape
    return np.ascontiguousarray(rho.transpose(1, 3, 0, 2)).reshape(n_seq * S, 2 * H)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max over rows of ||got - want|| / ||want|| (rows = all but the last axis)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    o = np.asarray(want, dtype=np.float64).reshape(-1, want.shape[-1])
    num = np.linalg.norm(g - o, axis=1)
    den = np.linalg.norm(o, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0


def row_errors(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Per-row ||got - want|| / ||want|| (rows = all but the last axis)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    o = np.asarray(want, dtype=np.float64).reshape(-1, want.shape[-1])
    den = np.linalg.norm(o, axis=1)
    return np.linalg.norm(g - o, axis=1) / np.where(den == 0, 1.0, den)


def bf16_gemm_excess(gpu_bits: np.ndarray, exact: np.ndarray, round_bf16) -> tuple[float, float]:
    """For a GEMM whose output is bf16: per row, the GPU's distance to the
    exact float64 product against the distance that rounding the exact
    product to bf16 costs by itself.  Returns (worst gpu / rounding ratio
    excess, worst gpu - 1.1 * rounding) so a test can require
    e_gpu <= 1.1 * e_round + 1e-3 on every row."""
    e_gpu = row_errors(bf16_to_f64(gpu_bits), exact)
    e_rnd = row_errors(bf16_to_f64(round_bf16(exact)), exact)
    return float(np.max(e_gpu - e_rnd)), float(np.max(e_gpu - 1.1 * e_rnd))


# ------------------------------------------------------- FP8 ReLU^2 MLP

def run_mlp(w: dict, seed: int = 42, x_bits=None, w12=None, dy_bits=None,
            backward: bool = True, grad_format: int = 0, pack_forward: bool = False):
    """Pack, forward (and backward) of the FP8 ReLU^2 MLP on the GPU; every
    stage's output as numpy arrays (bf16 as uint16 patterns).  pack_forward
    packs and runs the forward in one mlp_pack_forward call, on a cache
    whose status word starts with every bit set; h is then not returned."""
    T = w["n_seq"] * w["seq_len"]
    D, F = w["d_model"], w["d_ff"]
    say(f"[gpu] mlp T={T} D={D} F={F} grad_format={grad_format} pack_forward={pack_forward} "
        f"seed={seed}")
    if x_bits is None:
        x_bits = inputs.make_x(w, seed)
    if w12 is None:
        w12 = inputs.make_mlp_w(w, seed + 1)
    dims = B.MlpDims(D, F, grad_format)
    cache = B.MlpCache(dims)
    w1d, w2d = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in w12)
    if pack_forward:
        cache.status.fill_(-1)
        ws_f = torch.empty(B.mlp_workspace_bytes(dims, T, B.FPR_CALL_PACK_FORWARD),
                           dtype=torch.uint8, device="cuda")
        y, saved = B.mlp_pack_forward(dims, w1d, w2d, cache, bits_to_dev(x_bits), workspace=ws_f)
    else:
        B.mlp_pack_quantize_weights(dims, w1d, w2d, cache)
        ws_f = torch.empty(B.mlp_workspace_bytes(dims, T, B.FPR_CALL_FORWARD),
                           dtype=torch.uint8, device="cuda")
        y, saved = B.mlp_forward(dims, bits_to_dev(x_bits), cache, workspace=ws_f)
    torch.cuda.synchronize()
    lay = B.mlp_layout(dims, T)
    qlay = B.layout(B.make_dims(128, 1), 1)  # the blocked layout's parameters

    class _L:
        act_block_rows, k_block = qlay.act_block_rows, qlay.k_block

    Tp = lay.tokens_padded
    out = dict(T=T, Tp=Tp, x_bits=x_bits, w1=w12[0], w2=w12[1])
    for k in ("w1", "w1_t", "w2", "w2_t"):
        out["c_" + k] = getattr(cache, k).cpu().numpy()
    out["w_scales"] = cache.scales.cpu().numpy()
    x8 = unblock_rows(saved, lay.saved_x8, T, D, _L)
    h8 = unblock_rows(saved, lay.saved_h8, T, F, _L)
    out["x8"], out["x8_tail"] = x8[:T, :D], x8[T:Tp]
    out["h8"], out["h8_tail"] = h8[:T, :F], h8[T:Tp]
    out["x_scales"] = B.view_bytes(saved, lay.saved_x_scales, (2,), torch.float32).cpu().numpy()
    out["h_scales"] = B.view_bytes(saved, lay.saved_h_scales, (2,), torch.float32).cpu().numpy()
    out["h"] = None if pack_forward else dev_to_bits(
        B.view_bytes(ws_f, lay.fwd_h, (T, F), torch.bfloat16))
    out["y"] = dev_to_bits(y)
    if backward:
        if dy_bits is None:
            dy_bits = inputs.make_mlp_dy(w, seed + 2)
        ws_b = torch.empty(B.mlp_workspace_bytes(dims, T, B.FPR_CALL_BACKWARD),
                           dtype=torch.uint8, device="cuda")
        dx, dw1, dw2 = B.mlp_backward(dims, bits_to_dev(dy_bits), saved, cache, workspace=ws_b)
        torch.cuda.synchronize()
        out["dy"] = dy_bits
        dy8 = unblock_rows(ws_b, lay.bwd_dy8, T, D, _L)
        dp8 = unblock_rows(ws_b, lay.bwd_dpre8, T, F, _L)
        out["dy8"], out["dp8"], out["dp8_tail"] = dy8[:T, :D], dp8[:T, :F], dp8[T:Tp]
        out["dy_scales"] = B.view_bytes(ws_b, lay.bwd_dy_scales, (2,), torch.float32).cpu().numpy()
        out["dp_scales"] = B.view_bytes(ws_b, lay.bwd_dpre_scales, (2,),
                                        torch.float32).cpu().numpy()
        out["dpre"] = dev_to_bits(B.view_bytes(ws_b, lay.bwd_dpre, (T, F), torch.bfloat16))
        out["dx"] = dev_to_bits(dx)
        out["dw1"], out["dw2"] = dw1.cpu().numpy(), dw2.cpu().numpy()
    out["status"] = int(cache.status.cpu().item())
    say("[gpu] mlp done")
    return out
