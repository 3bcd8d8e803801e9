"""ORACLE -- TEST INFRASTRUCTURE ONLY.

A plain, slow, CPU reference for the packed FP8 QKV projection with
reduced-width Q/K heads.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the GPU library (``fp8_packed_reduced_amd``) and never
imports it; the two meet only in the seeded input generators.

What is computed, and where the pages say so:

* "96 is enough: shrinking attention's routing vectors", section "The
  change": Q/K heads 96 wide, V 128 wide, ``W_packed = [W_q | W_k | W_v]``
  (320 columns per head), one FP8 matmul ``qkv = x @ W_packed``, split into
  q, k, v, RMS-normalise q and k, then rotate them with RoPE.
* PR #344 page, section "Changes": both FP8 layouts of the packed weight come
  out of one weight read; quantisation of the logical Q/K and V packs with no
  concatenation; norm, RoPE and layout conversion fused; FP8 backward.
* "Where the eight seconds were hiding", section "The inventory": the
  transposed weight view is cached and reused by the backward pass.
* PR #344 page, section "Changes": the FP8 ReLU-squared MLP, forward and
  backward, pre not kept and relu(pre) recovered as sqrt(s_h dec(h8))
  (``mlp_forward`` / ``mlp_backward``, readings at that section).

Every floating-point step runs in float64.  FP8 codes, scales and bf16/fp32
output roundings are the only reduced-precision steps, and they are the
definitions the GPU path must reproduce.

Readings where the pages are silent:

* FP8 format: OCP E4M3 (max 448, no inf), round to nearest even, saturating.
* Per-tensor scales: ``s = fl32(amax/448)``, ``inv = fl32(448/amax)``,
  ``code = enc(fl32(v * inv))``; one scale for all of W_packed, one for x,
  one for the packed gradient dQKV (taken over its bf16 values).
* RMSNorm has no learnable gain (only the direction of q and k is used), eps
  inside the square root.
* RoPE on all d_qk dims, rotate-half pairing (i, i + d_qk/2),
  ``theta_i = base^(-2i/d_qk)``, positions 0-based within each sequence.
* Packed column order ``[Q h0..h(H-1) | K h0.. | V h0..]``.
* Output layout head-major ``[n_seq][H][S][d]``, bf16.
* Backward treats both quantisers as the identity (straight-through).

Parity pins live in ``tests/test_oracle_*.py``.  Parity unpinned: the RoPE
pairing convention and the activation/gradient scaling recipe are fixed by
contract only (the pages do not define them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "codec.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C codec with gcc (no fast-math; IEEE rounding matters)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode_table.argtypes = [ctypes.c_void_p]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_search.restype = ctypes.c_uint8
        L.orc_e4m3_encode_search.argtypes = [ctypes.c_float]
        L.orc_e4m3_encoders_disagree.restype = ctypes.c_int64
        L.orc_e4m3_encoders_disagree.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_e4m3_encode_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_quantize_f32.restype = ctypes.c_int
        L.orc_quantize_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.orc_quantize_bf16.restype = ctypes.c_int
        L.orc_quantize_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_void_p]
        L.orc_pack_quantize.restype = ctypes.c_int
        L.orc_pack_quantize.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        L.orc_e5m2_decode.restype = ctypes.c_double
        L.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
        L.orc_e5m2_decode_table.argtypes = [ctypes.c_void_p]
        L.orc_e5m2_encode.restype = ctypes.c_uint8
        L.orc_e5m2_encode.argtypes = [ctypes.c_float]
        L.orc_e5m2_encode_search.restype = ctypes.c_uint8
        L.orc_e5m2_encode_search.argtypes = [ctypes.c_float]
        L.orc_e5m2_encoders_disagree.restype = ctypes.c_int64
        L.orc_e5m2_encoders_disagree.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_e5m2_encode_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_quantize_bf16_e5m2.restype = ctypes.c_int
        L.orc_quantize_bf16_e5m2.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16.argtypes = [ctypes.c_double]
        L.orc_round_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_round_f32_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------- codec

def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3 codes (NaN for 0x7F, 0xFF)."""
    t = np.empty(256, dtype=np.float64)
    lib().orc_e4m3_decode_table(_ptr(t))
    return t


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return e4m3_decode_table()[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Nearest e4m3 code of each fp32 value (arithmetic encoder)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode_search_scalar(v: float) -> int:
    return int(lib().orc_e4m3_encode_search(ctypes.c_float(v)))


def e4m3_encoders_disagree(begin: int, end: int):
    """(count, first bad fp32 pattern) of the two encoders over [begin, end)."""
    first = ctypes.c_uint32(0)
    n = lib().orc_e4m3_encoders_disagree(begin, end, ctypes.byref(first))
    return int(n), int(first.value)


def e5m2_decode_table() -> np.ndarray:
    """float64 value of each of the 256 e5m2 codes (+-inf, NaN included)."""
    t = np.empty(256, dtype=np.float64)
    lib().orc_e5m2_decode_table(_ptr(t))
    return t


def e5m2_decode(codes: np.ndarray) -> np.ndarray:
    return e5m2_decode_table()[np.asarray(codes, dtype=np.uint8)]


def e5m2_encode(v) -> np.ndarray:
    """Nearest e5m2 code of each fp32 value (arithmetic encoder)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e5m2_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e5m2_encode_search_scalar(v: float) -> int:
    return int(lib().orc_e5m2_encode_search(ctypes.c_float(v)))


def e5m2_encoders_disagree(begin: int, end: int):
    """(count, first bad fp32 pattern) of the two e5m2 encoders over [begin, end)."""
    first = ctypes.c_uint32(0)
    n = lib().orc_e5m2_encoders_disagree(begin, end, ctypes.byref(first))
    return int(n), int(first.value)


def decode_table(fmt: str) -> np.ndarray:
    return {"e4m3": e4m3_decode_table, "e5m2": e5m2_decode_table}[fmt]()


def quantize_f32(v: np.ndarray):
    """Per-tensor e4m3 quantisation of fp32 values -> (codes, s, inv, rc)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    codes = np.empty(v.shape, dtype=np.uint8)
    sc = np.empty(2, dtype=np.float32)
    rc = lib().orc_quantize_f32(_ptr(v), v.size, _ptr(codes), _ptr(sc))
    return codes, np.float32(sc[0]), np.float32(sc[1]), int(rc)


def quantize_bf16(bits: np.ndarray, fmt: str = "e4m3"):
    """Per-tensor e4m3 (or e5m2) quantisation of bf16 values given as uint16
    patterns -> (codes, s, inv, rc)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    codes = np.empty(bits.shape, dtype=np.uint8)
    sc = np.empty(2, dtype=np.float32)
    fn = {"e4m3": lib().orc_quantize_bf16, "e5m2": lib().orc_quantize_bf16_e5m2}[fmt]
    rc = fn(_ptr(bits), bits.size, _ptr(codes), _ptr(sc))
    return codes, np.float32(sc[0]), np.float32(sc[1]), int(rc)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even, one rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_round_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float32)
    lib().orc_round_f32_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bf16 pattern is the top half of an fp32 pattern."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------- packed weights

def packed_columns(H: int, d_qk: int, d_v: int):
    """Column ranges of the logical W_packed: (q0, k0, v0, N)."""
    nq = H * d_qk
    return 0, nq, 2 * nq, 2 * nq + H * d_v


def pack_quantize(D, H, d_qk, d_v, wq, wk, wv):
    """Quantise the logical W_packed = [W_q | W_k | W_v] (each [D][cols] fp32,
    row-major, any row stride) with one scale, emitting both layouts.

    Returns (w_packed [D][N] uint8, w_packed_t [N][D] uint8, s, inv, rc)."""
    N = packed_columns(H, d_qk, d_v)[3]
    views = []
    for w, cols in ((wq, H * d_qk), (wk, H * d_qk), (wv, H * d_v)):
        w = np.asarray(w, dtype=np.float32)
        assert w.shape == (D, cols) and w.strides[1] == 4
        views.append(w)
    w_packed = np.empty((D, N), dtype=np.uint8)
    w_packed_t = np.empty((N, D), dtype=np.uint8)
    sc = np.empty(2, dtype=np.float32)
    rc = lib().orc_pack_quantize(
        D, H, d_qk, d_v,
        ctypes.c_void_p(views[0].ctypes.data), views[0].strides[0] // 4,
        ctypes.c_void_p(views[1].ctypes.data), views[1].strides[0] // 4,
        ctypes.c_void_p(views[2].ctypes.data), views[2].strides[0] // 4,
        _ptr(w_packed), _ptr(w_packed_t), _ptr(sc))
    return w_packed, w_packed_t, np.float32(sc[0]), np.float32(sc[1]), int(rc)


# ------------------------------------------------------------------ GEMM

def gemm_e4m3(a_codes: np.ndarray, b_codes: np.ndarray, s_a, s_b, a_fmt: str = "e4m3",
              b_fmt: str = "e4m3") -> np.ndarray:
    """C = s_a * s_b * dec(A) @ dec(B) in float64 ("96 is enough", "The
    change": Y = x W_packed as one FP8 product).  A is [M][K], B is [K][N]; each
    operand's codes are e4m3 unless its format says e5m2."""
    A = decode_table(a_fmt)[a_codes]
    B = decode_table(b_fmt)[b_codes]
    return (float(s_a) * float(s_b)) * (A @ B)


# ------------------------------------------------------- RMSNorm, RoPE

def rmsnorm(a: np.ndarray, eps: float):
    """u = a / sqrt(mean(a^2) + eps) over the last axis; returns (u, rho)."""
    ms = np.mean(a * a, axis=-1, keepdims=True)
    rho = 1.0 / np.sqrt(ms + eps)
    return a * rho, rho


def rope_cos_sin(positions: np.ndarray, d: int, base: float):
    """cos, sin of p * theta_i for theta_i = base^(-2i/d), i < d/2."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(phi), np.sin(phi)


def rope(u: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate pairs (i, i + d/2) of the last axis by p * theta_i.
    u has shape [T, R, d]; positions has shape [T]."""
    d = u.shape[-1]
    h = d // 2
    c, s = rope_cos_sin(positions, d, base)
    c = c[:, None, :]
    s = s[:, None, :]
    x, y = u[..., :h], u[..., h:]
    return np.concatenate([x * c - y * s, y * c + x * s], axis=-1)


def rope_inverse(g: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Apply the inverse (= transpose) rotation R_{-p}."""
    return rope(g, -np.asarray(positions, dtype=np.float64), base)


def qk_norm_rope_fwd(a: np.ndarray, positions, eps: float, base: float) -> np.ndarray:
    """a: [T, R, d] pre-norm q/k head rows -> rope(rmsnorm(a))."""
    u, _ = rmsnorm(a, eps)
    return rope(u, positions, base)


def qk_norm_rope_bwd(a: np.ndarray, dout: np.ndarray, positions, eps: float,
                     base: float) -> np.ndarray:
    """Gradient w.r.t. a of rope(rmsnorm(a)):
    du = R_{-p} dout;  da = rho * (du - u * <u, du> / d)."""
    d = a.shape[-1]
    u, rho = rmsnorm(a, eps)
    du = rope_inverse(dout, positions, base)
    dot = np.sum(u * du, axis=-1, keepdims=True)
    return rho * (du - u * dot / d)


# ------------------------------------------------------------ the chain

def positions_of(n_seq: int, S: int) -> np.ndarray:
    """Token t = b*S + s sits at position s of sequence b."""
    return np.tile(np.arange(S, dtype=np.int64), n_seq)


def to_head_major(rows: np.ndarray, n_seq: int, S: int) -> np.ndarray:
    """[T, H, d] token-major -> [n_seq, H, S, d] head-major."""
    T, H, d = rows.shape
    return np.ascontiguousarray(rows.reshape(n_seq, S, H, d).transpose(0, 2, 1, 3))


def from_head_major(x: np.ndarray) -> np.ndarray:
    """[n_seq, H, S, d] -> [T, H, d]."""
    n_seq, H, S, d = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(n_seq * S, H, d))


def pack_quantize_weights(dims, w_packed_f32: np.ndarray):
    """Convenience: split a [D][N] fp32 packed weight into its three logical
    pieces (as strided views) and quantise them."""
    D, H, d_qk, d_v = dims["d_model"], dims["n_heads"], dims["d_qk"], dims["d_v"]
    _, k0, v0, N = packed_columns(H, d_qk, d_v)
    W = np.asarray(w_packed_f32, dtype=np.float32)
    return pack_quantize(D, H, d_qk, d_v, W[:, :k0], W[:, k0:v0], W[:, v0:N])


def qkv_forward(dims, n_seq: int, S: int, x_bits: np.ndarray,
                w_packed: np.ndarray, s_w, y_bits: np.ndarray | None = None):
    """Forward chain.  x_bits: [T][D] bf16 patterns.  w_packed: [D][N] codes.

    Returns a dict of every intermediate.  If ``y_bits`` ([T][N] bf16) is
    given, the epilogue stage is fed those values instead of the oracle's own
    GEMM output (stage-wise comparison)."""
    H, d_qk, d_v = dims["n_heads"], dims["d_qk"], dims["d_v"]
    eps, base = dims["eps"], dims["rope_base"]
    _, k0, v0, N = packed_columns(H, d_qk, d_v)
    T = n_seq * S
    x8, s_x, inv_x, rc_x = quantize_bf16(x_bits)
    out = {"x8": x8, "s_x": s_x, "inv_x": inv_x, "rc_x": rc_x}
    if y_bits is None:
        y64 = gemm_e4m3(x8, w_packed, s_x, s_w)
        out["y64"] = y64
        y_bits = round_bf16(y64)
    out["y_bits"] = y_bits
    y = bf16_to_f64(y_bits)
    pos = positions_of(n_seq, S)
    qpre = y[:, :k0].reshape(T, H, d_qk)
    kpre = y[:, k0:v0].reshape(T, H, d_qk)
    vrow = y[:, v0:N].reshape(T, H, d_v)
    q64 = qk_norm_rope_fwd(qpre, pos, eps, base)
    k64 = qk_norm_rope_fwd(kpre, pos, eps, base)
    out["q64"] = to_head_major(q64, n_seq, S)
    out["k64"] = to_head_major(k64, n_seq, S)
    out["q_bits"] = round_bf16(out["q64"])
    out["k_bits"] = round_bf16(out["k64"])
    out["v_bits"] = to_head_major(y_bits[:, v0:N].reshape(T, H, d_v), n_seq, S)
    out["v64"] = to_head_major(vrow, n_seq, S)
    return out


def qkv_backward(dims, n_seq: int, S: int, dq_bits, dk_bits, dv_bits,
                 x8: np.ndarray, s_x, qk_pre_bits: np.ndarray,
                 w_packed: np.ndarray, s_w, dqkv_bits: np.ndarray | None = None,
                 grad_fmt: str = "e4m3"):
    """Backward chain.  dq/dk/dv: head-major bf16 patterns.  qk_pre_bits:
    [T][2*H*d_qk] bf16 pre-norm Q|K (saved by the forward).  If
    ``dqkv_bits`` is given, the GEMM stages are fed it instead of the
    oracle's own packed gradient (stage-wise comparison).  ``grad_fmt``
    "e5m2" quantises the packed gradient to e5m2 instead of e4m3."""
    H, d_qk, d_v = dims["n_heads"], dims["d_qk"], dims["d_v"]
    eps, base = dims["eps"], dims["rope_base"]
    _, k0, v0, N = packed_columns(H, d_qk, d_v)
    T = n_seq * S
    out = {}
    if dqkv_bits is None:
        pos = positions_of(n_seq, S)
        a = bf16_to_f64(qk_pre_bits)
        qpre = a[:, :k0].reshape(T, H, d_qk)
        kpre = a[:, k0:v0].reshape(T, H, d_qk)
        dq = from_head_major(bf16_to_f64(dq_bits))
        dk = from_head_major(bf16_to_f64(dk_bits))
        dv = from_head_major(bf16_to_f64(dv_bits))
        dqpre = qk_norm_rope_bwd(qpre, dq, pos, eps, base)
        dkpre = qk_norm_rope_bwd(kpre, dk, pos, eps, base)
        dqkv64 = np.concatenate(
            [dqpre.reshape(T, k0), dkpre.reshape(T, v0 - k0), dv.reshape(T, N - v0)],
            axis=1)
        out["dqkv64"] = dqkv64
        dqkv_bits = round_bf16(dqkv64)
    out["dqkv_bits"] = dqkv_bits
    g8, s_g, inv_g, rc_g = quantize_bf16(dqkv_bits, grad_fmt)
    out.update(g8=g8, s_g=s_g, inv_g=inv_g, rc_g=rc_g)
    # dX = dQKV @ W_packed^T, through the cached [D][N] codes
    dx64 = gemm_e4m3(g8, np.ascontiguousarray(w_packed.T), s_g, s_w, a_fmt=grad_fmt)
    out["dx64"] = dx64
    out["dx_bits"] = round_bf16(dx64)
    # dW = x^T @ dQKV
    dw64 = gemm_e4m3(np.ascontiguousarray(x8.T), g8, s_x, s_g, b_fmt=grad_fmt)
    out["dw64"] = dw64
    out["dw_f32"] = round_f32(dw64)
    return out


# ------------------------------------------------------ FP8 ReLU^2 MLP
#
# PR #344 page, "Changes": FP8 covers the whole ReLU-squared MLP, forward
# and backward, both projections and all four backward GEMMs; pre is not
# kept: the backward recovers relu(pre) from the squared activation.
# Readings where the page is silent: W1 is [D][F] and W2 is [F][D]
# (y = relu(x W1)^2 W2), one per-tensor e4m3 scale per tensor exactly as for
# the QKV path, and the kept h^2 is its e4m3 copy h8 with
# scale s_h, which the second projection and dW2 read anyway, so
# relu(pre) = sqrt(s_h dec(h8)).  The bf16 h that the quantiser reads is
# relu(pre)^2 rounded once.

def relu2(pre: np.ndarray) -> np.ndarray:
    """h = relu(pre)^2."""
    r = np.maximum(pre, 0.0)
    return r * r


def relu2_grad(dh: np.ndarray, h: np.ndarray) -> np.ndarray:
    """d relu(pre)^2 / d pre = 2 relu(pre), with relu(pre) = sqrt(h):
    dpre = 2 dh sqrt(h)."""
    return 2.0 * dh * np.sqrt(h)


def mlp_quantize_weights(w1: np.ndarray, w2: np.ndarray):
    """Per-tensor e4m3 codes of W1 [D][F] and W2 [F][D] in both layouts."""
    c1, s1, i1, rc1 = quantize_f32(w1)
    c2, s2, i2, rc2 = quantize_f32(w2)
    return dict(w1=c1, w1t=np.ascontiguousarray(c1.T), s_w1=s1, inv_w1=i1,
                w2=c2, w2t=np.ascontiguousarray(c2.T), s_w2=s2, inv_w2=i2, rc=rc1 | rc2)


def mlp_forward(x_bits: np.ndarray, wq: dict, h_bits: np.ndarray | None = None):
    """x_bits [T][D] bf16 -> y = fp8(h) @ fp8(W2), h = relu(fp8(x) @ fp8(W1))^2.

    If ``h_bits`` ([T][F] bf16) is given, the second projection is fed those
    values instead of the oracle's own (stage-wise comparison)."""
    x8, s_x, inv_x, rc_x = quantize_bf16(x_bits)
    out = dict(x8=x8, s_x=s_x, inv_x=inv_x, rc_x=rc_x)
    if h_bits is None:
        pre64 = gemm_e4m3(x8, wq["w1"], s_x, wq["s_w1"])
        out["pre64"] = pre64
        out["h64"] = relu2(pre64)
        h_bits = round_bf16(out["h64"])
    out["h_bits"] = h_bits
    h8, s_h, inv_h, rc_h = quantize_bf16(h_bits)
    out.update(h8=h8, s_h=s_h, inv_h=inv_h, rc_h=rc_h)
    y64 = gemm_e4m3(h8, wq["w2"], s_h, wq["s_w2"])
    out["y64"] = y64
    out["y_bits"] = round_bf16(y64)
    return out


def mlp_backward(dy_bits: np.ndarray, x8: np.ndarray, s_x, h8: np.ndarray, s_h, wq: dict,
                 dpre_bits: np.ndarray | None = None, grad_fmt: str = "e4m3"):
    """Backward of the FP8 ReLU^2 MLP from the saved x8, h8 and their scales;
    quantisers treated as the identity.

      dh   = dy @ W2^T            (through the cached [F][D] codes of W2)
      dpre = 2 dh sqrt(s_h dec(h8))
      dx   = dpre @ W1^T          (through the cached [D][F] codes of W1)
      dW1  = x^T dpre,  dW2 = h^T dy

    If ``dpre_bits`` is given, the stages after it are fed those values.
    ``grad_fmt`` "e5m2" quantises the gradients dy and dpre to e5m2."""
    g = grad_fmt
    dy8, s_dy, inv_dy, rc_dy = quantize_bf16(dy_bits, g)
    out = dict(dy8=dy8, s_dy=s_dy, inv_dy=inv_dy, rc_dy=rc_dy)
    if dpre_bits is None:
        dh64 = gemm_e4m3(dy8, np.ascontiguousarray(wq["w2"].T), s_dy, wq["s_w2"], a_fmt=g)
        h = float(s_h) * e4m3_decode(h8)
        out["dh64"] = dh64
        out["dpre64"] = relu2_grad(dh64, h)
        dpre_bits = round_bf16(out["dpre64"])
    out["dpre_bits"] = dpre_bits
    dp8, s_dp, inv_dp, rc_dp = quantize_bf16(dpre_bits, g)
    out.update(dp8=dp8, s_dp=s_dp, inv_dp=inv_dp, rc_dp=rc_dp)
    dx64 = gemm_e4m3(dp8, np.ascontiguousarray(wq["w1"].T), s_dp, wq["s_w1"], a_fmt=g)
    out["dx64"] = dx64
    out["dx_bits"] = round_bf16(dx64)
    dw1 = gemm_e4m3(np.ascontiguousarray(x8.T), dp8, s_x, s_dp, b_fmt=g)
    dw2 = gemm_e4m3(np.ascontiguousarray(h8.T), dy8, s_h, s_dy, b_fmt=g)
    out.update(dw1_64=dw1, dw2_64=dw2, dw1_f32=round_f32(dw1), dw2_f32=round_f32(dw2))
    return out
