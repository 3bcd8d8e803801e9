"""Pins of the oracle's FP8 GEMM stages (forward x @ W_packed, dX through the
cached weight codes, dW = x^T dQKV) by brute force on integer-valued inputs
(pure-Python integer sums, exact) and by adjoint identities, which fail for a
transposed or swapped operand."""
import numpy as np
import pytest

import oracle
from fp8_packed_reduced_amd import inputs


def _int_codes(rng, shape, lim=16):
    """Integers in [-lim, lim] (all exact in e4m3 for lim <= 16) and codes."""
    v = rng.integers(-lim, lim + 1, size=shape).astype(np.float32)
    return v, oracle.e4m3_encode(v)


def _brute(a, b):
    M, K = a.shape
    N = b.shape[1]
    ai = a.astype(np.int64).tolist()
    bi = b.astype(np.int64).tolist()
    return np.array([[sum(ai[i][k] * bi[k][j] for k in range(K)) for j in range(N)]
                     for i in range(M)], dtype=np.float64)


def test_gemm_integer_brute_force_exact():
    rng = np.random.default_rng(7)
    a, ac = _int_codes(rng, (9, 40))
    b, bc = _int_codes(rng, (40, 13))
    got = oracle.gemm_e4m3(ac, bc, 1.0, 1.0)
    assert np.array_equal(got, _brute(a, b))
    # the scales multiply through
    got2 = oracle.gemm_e4m3(ac, bc, np.float32(0.5), np.float32(0.25))
    assert np.array_equal(got2, _brute(a, b) / 8)


def test_forward_chain_integer_inputs_exact():
    # x holds small integers plus one 448 (so s_x = 1); W_packed likewise
    # (so s_w = 1).  Then x8, W8 hold the integers exactly and the GEMM output
    # is the exact integer product.
    w = dict(n_seq=1, seq_len=24, d_model=32, n_heads=1, d_qk=32, d_v=32)
    dims = inputs.dims_of(w)
    rng = np.random.default_rng(8)
    x = rng.integers(-16, 17, size=(24, 32)).astype(np.float32)
    x[3, 5] = 448.0
    W = rng.integers(-16, 17, size=(32, 96)).astype(np.float32)
    W[0, 0] = -448.0
    wp, wpt, s_w, inv_w, _ = oracle.pack_quantize_weights(dims, W)
    assert (s_w, inv_w) == (1.0, 1.0)
    out = oracle.qkv_forward(dims, 1, 24, inputs.f32_to_bf16_bits(x), wp, s_w)
    assert out["s_x"] == 1.0
    assert np.array_equal(out["y64"], _brute(x, W))


def test_backward_gemms_integer_inputs_exact():
    w = dict(n_seq=1, seq_len=16, d_model=32, n_heads=1, d_qk=32, d_v=32)
    dims = inputs.dims_of(w)
    rng = np.random.default_rng(9)
    x = rng.integers(-8, 9, size=(16, 32)).astype(np.float32)
    x[0, 0] = 448.0
    W = rng.integers(-8, 9, size=(32, 96)).astype(np.float32)
    W[1, 1] = 448.0
    g = rng.integers(-8, 9, size=(16, 96)).astype(np.float32)
    g[2, 2] = -448.0
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    x8, s_x, _, _ = oracle.quantize_bf16(inputs.f32_to_bf16_bits(x))
    gb = inputs.f32_to_bf16_bits(g)
    z = np.zeros((1, 1, 16, 32), dtype=np.uint16)
    out = oracle.qkv_backward(dims, 1, 16, z, z, z, x8, s_x, None, wp, s_w, dqkv_bits=gb)
    assert out["s_g"] == 1.0
    assert np.array_equal(out["dx64"], _brute(g, W.T))
    assert np.array_equal(out["dw64"], _brute(x.T, g))


def test_adjoint_identities_tie_forward_dx_and_dw():
    # With X = s_x dec(x8), W = s_w dec(w8), G = s_g dec(g8):
    #   Y = X W,  dX = G W^T,  dW = X^T G   =>   <G, Y> = <dX, X> = <dW, W>.
    w = inputs.WORKLOADS["tiny"]
    dims = inputs.dims_of(w)
    x = inputs.make_x(w, 1)
    W = inputs.make_w(w, 2)
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    fw = oracle.qkv_forward(dims, 1, 256, x, wp, s_w)
    rng = np.random.default_rng(3)
    gb = inputs.f32_to_bf16_bits(rng.standard_normal((256, 320)).astype(np.float32))
    z = np.zeros((1, 1, 256, 96), dtype=np.uint16)
    bw = oracle.qkv_backward(dims, 1, 256, z, z, z, fw["x8"], fw["s_x"], None, wp, s_w,
                             dqkv_bits=gb)
    t = oracle.e4m3_decode_table()
    X = t[fw["x8"]] * float(fw["s_x"])
    Wd = t[wp] * float(s_w)
    G = t[bw["g8"]] * float(bw["s_g"])
    a = np.sum(G * fw["y64"])
    b = np.sum(bw["dx64"] * X)
    c = np.sum(bw["dw64"] * Wd)
    assert abs(a - b) <= 1e-12 * abs(a) and abs(a - c) <= 1e-12 * abs(a)
