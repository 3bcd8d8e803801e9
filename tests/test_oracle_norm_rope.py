"""Pins of the oracle's split / RMSNorm / RoPE / head-major layout stage
("96 is enough", "The change": split, rms_norm on q and k, then rope on q and
k) and of its backward (PR #344, "Changes"; "Where the eight seconds were
hiding", "The inventory": norm, RoPE and backward kernels).

Pins: unit RMS after the norm, scale invariance, rotation properties (norm
preservation, identity at p = 0, inverse, the textbook 2-D rotation for
d = 2, scores depending only on the position difference), central finite
differences of the unquantised float64 forward, and structural special cases
of the whole chain (zeroed weight blocks, index-tagged layout)."""
import numpy as np
import pytest

import oracle
from fp8_packed_reduced_amd import inputs

EPS = 1e-6
BASE = 10000.0


def _rows(seed, T=64, R=3, d=96, scale=1.0):
    return np.random.default_rng(seed).standard_normal((T, R, d)) * scale


def test_rmsnorm_unit_rms_and_scale_invariance():
    a = _rows(0)
    u, rho = oracle.rmsnorm(a, EPS)
    ms = np.mean(a * a, axis=-1)
    assert np.allclose(np.mean(u * u, axis=-1), ms / (ms + EPS), rtol=1e-14, atol=0)
    u7, _ = oracle.rmsnorm(7.0 * a, EPS)
    assert np.allclose(u7, u, rtol=1e-6, atol=1e-9)      # equal up to eps
    u0, _ = oracle.rmsnorm(np.zeros((1, 1, 96)), EPS)
    assert not u0.any()


def test_rope_identity_at_position_zero_and_norm_preservation():
    a = _rows(1)
    pos = np.arange(64)
    r = oracle.rope(a, pos, BASE)
    assert np.array_equal(r[0], a[0])
    h = 48
    pair_in = a[..., :h] ** 2 + a[..., h:] ** 2
    pair_out = r[..., :h] ** 2 + r[..., h:] ** 2
    assert np.allclose(pair_in, pair_out, rtol=1e-13, atol=1e-13)


def test_rope_inverse_and_d2_textbook_rotation():
    a = _rows(2)
    pos = np.arange(64) * 977
    back = oracle.rope_inverse(oracle.rope(a, pos, BASE), pos, BASE)
    assert np.allclose(back, a, rtol=0, atol=1e-12)
    # d = 2: theta_0 = base^0 = 1, so position p rotates the plane by p rad
    v = np.array([[[0.3, -1.7]]])
    for p in (0, 1, 5, 12345):
        c, s = np.cos(p), np.sin(p)
        want = np.array([[c, -s], [s, c]]) @ v[0, 0]
        assert np.allclose(oracle.rope(v, np.array([p]), BASE)[0, 0], want, atol=1e-15)


def test_rope_frequencies_first_and_last_pair():
    # pair i of a d-wide row turns by p * base^(-2i/d)
    d, p = 96, 1000
    e = np.zeros((2, 1, d))
    e[:, 0, 0] = 1.0       # unit vector in the first coordinate of pair 0
    e[1, 0, 0] = 0.0
    e[1, 0, 47] = 1.0      # first coordinate of pair 47
    r = oracle.rope(e, np.array([p, p]), BASE)
    ang0 = np.arctan2(r[0, 0, 48], r[0, 0, 0])
    ang47 = np.arctan2(r[1, 0, 95], r[1, 0, 47])
    want0 = np.angle(np.exp(1j * p * 1.0))
    want47 = np.angle(np.exp(1j * p * BASE ** (-94 / 96)))
    assert abs(ang0 - want0) < 1e-12 and abs(ang47 - want47) < 1e-12


def test_scores_depend_only_on_position_difference():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 96))
    k = rng.standard_normal((1, 1, 96))
    P = 40
    pos = np.arange(P) * 1637   # large positions too
    Rq = oracle.rope(np.repeat(q, P, 0), pos, BASE)[:, 0]
    Rk = oracle.rope(np.repeat(k, P, 0), pos, BASE)[:, 0]
    S = Rq @ Rk.T
    for off in range(-P + 1, P):
        diag = np.diagonal(S, off)
        # positions reach 6.4e4 rad, whose double ulp is ~1e-11: allow 1e-9
        assert np.ptp(diag) < 1e-9 * (1 + np.abs(diag).max())


def test_norm_then_rope_commutes():
    a = _rows(4)
    pos = np.arange(64) * 31
    x = oracle.rope(oracle.rmsnorm(a, EPS)[0], pos, BASE)
    y = oracle.rmsnorm(oracle.rope(a, pos, BASE), EPS)[0]
    assert np.allclose(x, y, rtol=0, atol=1e-13)


def test_backward_matches_central_finite_differences():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((6, 2, 96))
    dout = rng.standard_normal((6, 2, 96))
    pos = np.array([0, 1, 2, 100, 4095, 65535])
    da = oracle.qk_norm_rope_bwd(a, dout, pos, EPS, BASE)
    h = 1e-6
    worst = 0.0
    for idx in [(0, 0, 0), (1, 1, 5), (2, 0, 47), (3, 1, 48), (4, 0, 95), (5, 1, 60),
                (5, 0, 1), (3, 0, 30)]:
        ap = a.copy()
        am = a.copy()
        ap[idx] += h
        am[idx] -= h
        fp = np.sum(dout * oracle.qk_norm_rope_fwd(ap, pos, EPS, BASE))
        fm = np.sum(dout * oracle.qk_norm_rope_fwd(am, pos, EPS, BASE))
        fd = (fp - fm) / (2 * h)
        worst = max(worst, abs(fd - da[idx]) / max(1e-3, abs(da[idx])))
    assert worst < 1e-7


def test_norm_gradient_is_nearly_orthogonal_to_input():
    # d rms_norm is orthogonal to a up to eps: <da, a> = <u, du> * eps / (ms + eps)
    rng = np.random.default_rng(6)
    a = rng.standard_normal((50, 2, 96)) * 0.01
    dout = rng.standard_normal((50, 2, 96))
    pos = np.arange(50)
    da = oracle.qk_norm_rope_bwd(a, dout, pos, EPS, BASE)
    u, _ = oracle.rmsnorm(a, EPS)
    du = oracle.rope_inverse(dout, pos, BASE)
    ms = np.mean(a * a, axis=-1)
    lhs = np.sum(da * a, axis=-1)
    rhs = np.sum(u * du, axis=-1) * EPS / (ms + EPS)
    assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-15)


def _chain(w, W, seed=1):
    dims = inputs.dims_of(w)
    x = inputs.make_x(w, seed)
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    return dims, x, wp, s_w, oracle.qkv_forward(dims, w["n_seq"], w["seq_len"], x, wp, s_w)


def test_chain_split_order_with_zeroed_weight_blocks():
    w = dict(n_seq=2, seq_len=32, d_model=64, n_heads=2, d_qk=32, d_v=64)
    W = inputs.make_w(w, 3)
    W[:, 64:] = 0.0          # only the Q block (first H*d_qk columns) is nonzero
    dims, x, wp, s_w, out = _chain(w, W)
    # (compare values: a zero product may carry a negative sign)
    assert out["q64"].any() and not out["k64"].any() and not out["v64"].any()
    W = inputs.make_w(w, 3)
    W[:, :128] = 0.0         # only V nonzero
    dims, x, wp, s_w, out = _chain(w, W)
    assert not out["q64"].any() and not out["k64"].any() and out["v64"].any()


def test_chain_layout_and_positions_by_index():
    w = dict(n_seq=2, seq_len=8, d_model=32, n_heads=2, d_qk=16, d_v=32)
    W = inputs.make_w(w, 4)
    dims, x, wp, s_w, out = _chain(w, W)
    H, dqk, dv, S = 2, 16, 32, 8
    y = out["y_bits"]
    for b in range(2):
        for h in range(H):
            for s in range(S):
                t = b * S + s
                for j in range(dv):
                    assert out["v_bits"][b, h, s, j] == y[t, 2 * H * dqk + h * dv + j]
    # first token of every sequence is at position 0: q there is only normalised
    yd = oracle.bf16_to_f64(y)
    for b in range(2):
        t = b * S
        for h in range(H):
            a = yd[t, h * dqk:(h + 1) * dqk]
            want = a / np.sqrt(np.mean(a * a) + EPS)
            assert np.allclose(out["q64"][b, h, 0], want, rtol=1e-14, atol=0)


def test_backward_chain_routes_each_gradient_to_its_block():
    w = dict(n_seq=1, seq_len=16, d_model=32, n_heads=2, d_qk=16, d_v=32)
    W = inputs.make_w(w, 5)
    dims, x, wp, s_w, out = _chain(w, W)
    dq, dk, dv = inputs.make_dy(w, 6)
    z_qk = np.zeros_like(dq)
    z_v = np.zeros_like(dv)
    qk_pre = out["y_bits"][:, :64]
    bw = oracle.qkv_backward(dims, 1, 16, z_qk, dk, z_v, out["x8"], out["s_x"], qk_pre, wp, s_w)
    g = bw["dqkv64"]
    assert not g[:, :32].any() and g[:, 32:64].any() and not g[:, 64:].any()
    assert not bw["dw64"][:, :32].any() and not bw["dw64"][:, 64:].any()
    bw = oracle.qkv_backward(dims, 1, 16, z_qk, z_qk, dv, out["x8"], out["s_x"], qk_pre, wp, s_w)
    # the V block of the packed gradient is the head-major dv, re-laid out
    gv = bw["dqkv_bits"][:, 64:].reshape(16, 2, 32)
    assert np.array_equal(gv, oracle.from_head_major(dv))
