"""Pins of the oracle's e5m2 gradient format (the optional attention-ready
variant: FP8 gradients in OCP E5M2) against torch's float8_e5m2 and the
definition of the format, and of the backward chain that uses it.

What torch provides is checked where it applies: its decoder on all 256
codes, and its round-to-nearest-even cast below its overflow threshold (it
turns larger values into infinity; the oracle saturates, a stated reading).
The two oracle encoders are independent and must agree on every fp32."""
import numpy as np
import torch

import oracle
from fp8_packed_reduced_amd import inputs

from test_oracle_codec import _class_patterns
from test_oracle_gemm import _brute


def test_decode_matches_torch_on_all_256_codes():
    t = oracle.e5m2_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], ref[ok])


def test_decode_named_values_of_the_e5m2_format():
    t = oracle.e5m2_decode_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -16                    # smallest subnormal
    assert t[0x03] == 3 * 2.0 ** -16                # largest subnormal
    assert t[0x04] == 2.0 ** -14                    # smallest normal
    assert t[0x3C] == 1.0 and t[0x3D] == 1.25 and t[0xBC] == -1.0
    assert t[0x7B] == 57344.0 and t[0xFB] == -57344.0
    assert np.isposinf(t[0x7C]) and np.isneginf(t[0xFC])
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    fin = t[:0x7C]
    assert np.all(np.diff(fin) > 0)                  # increasing over the finite codes


def test_encode_round_trips_every_finite_code():
    t = oracle.e5m2_decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    assert codes.size == 248
    assert np.array_equal(oracle.e5m2_encode(t[codes].astype(np.float32)), codes)


def test_encode_midpoints_round_to_even_and_neighbours_to_nearer():
    t = oracle.e5m2_decode_table()
    for c in range(0, 0x7B):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1e6))
        got = oracle.e5m2_encode(np.array([mid, below, above], dtype=np.float32))
        assert list(got) == [even, c, c + 1], c


def test_encode_saturates_and_keeps_sign():
    v = np.array([57344.0, 61439.0, 61440.0, 1e30, np.inf, -1e30, -np.inf, -0.0, -1e-30],
                 dtype=np.float32)
    assert list(oracle.e5m2_encode(v)) == [0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB, 0x80, 0x80]


def test_two_encoders_agree_on_every_fp32_pattern():
    n, first = oracle.e5m2_encoders_disagree(0, 1 << 32)
    assert n == 0, hex(first)


def test_encode_matches_torch_cast_below_the_overflow_threshold():
    v = _class_patterns()
    rng = np.random.default_rng(5)
    v = np.concatenate([v, rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64)
                        .astype(np.uint32).view(np.float32)])
    v = v[np.isfinite(v) & (np.abs(v) < 61440.0)]
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e5m2_encode(v), ref)


def test_quantiser_scale_amax_code_and_error_bound():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(20000) * 0.1).astype(np.float32)
    bits = inputs.f32_to_bf16_bits(v)
    vals = oracle.bf16_to_f64(bits)
    codes, s, inv, rc = oracle.quantize_bf16(bits, "e5m2")
    amax = np.float32(np.max(np.abs(vals)))
    assert rc == 0 and s == np.float32(amax / np.float32(57344.0))
    assert inv == np.float32(np.float32(57344.0) / amax)
    i = int(np.argmax(np.abs(vals)))
    assert codes[i] & 0x7F == 0x7B
    deq = oracle.e5m2_decode(codes) * float(s)
    # normal e5m2 values carry 2 fraction bits: half a step is 2^-3 relative
    big = np.abs(vals) > float(s) * 2.0 ** -14
    assert np.all(np.abs(deq[big] - vals[big]) <= 2.0 ** -3 * np.abs(vals[big]) * (1 + 1e-6))
    # all zero: unit scale; NaN: reported
    _, s0, i0, rc0 = oracle.quantize_bf16(np.zeros(8, np.uint16), "e5m2")
    assert (s0, i0, rc0) == (1.0, 1.0, 0)
    _, _, _, rcn = oracle.quantize_bf16(np.array([0x7FC0, 0x3F80], np.uint16), "e5m2")
    assert rcn == 1


def test_mixed_format_gemm_integer_brute_force():
    rng = np.random.default_rng(4)
    a = rng.choice([0, 1, -1, 2, -2, 3, -3, 5, -6, 7, 8, -12, 16], size=(7, 40)).astype(np.float32)
    b = rng.integers(-16, 17, size=(40, 11)).astype(np.float32)
    got = oracle.gemm_e4m3(oracle.e5m2_encode(a), oracle.e4m3_encode(b), 1.0, 1.0,
                           a_fmt="e5m2")
    assert np.array_equal(got, _brute(a, b))
    got_t = oracle.gemm_e4m3(oracle.e4m3_encode(b.T), oracle.e5m2_encode(a.T), 1.0, 1.0,
                             b_fmt="e5m2")
    assert np.array_equal(got_t, _brute(b.T, a.T))


def test_backward_chain_with_e5m2_gradients_integer_inputs_exact():
    w = dict(n_seq=1, seq_len=16, d_model=32, n_heads=1, d_qk=32, d_v=32)
    dims = inputs.dims_of(w)
    rng = np.random.default_rng(9)
    x = rng.integers(-8, 9, size=(16, 32)).astype(np.float32)
    x[0, 0] = 448.0
    W = rng.integers(-8, 9, size=(32, 96)).astype(np.float32)
    W[1, 1] = 448.0
    # e5m2-exact integers plus one -57344, so the gradient scale is exactly 1
    g = rng.choice([0, 1, -1, 2, -2, 3, -3, 4, -5, 6, -7, 8], size=(16, 96)).astype(np.float32)
    g[2, 2] = -57344.0
    wp, _, s_w, _, _ = oracle.pack_quantize_weights(dims, W)
    x8, s_x, _, _ = oracle.quantize_bf16(inputs.f32_to_bf16_bits(x))
    gb = inputs.f32_to_bf16_bits(g)
    z = np.zeros((1, 1, 16, 32), dtype=np.uint16)
    out = oracle.qkv_backward(dims, 1, 16, z, z, z, x8, s_x, None, wp, s_w, dqkv_bits=gb,
                              grad_fmt="e5m2")
    assert out["s_g"] == 1.0
    assert np.array_equal(oracle.e5m2_decode(out["g8"]), g.astype(np.float64))
    assert np.array_equal(out["dx64"], _brute(g, W.T))
    assert np.array_equal(out["dw64"], _brute(x.T, g))
    # the same gradient read as e4m3 codes would not be exact: the format matters
    wrong = oracle.e4m3_decode(out["g8"])
    assert not np.array_equal(wrong[np.isfinite(wrong)], g[np.isfinite(wrong)])
