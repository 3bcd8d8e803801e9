"""Pins of the oracle's per-tensor quantiser and of the dual-layout packed
weight quantiser (PR #344 page, "Changes": both FP8 layouts from one weight
read, no materialised concatenation; "96 is enough", "The change": W_packed =
[W_q | W_k | W_v]).  Checked against invariants that any correct amax-scaled
e4m3 quantiser must satisfy, not against the oracle itself."""
import json
import os

import numpy as np
import pytest

import oracle
from fp8_packed_reduced_amd import inputs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_amax_element_encodes_to_448(seed):
    v = np.random.default_rng(seed).standard_normal(5000).astype(np.float32) * 0.01
    codes, s, inv, rc = oracle.quantize_f32(v)
    assert rc == 0
    i = int(np.argmax(np.abs(v)))
    t = oracle.e4m3_decode_table()
    assert abs(t[codes[i]]) == 448.0
    assert np.all(np.abs(t[codes]) <= 448.0)
    # s and inv are the fp32 quotients of amax and 448
    amax = np.float32(np.max(np.abs(v)))
    assert s == np.float32(amax / np.float32(448)) and inv == np.float32(np.float32(448) / amax)


def test_containing_448_gives_unit_scale_and_plain_codes():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(4096) * 40).astype(np.float32)
    v[17] = -448.0
    codes, s, inv, rc = oracle.quantize_f32(v)
    assert (s, inv, rc) == (1.0, 1.0, 0)
    assert np.array_equal(codes, oracle.e4m3_encode(v))


def test_relative_error_is_within_half_an_e4m3_step():
    # e4m3 keeps 4 significant bits: in the normal range the rounding error of
    # v*inv is at most 2^-4 of it; in the subnormal range at most 2^-10.
    v = np.random.default_rng(4).standard_normal(1 << 16).astype(np.float32)
    codes, s, inv, _ = oracle.quantize_f32(v)
    t = oracle.e4m3_decode_table()
    scaled = (v * inv).astype(np.float64)
    err = np.abs(t[codes] - scaled)
    bound = np.maximum(np.abs(scaled) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound)


def test_requantising_dequantised_values_is_idempotent():
    v = np.random.default_rng(5).standard_normal(10000).astype(np.float32)
    codes, s, inv, _ = oracle.quantize_f32(v)
    t = oracle.e4m3_decode_table()
    deq = (t[codes] * np.float64(s)).astype(np.float32)
    codes2, s2, inv2, _ = oracle.quantize_f32(deq)
    assert np.array_equal(codes, codes2)


def test_zero_tensor_and_nonfinite_amax():
    codes, s, inv, rc = oracle.quantize_f32(np.zeros(100, dtype=np.float32))
    assert (s, inv, rc) == (1.0, 1.0, 0) and not codes.any()
    v = np.ones(10, dtype=np.float32)
    v[3] = np.nan
    assert oracle.quantize_f32(v)[3] == 1
    v[3] = np.inf
    assert oracle.quantize_f32(v)[3] == 1
    # a tiny amax whose 448/amax overflows falls back to unit scale
    v = np.full(4, np.float32(1e-45), dtype=np.float32)
    assert oracle.quantize_f32(v)[1:] == (1.0, 1.0, 0)


def test_bf16_quantiser_equals_fp32_quantiser_on_widened_values():
    bits = inputs.f32_to_bf16_bits(np.random.default_rng(6).standard_normal(30000).astype(np.float32))
    a = oracle.quantize_bf16(bits)
    b = oracle.quantize_f32(oracle.bf16_to_f64(bits).astype(np.float32))
    assert np.array_equal(a[0], b[0]) and a[1:] == b[1:]


@pytest.mark.parametrize("wl", ["tiny", "fwd_16k", "sweep_64"])
def test_packed_weight_both_layouts_and_column_order(wl):
    w = inputs.WORKLOADS[wl]
    W = inputs.make_w(w, 11)
    wq, wk, wv = inputs.split_w(w, W)
    D, H, dqk, dv = w["d_model"], w["n_heads"], w["d_qk"], w["d_v"]
    wp, wpt, s, inv, rc = oracle.pack_quantize(D, H, dqk, dv, wq, wk, wv)
    assert rc == 0
    assert wp.shape == (D, inputs.packed_width(w)) and wpt.shape == wp.shape[::-1]
    assert np.array_equal(wpt, wp.T)                     # the two layouts agree
    # the packed codes are the per-tensor quantisation of the explicit
    # concatenation [Wq | Wk | Wv] (built here, never by the oracle)
    cat = np.ascontiguousarray(np.concatenate([wq, wk, wv], axis=1))
    codes, s2, inv2, _ = oracle.quantize_f32(cat)
    assert np.array_equal(wp, codes) and (s, inv) == (s2, inv2)


def test_packed_widths_match_the_pages():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "pages_packed_widths.json")))
    for H in (1, 6):
        n = oracle.packed_columns(H, g["d_qk"], g["d_v"])[3]
        n128 = oracle.packed_columns(H, g["d_v"], g["d_v"])[3]
        assert n == g["packed_columns_per_head"] * H
        assert n128 == g["packed_columns_per_head_at_128_wide_qk"] * H
        assert round(100 * (1 - n / n128), 1) == g["qkv_width_reduction_percent"]
    assert round(100 * (1 - g["d_qk"] / g["d_v"])) == g["qk_projection_reduction_percent"]
