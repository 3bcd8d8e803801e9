"""Pins of the oracle's e4m3 codec and bf16 rounding against things other than
itself: the OCP OFP8 E4M3 definition (named values, value count, ordering),
torch's own float8_e4m3fn / bfloat16 conversions (an independent library
implementation), a second encoder by table search, and exact midpoints.

The pages only say "FP8"; the E4M3 reading is the one every fixture here
assumes (see the oracle's header)."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_decode_matches_torch_on_all_256_codes():
    ours = oracle.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # sign of zero too
    assert math.copysign(1.0, ours[0x80]) == -1.0 and math.copysign(1.0, ours[0x00]) == 1.0


def test_decode_named_values_of_the_e4m3_format():
    # OCP 8-bit Floating Point Specification (OFP8), E4M3 column of the table
    # of format parameters: max normal 448 = S.1111.110, min normal 2^-6,
    # max subnormal 0.875 * 2^-6, min subnormal 2^-9, NaN = S.1111.111,
    # no infinities; exponent bias 7.
    t = oracle.e4m3_decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6
    assert t[0x07] == 0.875 * 2.0 ** -6
    assert t[0x01] == 2.0 ** -9
    assert t[0x38] == 1.0          # exponent field 7 = bias
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert not np.any(np.isinf(t))


def test_decode_count_order_symmetry():
    t = oracle.e4m3_decode_table()
    fin = t[~np.isnan(t)]
    assert fin.size == 254
    assert np.unique(fin).size == 253          # +0 and -0 coincide
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)            # strictly increasing codes 0..126
    assert np.array_equal(t[0x80:0xFF], -pos)  # sign bit mirrors


def test_encode_round_trips_every_finite_code():
    t = oracle.e4m3_decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = t[codes].astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encode_midpoints_round_to_even_and_neighbours_to_nearer():
    t = oracle.e4m3_decode_table()
    for c in range(0, 126):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)        # exact: at most 5 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1000))
        got = oracle.e4m3_encode(np.array([mid, below, above], dtype=np.float32))
        assert list(got) == [even, c, c + 1], c
        gotn = oracle.e4m3_encode(-np.array([mid, below, above], dtype=np.float32))
        assert list(gotn) == [0x80 | even, 0x80 | c, 0x80 | (c + 1)], c


def test_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 463.99, 464.0, 1e30, np.inf, -1e30, -np.inf, -0.0, -1e-30, 1e-30],
                 dtype=np.float32)
    got = oracle.e4m3_encode(v)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x80, 0x00]


def test_two_encoders_agree_on_every_fp32_pattern():
    n, first = oracle.e4m3_encoders_disagree(0, 1 << 32)
    assert n == 0, hex(first)


def _class_patterns():
    """Every fp32 whose low 16 bits are one of a few tails, i.e. every
    (sign, exponent, top-7 mantissa bits) prefix with sticky bits absent,
    lowest, middle or all set: covers every rounding class of e4m3."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    tails = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | tails[None, :]).ravel()
    return bits.view(np.float32)


def test_encode_matches_torch_cast_below_the_overflow_threshold():
    # torch's float -> float8_e4m3fn is round-to-nearest-even and turns
    # values of magnitude >= 464 into NaN (it does not saturate); below that
    # threshold it must agree with our encoder bit for bit.
    v = _class_patterns()
    rng = np.random.default_rng(0)
    v = np.concatenate([v, rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64)
                        .astype(np.uint32).view(np.float32)])
    keep = np.isfinite(v) & (np.abs(v) < 464.0)
    v = v[keep]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


def test_round_bf16_matches_torch_on_fp32_inputs():
    v = _class_patterns()
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16(v.astype(np.float64)), ref)


def test_round_bf16_rounds_once_from_double():
    # 1 + 2^-8 is the midpoint between the bf16 neighbours 1 and 1 + 2^-7.
    # Slightly above it the correct result is 1 + 2^-7; rounding through fp32
    # first would land exactly on the midpoint and then tie to 1.
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])
    got = oracle.bf16_to_f64(oracle.round_bf16(x))
    assert list(got) == [1.0 + 2.0 ** -7, 1.0, 1.0 + 2.0 ** -6]


def test_bf16_widening_is_exact():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
