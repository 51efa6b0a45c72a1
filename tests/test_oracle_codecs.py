"""Pins of the oracle's element codecs against library routines and the format tables."""

import numpy as np
import pytest
import torch

from oracle import codecs


def test_e2m1_decode_all_16_codes():
    # The E2M1 value set {0, .5, 1, 1.5, 2, 3, 4, 6} with the sign in bit 3: each code
    # is sign * 2^(e-1) * (1 + m/2) for e >= 1, and m/2 for e == 0.
    for c in range(16):
        s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        want = -mag if s else mag
        got = codecs.e2m1_decode(np.array([c]))[0]
        assert got == want and np.signbit(got) == bool(s)


def test_e2m1_encode_round_trip_and_ties():
    vals = codecs.e2m1_decode(np.arange(16))
    assert np.array_equal(codecs.e2m1_encode(vals), np.arange(16, dtype=np.uint8))
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in ties.items():
        assert codecs.e2m1_encode(np.array([v]))[0] == c
        assert codecs.e2m1_encode(np.array([-v]))[0] == c | 8
    assert codecs.e2m1_encode(np.array([7.0, 1e30, -100.0])).tolist() == [7, 7, 15]


def test_e2m1_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(0)
    y = rng.uniform(-8, 8, 20000)
    codes = codecs.e2m1_encode(y)
    dec = codecs.e2m1_decode(codes)
    grid = codecs.e2m1_decode(np.arange(16))
    best = np.min(np.abs(y[:, None] - grid[None, :]), axis=1)
    assert np.array_equal(np.abs(y - dec), best)


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2                                   # only S.1111.111
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_e4m3_encode_matches_torch_on_a_dense_sweep():
    rng = np.random.default_rng(1)
    s = np.concatenate([
        np.linspace(0, 448, 200001, dtype=np.float32),
        rng.uniform(0, 2 ** -6, 50000).astype(np.float32),              # subnormal range
        (codecs.E4M3_MAGNITUDES[:-1] + codecs.E4M3_MAGNITUDES[1:]).astype(np.float32) / 2,  # midpoints
        np.array([450.0, 463.9, 464.0, 1e9], np.float32),               # saturation
    ])
    ours = codecs.e4m3_encode(s.astype(np.float64))
    ref = torch.from_numpy(np.minimum(s, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_rounding_matches_torch_for_fp32_inputs():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 0.0, 2 ** -130])])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.f64_to_bf16_bits(v.astype(np.float64)), ref)


def test_bf16_rounding_of_float64_rounds_once():
    # 1 + 2^-8 + 2^-30 is just above the BF16 midpoint between 1 and 1 + 2^-7, so it
    # rounds up; rounding through fp32 first would lose the 2^-30 and tie down to 1.
    v = np.array([1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8], np.float64)
    out = codecs.bf16_bits_to_f32(codecs.f64_to_bf16_bits(v))
    assert out.tolist() == [1 + 2 ** -7, 1.0]


def test_bf16_bits_to_f32_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = codecs.bf16_bits_to_f32(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
