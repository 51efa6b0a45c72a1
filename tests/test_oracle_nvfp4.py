"""Pins of the oracle's group-16 NVFP4 quantization: hand-worked blocks and invariants."""

import os

import numpy as np
import pytest

from oracle import codecs, nvfp4, calib

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_blocks.txt")


def _golden_blocks():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, q, vals, scale, codes = [p.strip() for p in line.split("|")]
        rows.append((name, np.float32(float(q)), np.array(vals.split(), np.float32),
                     int(scale, 16), [int(c, 16) for c in codes.split()]))
    return rows


@pytest.mark.parametrize("block", _golden_blocks(), ids=lambda b: b[0])
def test_hand_worked_blocks(block):
    name, q, v, scale, codes = block
    c, s = nvfp4.quantize_nvfp4(v[None, :], q)
    assert s[0].tolist() == [scale]
    assert c[0].tolist() == codes


def _random_rows(seed, n=512, K=256):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, K)).astype(np.float32)
    v *= np.exp(rng.uniform(-8, 8, (n, 1))).astype(np.float32)     # wide dynamic range
    v[rng.random((n, K)) < 0.05] = 0.0
    return v


def test_every_decoded_value_is_a_code_times_its_block_scale():
    v = _random_rows(0)
    _, q = calib.global_scale_from_amax(np.max(np.abs(v)))
    c, s = nvfp4.quantize_nvfp4(v, q)
    dec = nvfp4.dequantize_nvfp4(c, s)
    sv = codecs.e4m3_decode(s)
    ratio = dec.reshape(v.shape[0], -1, 16) / np.where(sv == 0, 1, sv)[..., None]
    grid = set(codecs.e2m1_decode(np.arange(16)).tolist())
    assert set(np.unique(ratio).tolist()) <= grid
    assert not np.any(np.isnan(sv))


def test_block_amax_lands_on_code_six_for_normal_scales():
    # With s a normal E4M3 value, s is within 1/16 (relative) of amax*q/6, so amax*enc
    # lies in [6/(1+1/16), 6/(1-1/16)] = [5.65, 6.4], which always rounds to 6.
    v = _random_rows(1)
    for q in (np.float32(1.0), np.float32(37.5), np.float32(3e3)):
        c, s = nvfp4.quantize_nvfp4(v, q)
        blocks = np.abs(v).reshape(v.shape[0], -1, 16)
        arg = np.argmax(blocks, axis=-1)
        cb = c.reshape(v.shape[0], -1, 16)
        amax_code = np.take_along_axis(cb, arg[..., None], -1)[..., 0] & 7
        normal = (s & 0x78) != 0                       # exponent field > 0
        unsat = codecs.e4m3_decode(s) < 448
        sel = normal & unsat & (blocks.max(-1) > 0)
        assert sel.sum() > 100
        assert np.all(amax_code[sel] == 7)


def test_quantization_error_bound_below_saturation():
    # |v - dec/q| <= half the E2M1 step at |v*enc| times s/q (plus fp32 rounding of
    # v*enc); steps are .5 below 2, 1 in [2, 4), 2 in [4, 6].
    v = _random_rows(2)
    q = np.float32(5.0)
    c, s = nvfp4.quantize_nvfp4(v, q)
    dec = nvfp4.dequantize_nvfp4(c, s) / np.float64(q)
    sv = np.repeat(codecs.e4m3_decode(s), 16, axis=1)
    y = np.abs(v.astype(np.float64)) * np.float64(q) / np.where(sv == 0, np.inf, sv)
    half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    bound = half_step * sv / np.float64(q) * (1 + 1e-6) + 1e-30
    ok = (sv > 0) & (y <= 6.0)
    assert np.all(np.abs(v - dec)[ok] <= bound[ok])


def test_zero_and_signed_zero_blocks():
    v = np.zeros((2, 32), np.float32)
    v[1, :16] = -0.0
    c, s = nvfp4.quantize_nvfp4(v, np.float32(1.0))
    assert s.tolist() == [[0, 0], [0, 0]]
    assert c[0].tolist() == [0] * 32
    assert c[1, :16].tolist() == [8] * 16


def test_scale_saturates_at_448():
    v = np.full((1, 16), 1000.0, np.float32)
    c, s = nvfp4.quantize_nvfp4(v, np.float32(10.0))       # amax*q/6 = 1666 > 448
    assert s[0, 0] == 0x7E and set(c[0].tolist()) == {7}


def test_pack_unpack_round_trip_and_nibble_order():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    p = nvfp4.pack_nibbles(c)
    assert p.shape == (7, 32)
    assert np.array_equal(nvfp4.unpack_nibbles(p), c)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))


def test_per_row_global_scale_broadcast():
    v = _random_rows(4, n=8, K=64)
    q = np.arange(1, 9, dtype=np.float32)
    c, s = nvfp4.quantize_nvfp4(v, q)
    for r in range(8):
        cr, sr = nvfp4.quantize_nvfp4(v[r:r + 1], q[r])
        assert np.array_equal(cr[0], c[r]) and np.array_equal(sr[0], s[r])


def test_calibration_puts_tensor_amax_at_scale_448_code_6():
    v = _random_rows(5, n=16, K=128)
    d, q = calib.global_scale_from_amax(np.max(np.abs(v)))
    c, s = nvfp4.quantize_nvfp4(v, q)
    r, col = np.unravel_index(np.argmax(np.abs(v)), v.shape)
    assert codecs.e4m3_decode(s[r, col // 16]) in (448.0, 416.0)   # 448 up to fp32 rounding of q
    assert c[r, col] & 7 == 7
    assert calib.global_scale_from_amax(np.float32(0.0)) == (np.float32(1.0), np.float32(1.0))
