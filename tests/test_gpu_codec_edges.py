"""The hardware conversions inside the GPU quantizer, pinned against the oracle at their
decision points.

The kernels encode with gfx950's fp32 -> E4M3 conversion (the block scale, after the clamp
to 448) and its fp32 -> E2M1 conversion with scale 1 (the codes), and form amax*q/6 with a
reciprocal product and one FMA correction (pinned over every float by
test_nvfp4_scale_division.py).  Here moe_quantize_nvfp4 runs on crafted blocks:
  * the block scale's quotient s32 = fp32(fp32(amax*q)/6) on every midpoint between two
    E4M3 values -- subnormal, normal, and above 448 -- and one float step either side
    (two steps where a float quotient lands there);
  * v*enc on every midpoint between two E2M1 magnitudes (and their negatives) and 1 or 2
    float steps either side, with block scales 2^b for b = -9 (the smallest subnormal
    scale) to 8.
Codes and scales must equal oracle.quantize_nvfp4 bit for bit.  The inputs (BF16 values and
the fp32 q of each block) are found on the host by searching float neighbours; the expected
values come from the oracle only."""

import sys

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import f32_to_bf16_bits
from tests.gpu_harness import dev, host, quantize_on_gpu

pytestmark = pytest.mark.gpu

F = np.float32


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _steps(x, k):
    """x moved k float32 steps (k may be negative)."""
    return np.nextafter(F(x), F(np.inf if k > 0 else -np.inf)) if k == 1 or k == -1 else (
        _steps(_steps(x, np.sign(k)), k - np.sign(k)) if k else F(x))


def _scale_quotient(amax, q):
    return F(F(F(amax) * F(q)) / F(6.0))


AMAX_CHOICES = (6.0, 5.0, 7.0, 3.5, 4.5, 6.5, 5.5, 3.0)      # exact in BF16


def _e4m3_cases(rng):
    """(block values fp32 [16], q) with fp32(fp32(amax*q)/6) at E4M3 midpoints (amax one
    of a few BF16 values, q searched among the floats near 6*target/amax)."""
    grid = np.array(sorted(set(oracle.codecs.E4M3_MAGNITUDES.tolist())), np.float64)
    mids = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])] + [464.0, 500.0, 1e6]
    cases, hit = [], 0
    for m in mids:
        for k in (-2, -1, 0, 1, 2):
            target = _steps(F(m), k)
            done = False
            # (x = amax*q lies two binades above x/6, so neighbouring quotients are 2/3 or
            # 4/3 of a step apart: the second neighbours are reached only sometimes)
            for amax in AMAX_CHOICES:
                q0 = F(np.float64(target) * 6.0 / amax)
                for d in range(-8, 9):
                    q = _steps(q0, d)
                    if _scale_quotient(amax, q) == target:
                        v = oracle.bf16_bits_to_f32(f32_to_bf16_bits(
                            (rng.uniform(-1, 1, 16) * amax).astype(F)))
                        v[0] = amax
                        cases.append((v, q))
                        done = True
                        break
                if done:
                    break
            hit += done and abs(k) <= 1
    return cases, hit, 3 * len(mids)


E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_cases():
    """(block values fp32 [16], q) with a block scale of 2^b and v*enc on E2M1 midpoints:
    for a BF16 v near the target t, q (within 1/32 of 1, so the scale stays 2^b and
    enc = q*2^-b exactly) is chosen with fp32(v*q) == t; the block holds 6*2^b (its amax),
    v*2^b and -v*2^b."""
    bf = lambda a: oracle.bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, F)))
    cases, hit, want = [], 0, 0
    for b in (-9, -8, -7, -6, -3, 0, 3, 6, 8):
        for t in E2M1_MIDS:
            for k in (-2, -1, 0, 1, 2):
                want += 1
                target = _steps(F(t), k)
                found = False
                for v in np.unique(bf(np.array([t * (1 + e) for e in
                                                np.linspace(-0.02, 0.02, 9)], F))):
                    q0 = F(np.float64(target) / np.float64(v))
                    for d in range(-6, 7):
                        q = _steps(q0, d)
                        if abs(float(q) - 1.0) < 1.0 / 32 and F(F(v) * q) == target:
                            blk = np.zeros(16, F)
                            blk[0] = F(6.0 * 2.0 ** b)
                            blk[1] = F(v * 2.0 ** b)
                            blk[2] = -blk[1]
                            blk[3:] = F(2.0 ** b) * np.array(
                                [0, .5, 1, 1.5, 2, 3, 4, -6, -.25, .75, 5, -3.5, 2.5], F)
                            cases.append((blk, q))
                            found = True
                            break
                    if found:
                        break
                hit += found
    return cases, hit, want


def _run(cases):
    vals = np.stack([c[0] for c in cases]).astype(F)
    q = np.array([c[1] for c in cases], F)
    bits = f32_to_bf16_bits(vals)
    assert np.array_equal(oracle.bf16_bits_to_f32(bits), vals)      # exact BF16 inputs
    codes, scales = quantize_on_gpu(dev(bits), len(cases), 1, 16, dev(q))
    torch.cuda.synchronize()
    want_c, want_s = oracle.quantize_nvfp4(vals, q)
    assert np.array_equal(host(scales).reshape(-1), want_s.reshape(-1))
    assert np.array_equal(host(codes), oracle.pack_nibbles(want_c))
    return want_s.reshape(-1), want_c


def test_e4m3_scale_midpoints_bit_exact():
    cases, hit, want = _e4m3_cases(np.random.default_rng(5))
    _say(f"E4M3 scale midpoints: {hit} of {want} midpoint and one-step targets reached, "
         f"{len(cases)} blocks")
    assert hit == want
    s, _ = _run(cases)
    # the cases span subnormal, normal and saturated scales
    assert (s == 0).any() and (s < 8).any() and (s == 0x7E).any() and len(np.unique(s)) > 100


def test_e2m1_code_midpoints_bit_exact_in_every_scale_binade():
    cases, hit, want = _e2m1_cases()
    _say(f"E2M1 midpoints: {hit} of {want} targets reached")
    assert hit == want
    s, c = _run(cases)
    assert len(np.unique(s)) >= 9                     # one scale per binade
    assert len(np.unique(c)) == 16                    # every code, both signs
