"""CPU checks of the parity-comparison rules themselves (tests/compare.py)."""

import numpy as np
import pytest

import oracle
from tests import compare


def test_code_diff_counting():
    rng = np.random.default_rng(0)
    c = rng.integers(0, 16, (4, 64)).astype(np.uint8)
    s = rng.integers(1, 120, (4, 4)).astype(np.uint8)
    st = compare.code_diff_stats(c, s, c, s)
    assert st["n_diff"] == 0 and st["max_step_same_scale"] == 0
    g = c.copy(); gs = s.copy()
    g[0, 3] = {0: 1, 8: 9}.get(int(c[0, 3]), c[0, 3] ^ 1)   # some change of the code
    gs[2, 1] += 1                                             # one block scale differs
    st = compare.code_diff_stats(g, gs, c, s)
    assert st["scale_diff_blocks"] == 1 and st["n_diff"] >= 16
    assert set(st["rows_with_diff"].tolist()) >= {2}
    # +0 vs -0 is no step; 4 vs 6 (codes 6, 7) is one step; 4 vs 3 is one step
    a = np.array([[0, 6, 6] + [0] * 13], np.uint8); b = np.array([[8, 7, 5] + [0] * 13], np.uint8)
    st = compare.code_diff_stats(a, np.ones((1, 1), np.uint8), b, np.ones((1, 1), np.uint8))
    assert st["max_step_same_scale"] == 1 and st["n_diff"] == 2


def test_output_bound_is_two_percent_of_the_unrounded_row_rms():
    ref = np.array([[3.0, -1.0, 0.5, 0.25] * 8])
    rms = np.sqrt(np.mean(ref ** 2))
    # the BF16 rounding of the reference itself passes (here exact)
    res = compare.check_output(oracle.f64_to_bf16_bits(ref), ref)
    assert res["ratio"] == 0.0 and res["rows_widened"] == 0
    # a deviation just inside 2e-2 * rms passes, one just outside fails: no ulp slack
    bits = oracle.f64_to_bf16_bits(ref)                        # exact: err = |shift|
    for frac, ok in ((0.0199, True), (0.0201, False)):
        moved = ref.copy(); moved[0, 0] -= frac * rms          # reference shifted, rms kept
        moved_rms = np.sqrt(np.mean(moved ** 2))
        moved[0, 0] = ref[0, 0] - frac * moved_rms
        if ok:
            assert compare.check_output(bits, moved)["ratio"] <= 1.0
        else:
            with pytest.raises(AssertionError):
                compare.check_output(bits, moved)
    far = oracle.f64_to_bf16_bits(ref + 0.2 * rms)
    with pytest.raises(AssertionError):
        compare.check_output(far, ref)
    # a large deviation is accepted only when the flip effect dy accounts for it, and the
    # row is reported as widened
    res = compare.check_output(far, ref, dy=np.full(ref.shape, 0.2 * rms))
    assert res["rows_widened"] == 1


def test_flip_effect_is_the_fc2_difference():
    rng = np.random.default_rng(1)
    I, H = 32, 8
    rc = rng.integers(0, 16, (I,)).astype(np.uint8); rs = np.array([0x38, 0x40], np.uint8)
    gc = rc.copy(); gc[5] = (rc[5] & 8) | min((rc[5] & 7) + 1, 7)
    w2 = rng.standard_normal((H, I))
    d = compare.flip_effect(gc, rs, rc, rs, w2, 2.0)
    want = 2.0 * w2 @ (oracle.dequantize_nvfp4(gc, rs) - oracle.dequantize_nvfp4(rc, rs))
    assert np.allclose(d, want)
