"""Comparison rules of the GPU parity tests.

  * Integer results (routing, NVFP4 codes and scales of the input x, int8 codes) must be
    bit-exact.
  * Intermediate NVFP4 codes of the SiTU output may differ, because the fp32 accumulation
    order of the GPU differs from the exact dot product of the oracle: at most 0.1% of
    the codes may differ (a block whose E4M3 scale differs counts all 16 of its codes),
    and within blocks of equal scale a differing code is at most one E2M1 step away.
  * The BF16 output must satisfy, per row and element,
        |out - ref| <= 2e-2 * rms(ref row) + |dy|
    where ref is the oracle's output before its final BF16 rounding (float64) and dy is
    the exact linear effect on the output of the intermediate codes that differ (FC2 and
    finalization are linear in the decoded intermediate):
        dy[t, h] = sum_j w[t, j] * alpha2[e] * sum_i (ahat_gpu - ahat_ref)[i] * w2hat[e, h, i].
    For a row with no differing code dy = 0 and this is the plain 2e-2 * rms bound; a
    single one-step code flip can move an output element by more than that, so the bound
    of such a row is widened by exactly the flip's effect (computed from the codes, never
    from GPU outputs), and the number of rows that needed it is reported.
"""

import numpy as np

import oracle

OUT_RTOL = 2e-2
CODE_DIFF_FRAC = 1e-3
def x_dec_max_rows():
    """moe_forward writes the f16 copy of x (x_dec) only below two 128-row tiles per compute
    unit of routed rows (65536 on the 256-CU MI355X)."""
    import torch
    return 2 * torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count * 128

# signed position of each E2M1 code on the value line (+0 and -0 share position 0)
_POS = np.array([0, 1, 2, 3, 4, 5, 6, 7, 0, -1, -2, -3, -4, -5, -6, -7])


def unpack(packed):
    return oracle.unpack_nibbles(packed)


def code_diff_stats(gpu_codes_unpacked, gpu_scales, ref_codes_unpacked, ref_scales):
    """Counts of differing intermediate codes (see module docstring)."""
    R, I = ref_codes_unpacked.shape
    g = gpu_codes_unpacked.reshape(R, I // 16, 16)
    r = ref_codes_unpacked.reshape(R, I // 16, 16)
    scale_diff = gpu_scales != ref_scales
    step = np.abs(_POS[g] - _POS[r])
    same = ~scale_diff[..., None]
    n_diff = int(scale_diff.sum()) * 16 + int(((step > 0) & same).sum())
    max_step = int(step[np.broadcast_to(same, step.shape)].max()) if same.any() else 0
    return {"n_codes": R * I, "n_diff": n_diff, "frac": n_diff / max(R * I, 1),
            "max_step_same_scale": max_step, "scale_diff_blocks": int(scale_diff.sum()),
            "rows_with_diff": np.nonzero((scale_diff.any(1)) | ((step > 0) & same).any((1, 2)))[0]}


def flip_effect(gpu_codes_u, gpu_scales, ref_codes_u, ref_scales, w2hat, alpha2_e):
    """Exact change of one routed row's FC2 output caused by its differing codes."""
    dg = oracle.dequantize_nvfp4(gpu_codes_u, gpu_scales)
    dr = oracle.dequantize_nvfp4(ref_codes_u, ref_scales)
    return np.float64(alpha2_e) * (w2hat @ (dg - dr))


def check_output(gpu_bits, ref_f64, dy=None):
    """Assert the output bound against the oracle's unrounded output ref_f64 [n, H].

    Returns a dict: ``ratio`` = worst err / (2e-2 * rms) over rows without a differing
    intermediate code (the plain bound, never widened), ``ratio_all`` = worst
    err / tol over all rows, ``rows_widened`` = rows whose bound includes a flip's dy.
    """
    out = oracle.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    ref = np.asarray(ref_f64, dtype=np.float64)
    dy = np.zeros_like(ref) if dy is None else np.abs(np.asarray(dy, dtype=np.float64))
    widened = np.any(dy > 0, axis=1)
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    base = np.maximum(OUT_RTOL * rms, 1e-300)
    tol = OUT_RTOL * rms + dy
    err = np.abs(out - ref)
    bad = err > tol
    assert not bad.any(), (
        f"{bad.sum()} output elements out of bound; worst row "
        f"{np.argmax(bad.sum(1))}, max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3g}")
    plain = err / base
    ratio = float(np.max(plain[~widened])) if (~widened).any() else 0.0
    return {"ratio": ratio, "ratio_all": float(np.max(err / np.maximum(tol, 1e-300))),
            "rows_widened": int(widened.sum()), "rows": int(ref.shape[0])}


def fmt(res):
    return (f"worst err/(2e-2 rms) {res['ratio']:.3f} (rows with a flipped code: "
            f"{res['rows_widened']}/{res['rows']}, worst err/bound there "
            f"{res['ratio_all']:.3f})")


def out_exponents(alpha2, I):
    """The FC2 row exponent of each expert: s = clamp(141 - E, -126, 126) with E the fp32
    biased exponent of |alpha2| * I * 2688^2 (the bound on an FC2 sum of I products of two
    decoded NVFP4 values), so that every stored value O * 2^s is below 2^15."""
    b = np.abs(np.asarray(alpha2, np.float32)) * (np.float32(I) * np.float32(2688 * 2688))
    e = (b.astype(np.float32).view(np.uint32) >> 23) & 0xFF
    return np.clip(141 - e.astype(np.int64), -126, 126)


def flip_widening(p, gc, gs, ref, rows):
    """dy [T, H]: the exact output effect of the differing intermediate codes of the given
    rows (reference sorted order; gc unpacked codes and gs scales in that order)."""
    cfg = p["cfg"]
    dy = np.zeros((cfg.T, cfg.H))
    for i in rows:
        e = int(ref["sorted_ids"][i])
        f = int(ref["sorted_row_idx"][i])
        t, j = f // cfg.k, f % cfg.k
        _, w2d = oracle.expert_weights_decoded(p["w13"], p["w13_sf"], p["w2"], p["w2_sf"], e)
        dO = flip_effect(gc[i], gs[i], ref["a_codes"][i], ref["a_scales"][i], w2d,
                         p["alpha2"][e])
        dy[t] += float(oracle.bf16_bits_to_f32(p["rw"][t, j])) * dO
    return dy


def check_layer(p, gpu_out, inter, ref):
    """All parity checks of one moe_forward call against the grouped oracle (see above)."""
    cfg = p["cfg"]
    # bit-exact: x codes and scales, routing
    assert np.array_equal(inter["x_scales"], ref["x_scales"])
    assert np.array_equal(inter["x_codes"], oracle.pack_nibbles(ref["x_codes"]))
    # FC1's f16 operand: the exact values of x's NVFP4 blocks (written below 65536 routed
    # rows; with more, FC1 stages the codes)
    if cfg.T * cfg.k < x_dec_max_rows():
        assert np.array_equal(inter["x_dec"].astype(np.float64),
                              oracle.dequantize_nvfp4(ref["x_codes"], ref["x_scales"]))
    for key in ("sorted_ids", "sorted_row_idx", "expanded_row_idx", "counts", "cumsum"):
        assert np.array_equal(inter[key], ref[key]), key
    # intermediate codes
    gc = unpack(inter["a_codes"])
    st = code_diff_stats(gc, inter["a_scales"], ref["a_codes"], ref["a_scales"])
    assert st["max_step_same_scale"] <= 1, st
    assert st["frac"] <= CODE_DIFF_FRAC, st
    # output, widened by the exact effect of differing codes
    dy = flip_widening(p, gc, inter["a_scales"], ref, st["rows_with_diff"])
    res = check_output(gpu_out, ref["out_f64"], dy)
    # FC2 row exponents: the expert's, for every row of an in-range id
    f, e = ref["sorted_row_idx"], ref["sorted_ids"]
    ok = f >= 0
    assert np.array_equal(inter["o_exp"][f[ok]], out_exponents(p["alpha2"], cfg.I)[e[ok]])
    # amax statistic: per expert max |SiTU output| of the expert's rows
    amax_ref = np.zeros(cfg.E, np.float32)
    np.maximum.at(amax_ref, ref["sorted_ids"], np.max(np.abs(ref["a"]), axis=1))
    assert np.allclose(inter["a_amax"], amax_ref, rtol=1e-4, atol=0)
    return st, res
