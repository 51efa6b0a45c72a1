"""The routed MoE layer, step by step: FC1, SiTU, requantization, FC2, finalization.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Cake SiTU backend", intro: BF16 x -> group-16 NVFP4 quantization -> routing -> FC1 ->
SiTU -> NVFP4 requantization -> FC2 -> BF16 weighted finalization; H=3584, I=384,
E=896, top-k=16, int32 expert ids, BF16 route weights.  Section "Prepared weights and
scales": FC1 weights are [E, 2I, H] (stored [E, 768, 1792] packed), FC2 weights
[E, H, I]; the six quant scales qX, FC1 block scales, dX*dW13 [E], qA [E], FC2 block
scales, dA*dW2 [E]; SiTU(g, u) = (4 tanh(g/4) sigmoid(g)) * (25 tanh(u/25)), with
optional per-expert float32 situ_beta / situ_linear_beta replacing 4 / 25.
"Nvfp4 Tensor": the per-expert global scale multiplies after block dequantization.

Readings where the pages are silent:
  * FC1 rows [0, I) are the gate g, rows [I, 2I) the up projection u.
  * An FC dot product is computed exactly (see ``fc_exact``), rounded once to fp32,
    then multiplied by the per-expert alpha in fp32.
  * SiTU is evaluated in float64 on the fp32 g, u, beta, lambda and rounded once to fp32.
  * The requantization groups are 16 consecutive intermediate channels of one routed
    row, with the routed row's expert's qA.
  * Finalization: y[t] = sum_j w[t, j] * O[row of (t, j)] in j order in float64, then one
    round-to-nearest-even to BF16.  Route weights are used as given.
"""

from fractions import Fraction

import numpy as np
from scipy.special import expit

from .codecs import bf16_bits_to_f32, f64_to_bf16_bits
from .nvfp4 import quantize_nvfp4, dequantize_nvfp4, unpack_nibbles
from .calib import global_scale_from_amax
from .routing import route

DEFAULT_SITU_BETA = 4.0
DEFAULT_SITU_LINEAR_BETA = 25.0


def situ(g, u, beta=DEFAULT_SITU_BETA, lam=DEFAULT_SITU_LINEAR_BETA):
    """(beta*tanh(g/beta)*sigmoid(g)) * (lam*tanh(u/lam)) in float64, rounded once to fp32."""
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    b = np.float64(np.float32(beta))
    lm = np.float64(np.float32(lam))
    gate = b * np.tanh(g / b) * expit(g)
    lin = lm * np.tanh(u / lm)
    return (gate * lin).astype(np.float32)


def _round_fraction_to_f32(fr):
    """Nearest float32 to an exact rational, ties to even (only used by the int64 path)."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def fc_exact(a_dec, w_dec):
    """fp32( a_dec @ w_dec.T ) with the dot products computed exactly.

    a_dec [R, K], w_dec [N, K]: float64 NVFP4-decoded values, each an integer multiple of
    2^-10 with magnitude <= 2688, so each product is a multiple of 2^-20.  A float64 sum
    of such terms is exact while every partial sum stays below 2^33 in magnitude, which
    holds when sum |terms| < 2^33 (checked with margin per output); otherwise the sum is
    redone in int64 on the scaled integers (|term| < 2^44, K <= 7168: no overflow) and
    rounded to fp32 exactly.
    """
    a = np.asarray(a_dec, dtype=np.float64)
    w = np.asarray(w_dec, dtype=np.float64)
    s = a @ w.T
    bound = np.abs(a) @ np.abs(w).T
    bad = bound >= 2.0 ** 32
    out = s.astype(np.float32)
    if np.any(bad):
        ai = np.rint(a * 1024.0).astype(np.int64)
        wi = np.rint(w * 1024.0).astype(np.int64)
        for r, n in zip(*np.nonzero(bad)):
            si = int(np.dot(ai[r], wi[n]))
            out[r, n] = _round_fraction_to_f32(Fraction(si, 1 << 20))
    return out


def expert_weights_decoded(w13, w13_sf, w2, w2_sf, e):
    """float64 decoded FC1 [2I, H] and FC2 [H, I] weights of expert e (canonical packing)."""
    w13d = dequantize_nvfp4(unpack_nibbles(w13[e]), w13_sf[e])
    w2d = dequantize_nvfp4(unpack_nibbles(w2[e]), w2_sf[e])
    return w13d, w2d


def expert_rows(xdec_rows, w13d, w2d, alpha1_e, qA_e, alpha2_e, beta_e, lam_e):
    """FC1 -> SiTU -> requant -> FC2 for routed rows of one expert.

    xdec_rows [R, H] float64 decoded NVFP4 token rows; w13d [2I, H], w2d [H, I] decoded
    weights.  Returns h [R, 2I] (fp32 FC1 output after alpha1), a [R, I] (fp32 SiTU),
    the requantized codes [R, I] and scales [R, I/16], and o [R, H] (fp32 FC2 output)."""
    I = w2d.shape[1]
    h = (fc_exact(xdec_rows, w13d) * np.float32(alpha1_e)).astype(np.float32)   # [R, 2I]
    g, u = h[:, :I], h[:, I:]
    a = situ(g, u, beta_e, lam_e)
    a_codes, a_scales = quantize_nvfp4(a, np.float32(qA_e))
    a_dec = dequantize_nvfp4(a_codes, a_scales)
    o = (fc_exact(a_dec, w2d) * np.float32(alpha2_e)).astype(np.float32)        # [R, H]
    return h, a, a_codes, a_scales, o


def _situ_params(E, beta, lam):
    b = np.full(E, DEFAULT_SITU_BETA, np.float32) if beta is None else np.asarray(beta, np.float32)
    lm = np.full(E, DEFAULT_SITU_LINEAR_BETA, np.float32) if lam is None else np.asarray(lam, np.float32)
    return b, lm


def layer_forward(x_bits, expert_ids, rw_bits, w13, w13_sf, w2, w2_sf,
                  qX, alpha1, qA, alpha2, beta=None, lam=None):
    """Grouped (expert-sorted) evaluation of the whole layer.

    x_bits [T, H] uint16 BF16; expert_ids [T, k] int32; rw_bits [T, k] uint16 BF16;
    w13 [E, 2I, H/2] u8, w13_sf [E, 2I, H/16] u8, w2 [E, H, I/2] u8, w2_sf [E, H, I/16] u8;
    qX float32 scalar; alpha1, qA, alpha2 float32 [E]; beta, lam float32 [E] or None.
    Returns a dict with every intermediate (rows in expert-sorted order) and
    ``out`` [T, H] uint16 BF16.
    """
    x_bits = np.asarray(x_bits, np.uint16)
    T, H = x_bits.shape
    k = expert_ids.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    beta_a, lam_a = _situ_params(E, beta, lam)
    x = bf16_bits_to_f32(x_bits)
    x_codes, x_scales = quantize_nvfp4(x, np.float32(qX))
    xdec = dequantize_nvfp4(x_codes, x_scales)
    r = route(expert_ids, E)
    R = T * k
    h_all = np.zeros((R, 2 * I), np.float32)
    a_all = np.zeros((R, I), np.float32)
    ac_all = np.zeros((R, I), np.uint8)
    as_all = np.zeros((R, I // 16), np.uint8)
    o_all = np.zeros((R, H), np.float32)
    start = 0
    for e in range(E):
        cnt = int(r["counts"][e])
        if cnt == 0:
            continue
        pos = np.arange(start, start + cnt)
        tok = r["sorted_row_idx"][pos].astype(np.int64) // k
        w13d, w2d = expert_weights_decoded(w13, w13_sf, w2, w2_sf, e)
        h, a, ac, as_, o = expert_rows(xdec[tok], w13d, w2d, alpha1[e], qA[e], alpha2[e],
                                        beta_a[e], lam_a[e])
        h_all[pos], a_all[pos], ac_all[pos], as_all[pos], o_all[pos] = h, a, ac, as_, o
        start += cnt
    rows = r["expanded_row_idx"].reshape(T, k)
    acc = combine(o_all[rows], rw_bits)
    out = dict(r)
    out.update(x_codes=x_codes, x_scales=x_scales, h=h_all, a=a_all, a_codes=ac_all,
               a_scales=as_all, o=o_all, out_f64=acc, out=f64_to_bf16_bits(acc))
    return out


def combine(o_tk, rw_bits):
    """Finalization before the BF16 rounding: y[t] = sum_j w[t, j] * o[t, j] in j order,
    float64.  o_tk [n, k, H] fp32 FC2 outputs of each token's k routed rows; rw_bits
    [n, k] BF16 route weights (used as given).  The layer output is BF16(y), one
    round-to-nearest-even (``f64_to_bf16_bits``)."""
    o_tk = np.asarray(o_tk)
    wts = bf16_bits_to_f32(np.asarray(rw_bits, np.uint16)).astype(np.float64)
    acc = np.zeros((o_tk.shape[0], o_tk.shape[2]), np.float64)
    for j in range(o_tk.shape[1]):
        acc += wts[:, j:j + 1] * o_tk[:, j].astype(np.float64)
    return acc


def token_forward(tokens, x_bits, expert_ids, rw_bits, w13, w13_sf, w2, w2_sf,
                  qX, alpha1, qA, alpha2, beta=None, lam=None, weight_cache=None):
    """Dense evaluation of selected tokens: each (t, j) goes through expert ids[t, j]
    directly, with no sorting or grouping.

    Returns dict: out [n, H] uint16 BF16, out_f64, and per (t, j) the intermediates
    h [n, k, 2I], a_codes [n, k, I], a_scales [n, k, I/16], o [n, k, H].
    ``weight_cache`` (a dict) may carry decoded expert weights between calls.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    x_bits = np.asarray(x_bits, np.uint16)
    H = x_bits.shape[1]
    k = expert_ids.shape[1]
    E = w13.shape[0]
    I = w2.shape[2] * 2
    beta_a, lam_a = _situ_params(E, beta, lam)
    cache = {} if weight_cache is None else weight_cache
    n = tokens.size
    res = {
        "out_f64": np.zeros((n, H), np.float64),
        "h": np.zeros((n, k, 2 * I), np.float32),
        "a_codes": np.zeros((n, k, I), np.uint8),
        "a_scales": np.zeros((n, k, I // 16), np.uint8),
        "o": np.zeros((n, k, H), np.float32),
        "x_codes": np.zeros((n, H), np.uint8),
        "x_scales": np.zeros((n, H // 16), np.uint8),
    }
    for i, t in enumerate(tokens):
        xc, xs = quantize_nvfp4(bf16_bits_to_f32(x_bits[t:t + 1]), np.float32(qX))
        res["x_codes"][i], res["x_scales"][i] = xc[0], xs[0]
        xdec = dequantize_nvfp4(xc, xs)
        for j in range(k):
            e = int(expert_ids[t, j])
            if e not in cache:
                cache[e] = expert_weights_decoded(w13, w13_sf, w2, w2_sf, e)
            w13d, w2d = cache[e]
            h, _, ac, as_, o = expert_rows(xdec, w13d, w2d, alpha1[e], qA[e], alpha2[e],
                                            beta_a[e], lam_a[e])
            res["h"][i, j], res["a_codes"][i, j], res["a_scales"][i, j] = h[0], ac[0], as_[0]
            res["o"][i, j] = o[0]
            wt = np.float64(bf16_bits_to_f32(np.asarray(rw_bits, np.uint16)[t, j]))
            res["out_f64"][i] += wt * o[0].astype(np.float64)
    res["out"] = f64_to_bf16_bits(res["out_f64"])
    return res


def layer_forward_dense(x_bits, expert_ids, rw_bits, w13, w13_sf, w2, w2_sf,
                        qX, alpha1, qA, alpha2, beta=None, lam=None):
    """Every token through ``token_forward`` (brute force; tiny shapes only)."""
    T = np.asarray(x_bits).shape[0]
    return token_forward(np.arange(T), x_bits, expert_ids, rw_bits, w13, w13_sf, w2, w2_sf,
                         qX, alpha1, qA, alpha2, beta, lam)


def intermediate_amax_per_expert(tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX,
                                 alpha1, beta=None, lam=None, weight_cache=None):
    """Largest |SiTU output| of each expert over the routed rows of the given tokens:
    float32 [E], 0 for an expert none of those rows is routed to (calibration pass)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    E = w13.shape[0]
    I = w2.shape[2] * 2
    beta_a, lam_a = _situ_params(E, beta, lam)
    xc, xs = quantize_nvfp4(bf16_bits_to_f32(np.asarray(x_bits, np.uint16)[tokens]), np.float32(qX))
    xdec = dequantize_nvfp4(xc, xs)
    amax = np.zeros(E, np.float32)
    ids = np.asarray(expert_ids)[tokens]
    for e in np.unique(ids):
        rows = np.nonzero(np.any(ids == e, axis=1))[0]
        if weight_cache is not None and e in weight_cache:
            w13d = weight_cache[e][0]
        else:
            w13d = dequantize_nvfp4(unpack_nibbles(w13[e]), w13_sf[e])
        h = (fc_exact(xdec[rows], w13d) * np.float32(alpha1[e])).astype(np.float32)
        a = situ(h[:, :I], h[:, I:], beta_a[e], lam_a[e])
        amax[e] = np.float32(np.max(np.abs(a)))
    return amax


def intermediate_amax(tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX, alpha1,
                      beta=None, lam=None, weight_cache=None):
    """Largest |SiTU output| over the routed rows of the given tokens (calibration pass)."""
    return np.float32(np.max(intermediate_amax_per_expert(
        tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX, alpha1, beta, lam,
        weight_cache)))


def calibrate_intermediate(tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX, alpha1,
                           beta=None, lam=None, weight_cache=None):
    """Reading taken: one shared dA = amax|SiTU output| / 2688 over a calibration set of
    tokens, expanded to [E] (the page asks for a shared intermediate scale expanded to an
    [E] tensor during model preparation).  Returns (dA [E], qA [E]) float32."""
    E = w13.shape[0]
    amax = intermediate_amax(tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX, alpha1,
                             beta, lam, weight_cache)
    d, q = global_scale_from_amax(amax)
    return np.full(E, d, np.float32), np.full(E, q, np.float32)


def calibrate_intermediate_per_expert(tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX,
                                      alpha1, beta=None, lam=None, weight_cache=None):
    """Per-expert intermediate scales: dA[e] = amax_e / 2688 with amax_e the largest
    |SiTU output| of expert e's routed rows among the calibration tokens (the page's qA is
    a float32 [E] tensor, one value per expert).  Reading taken: an expert with no routed
    row in the calibration set takes the shared scale of the whole set.
    Returns (dA [E], qA [E]) float32."""
    per = intermediate_amax_per_expert(tokens, x_bits, expert_ids, w13, w13_sf, w2, w2_sf, qX,
                                       alpha1, beta, lam, weight_cache)
    shared = np.float32(np.max(per)) if per.size else np.float32(0.0)
    d, q = global_scale_from_amax(np.where(per > 0, per, shared).astype(np.float32))
    return np.asarray(d, np.float32), np.asarray(q, np.float32)
