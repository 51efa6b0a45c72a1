"""Builds complete layer problems (inputs, oracle calibration, oracle-quantized weights).

Test helper: uses ``moe_inputs`` for the random draws and ``oracle`` for every value
derived from them.  Nothing here comes from the HIP path.
"""

import sys

import numpy as np

import oracle
from moe_inputs import (LayerConfig, draw_layer_tokens, draw_all_expert_weights,
                        draw_situ_params)


def build_layer_problem(cfg: LayerConfig, calib_tokens=None, w13_bits=None, w2_bits=None,
                        quantize_weights=True, per_expert_qa=False):
    """Inputs and every scale of a layer workload.

    Weight amax calibration is per expert; dX over all tokens; dA from the oracle's
    calibration pass over ``calib_tokens`` (default: all tokens), one shared value or,
    with ``per_expert_qa``, one value per expert from that expert's own rows.
    With ``quantize_weights`` the canonical NVFP4 weight storage is made by the oracle.
    """
    x, ids, rw = draw_layer_tokens(cfg)
    if w13_bits is None:
        w13_bits, w2_bits = draw_all_expert_weights(cfg)
    sc = oracle.calibrate_layer(x, w13_bits, w2_bits)
    beta, lam = draw_situ_params(cfg)
    alpha1 = (sc["dX"] * sc["dW13"]).astype(np.float32)
    p = dict(cfg=cfg, x=x, ids=ids, rw=rw, w13_bits=w13_bits, w2_bits=w2_bits, beta=beta,
             lam=lam, qX=np.float32(sc["qX"]), dX=np.float32(sc["dX"]), qW13=sc["qW13"],
             qW2=sc["qW2"], dW13=sc["dW13"], dW2=sc["dW2"], alpha1=alpha1)
    if quantize_weights:
        p["w13"], p["w13_sf"] = oracle.quantize_expert_stack(w13_bits, sc["qW13"])
        p["w2"], p["w2_sf"] = oracle.quantize_expert_stack(w2_bits, sc["qW2"])
        tokens = np.arange(cfg.T) if calib_tokens is None else np.asarray(calib_tokens)
        calib = (oracle.calibrate_intermediate_per_expert if per_expert_qa
                 else oracle.calibrate_intermediate)
        dA, qA = calib(tokens, x, ids, p["w13"], p["w13_sf"], p["w2"], p["w2_sf"], p["qX"],
                       alpha1, beta, lam)
        p["dA"], p["qA"] = dA, qA
        p["alpha2"] = (dA * sc["dW2"]).astype(np.float32)
    return p


def constant_weight_problem(cfg: LayerConfig, seed=7):
    """A layer whose FC2 sums reach their bound I * 2688^2: every gate row of an expert holds
    one value a_e, every up row one value b_e and every W2 entry one value c_e (BF16).  Each
    weight then quantizes to code 6 with block scale 448 (decoded 2688), FC1 gives a token
    one gate and one up value, so its SiTU output is the same in every channel, and with a
    qA per expert the expert's largest-output token requantizes to code 6, scale 448 in
    every block: its FC2 sums are +-I * 2688^2."""
    from moe_inputs import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    E, H, I = cfg.E, cfg.H, cfg.I
    w13 = np.empty((E, 2 * I, H), np.uint16)
    w2 = np.empty((E, H, I), np.uint16)
    for e in range(E):
        a, b, c = rng.uniform(0.01, 0.05, 3).astype(np.float32)
        sign = np.float32(1.0 if e % 2 == 0 else -1.0)
        w13[e, :I] = f32_to_bf16_bits(np.full((I, H), a, np.float32))
        w13[e, I:] = f32_to_bf16_bits(np.full((I, H), b, np.float32))
        w2[e] = f32_to_bf16_bits(np.full((H, I), sign * c, np.float32))
    return build_layer_problem(cfg, w13_bits=w13, w2_bits=w2, per_expert_qa=True)


def oracle_forward(p):
    return oracle.layer_forward(p["x"], p["ids"], p["rw"], p["w13"], p["w13_sf"], p["w2"],
                                p["w2_sf"], p["qX"], p["alpha1"], p["qA"], p["alpha2"],
                                p["beta"], p["lam"])


def oracle_dense(p, tokens=None, weight_cache=None):
    toks = np.arange(p["cfg"].T) if tokens is None else tokens
    return oracle.token_forward(toks, p["x"], p["ids"], p["rw"], p["w13"], p["w13_sf"], p["w2"],
                                p["w2_sf"], p["qX"], p["alpha1"], p["qA"], p["alpha2"],
                                p["beta"], p["lam"], weight_cache=weight_cache)


class ExpertStore:
    """Array-like canonical NVFP4 weights of a subset of experts, quantized by the oracle.

    ``w13[e]``, ``w13_sf[e]``, ``w2[e]``, ``w2_sf[e]`` work for the experts given at
    construction (drawn and quantized in parallel threads); ``.shape`` is the full
    [E, ...] shape so the oracle functions can read E and I from it.
    """

    class _View:
        def __init__(self, data, shape):
            self._data, self.shape = data, shape

        def __getitem__(self, e):
            return self._data[int(e)]

    def __init__(self, cfg, qW13, qW2, experts, threads=16):
        from concurrent.futures import ThreadPoolExecutor
        from moe_inputs import draw_expert_weights
        experts = sorted(set(int(e) for e in experts))
        d13, s13, d2, s2 = {}, {}, {}, {}

        def one(e):
            w13b, w2b = draw_expert_weights(cfg, e)
            a, b = oracle.quantize_expert_stack(w13b[None], qW13[e:e + 1])
            c, d = oracle.quantize_expert_stack(w2b[None], qW2[e:e + 1])
            d13[e], s13[e], d2[e], s2[e] = a[0], b[0], c[0], d[0]

        with ThreadPoolExecutor(threads) as ex:
            for n, _ in enumerate(ex.map(one, experts)):
                if (n + 1) % 128 == 0:
                    print(f"    quantized {n + 1}/{len(experts)} experts", file=sys.stderr,
                          flush=True)
        E, H, I = cfg.E, cfg.H, cfg.I
        self.experts = experts
        self.w13 = self._View(d13, (E, 2 * I, H // 2))
        self.w13_sf = self._View(s13, (E, 2 * I, H // 16))
        self.w2 = self._View(d2, (E, H, I // 2))
        self.w2_sf = self._View(s2, (E, H, I // 16))


def build_full_problem(cfg, w13_bits, w2_bits, select, wscales=None, per_expert_qa=False):
    """A full-shape workload whose weights live on the CPU as BF16 bits (all experts, for
    upload to the GPU) and, for the experts the checked rows touch, as oracle-quantized
    canonical storage.  ``select(ids)`` returns (pairs [n, 2] of (token, pick) routed rows
    whose intermediate and FC2 rows are checked, tokens whose whole output is checked).
    Scales: per-expert weight amax, global x amax, dA from the oracle's calibration pass
    over the first 8 checked tokens (shared, or per expert with ``per_expert_qa``)."""
    x, ids, rw = draw_layer_tokens(cfg)
    pairs, tokens = select(ids)
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    tokens = np.asarray(tokens, np.int64)
    dX, qX = oracle.calibrate_tokens(x)
    if wscales is None:
        wscales = oracle.calibrate_weights(w13_bits) + oracle.calibrate_weights(w2_bits)
    dW13, qW13, dW2, qW2 = wscales
    beta, lam = draw_situ_params(cfg)
    alpha1 = (dX * dW13).astype(np.float32)
    used = np.unique(np.concatenate([ids[pairs[:, 0], pairs[:, 1]], ids[tokens].ravel()]))
    store = ExpertStore(cfg, qW13, qW2, used)
    calib = (oracle.calibrate_intermediate_per_expert if per_expert_qa
             else oracle.calibrate_intermediate)
    dA, qA = calib(tokens[:8], x, ids, store.w13, store.w13_sf, store.w2, store.w2_sf, qX,
                   alpha1, beta, lam)
    alpha2 = (dA * dW2).astype(np.float32)
    return dict(cfg=cfg, x=x, ids=ids, rw=rw, beta=beta, lam=lam, qX=np.float32(qX),
                dX=np.float32(dX), qW13=qW13, qW2=qW2, dW13=dW13, dW2=dW2, alpha1=alpha1,
                dA=dA, qA=qA, alpha2=alpha2, w13=store.w13, w13_sf=store.w13_sf, w2=store.w2,
                w2_sf=store.w2_sf, store=store, pairs=pairs, tokens=tokens)


def oracle_pairs(p, pairs, threads=16):
    """The oracle's FC1 -> SiTU -> requantization -> FC2 of routed rows pairs [(t, j)],
    evaluated expert by expert (each expert's weights decoded once, experts in parallel
    threads).  Returns per pair: a_codes [n, I], a_scales [n, I/16], o [n, H] fp32; and the
    NVFP4 codes and scales of the tokens involved."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = p["cfg"]
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    t, j = pairs[:, 0], pairs[:, 1]
    e_of = np.asarray(p["ids"])[t, j]
    toks, tok_row = np.unique(t, return_inverse=True)
    xc, xs = oracle.quantize_nvfp4(oracle.bf16_bits_to_f32(p["x"][toks]), np.float32(p["qX"]))
    xdec = oracle.dequantize_nvfp4(xc, xs)
    n, H, I = pairs.shape[0], cfg.H, cfg.I
    beta = np.full(cfg.E, 4.0, np.float32) if p["beta"] is None else p["beta"]
    lam = np.full(cfg.E, 25.0, np.float32) if p["lam"] is None else p["lam"]
    res = {"a_codes": np.zeros((n, I), np.uint8), "a_scales": np.zeros((n, I // 16), np.uint8),
           "o": np.zeros((n, H), np.float32),
           "x_codes": xc, "x_scales": xs, "tokens": toks}

    def one(e):
        sel = np.nonzero(e_of == e)[0]
        w13d, w2d = oracle.expert_weights_decoded(p["w13"], p["w13_sf"], p["w2"], p["w2_sf"], e)
        _, _, ac, as_, o = oracle.expert_rows(xdec[tok_row[sel]], w13d, w2d, p["alpha1"][e],
                                              p["qA"][e], p["alpha2"][e], beta[e], lam[e])
        return sel, ac, as_, o

    experts = np.unique(e_of)
    with ThreadPoolExecutor(threads) as ex:
        for n, (sel, ac, as_, o) in enumerate(ex.map(one, experts)):
            res["a_codes"][sel], res["a_scales"][sel], res["o"][sel] = ac, as_, o
            if (n + 1) % 128 == 0:
                print(f"    oracle rows of {n + 1}/{experts.size} experts", flush=True)
    return res
