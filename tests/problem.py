"""Builds complete layer problems (inputs, oracle calibration, oracle-quantized weights).

Test helper: uses ``moe_inputs`` for the random draws and ``oracle`` for every value
derived from them.  Nothing here comes from the HIP path.
"""

import numpy as np

import oracle
from moe_inputs import (LayerConfig, draw_layer_tokens, draw_all_expert_weights,
                        draw_situ_params)


def build_layer_problem(cfg: LayerConfig, calib_tokens=None, w13_bits=None, w2_bits=None,
                        quantize_weights=True):
    """Inputs and every scale of a layer workload.

    Weight amax calibration is per expert; dX over all tokens; dA from the oracle's
    calibration pass over ``calib_tokens`` (default: all tokens).
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
        dA, qA = oracle.calibrate_intermediate(tokens, x, ids, p["w13"], p["w13_sf"], p["w2"],
                                               p["w2_sf"], p["qX"], alpha1, beta, lam)
        p["dA"], p["qA"] = dA, qA
        p["alpha2"] = (dA * sc["dW2"]).astype(np.float32)
    return p


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
            list(ex.map(one, experts))
        E, H, I = cfg.E, cfg.H, cfg.I
        self.experts = experts
        self.w13 = self._View(d13, (E, 2 * I, H // 2))
        self.w13_sf = self._View(s13, (E, 2 * I, H // 16))
        self.w2 = self._View(d2, (E, H, I // 2))
        self.w2_sf = self._View(s2, (E, H, I // 16))


def build_full_problem(cfg, w13_bits, w2_bits, sample_tokens, calib_tokens, wscales=None):
    """A full-shape workload whose weights live on the CPU as BF16 bits (all experts, for
    upload to the GPU) and, for the experts the sampled and calibration tokens touch, as
    oracle-quantized canonical storage.  Scales: per-expert weight amax, global x amax,
    dA from the oracle's calibration pass over ``calib_tokens``."""
    x, ids, rw = draw_layer_tokens(cfg)
    dX, qX = oracle.calibrate_tokens(x)
    if wscales is None:
        wscales = oracle.calibrate_weights(w13_bits) + oracle.calibrate_weights(w2_bits)
    dW13, qW13, dW2, qW2 = wscales
    beta, lam = draw_situ_params(cfg)
    alpha1 = (dX * dW13).astype(np.float32)
    sample_tokens = np.asarray(sample_tokens)
    calib_tokens = np.asarray(calib_tokens)
    used = np.unique(np.concatenate([ids[sample_tokens].ravel(), ids[calib_tokens].ravel()]))
    store = ExpertStore(cfg, qW13, qW2, used)
    cache = {}
    dA, qA = oracle.calibrate_intermediate(calib_tokens, x, ids, store.w13, store.w13_sf,
                                           store.w2, store.w2_sf, qX, alpha1, beta, lam,
                                           weight_cache=cache)
    alpha2 = (dA * dW2).astype(np.float32)
    return dict(cfg=cfg, x=x, ids=ids, rw=rw, beta=beta, lam=lam, qX=np.float32(qX),
                dX=np.float32(dX), qW13=qW13, qW2=qW2, dW13=dW13, dW2=dW2, alpha1=alpha1,
                dA=dA, qA=qA, alpha2=alpha2, w13=store.w13, w13_sf=store.w13_sf, w2=store.w2,
                w2_sf=store.w2_sf, store=store, weight_cache=cache, sample=sample_tokens)
