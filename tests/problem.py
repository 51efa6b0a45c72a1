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
        dA, qA = oracle.calibrate_intermediate(tokens, x, ids, p["w13"], p["w13_sf"], p["qX"],
                                               alpha1, beta, lam)
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
