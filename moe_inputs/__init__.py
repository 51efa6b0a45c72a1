"""Seeded synthetic inputs for the routed MoE layer.

This module only draws random numbers: it holds none of the layer's arithmetic (no
quantization, no routing, no GEMM).  Tests, the smoke check and the benchmark all draw
their inputs here, so the CPU oracle and the HIP library see identical bytes.

Recipe (every draw is numpy PCG64; each stream has its own SeedSequence entropy
[base_seed, stream_tag, index] so any expert's weights regenerate on their own):
  * x: N(0, 1) fp32, optionally with a fixed random set of round(frac*H) outlier
    columns multiplied by a factor, then rounded once (nearest-even) to BF16.
  * expert ids: top-k without replacement from a popularity p_e ~ (e+1)^-s over the E
    experts (s = 0 is uniform), drawn per token with the Gumbel-top-k trick (equal in law
    to sequential sampling without replacement); ids are listed in draw order.
  * route weights: softmax over the k picks of N(0, 1) logits, in fp32, then BF16.
  * expert weights: W13 [2I, H] and W2 [H, I] per expert, N(0, std) fp32, then BF16.
  * SiTU parameters (when per-expert): beta ~ U(3, 5), lambda ~ U(20, 30), fp32.

BF16 values travel as uint16 bit patterns.
"""

from dataclasses import dataclass
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

BASE_SEED = 20261202

_TAG_X, _TAG_IDS, _TAG_LOGITS, _TAG_W13, _TAG_W2, _TAG_SITU, _TAG_OUTLIER = range(1, 8)


@dataclass(frozen=True)
class LayerConfig:
    """Shape and input distribution of one routed-MoE workload."""
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    zipf_s: float = 0.0            # 0 = uniform distinct experts
    w_std: float = 0.02
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    per_expert_situ: bool = False
    seed_index: int = 0
    weight_seed_index: int = -1     # -1: same as seed_index

    @property
    def wseed(self):
        return self.seed_index if self.weight_seed_index < 0 else self.weight_seed_index


@dataclass(frozen=True)
class RouteConfig:
    """Shape and input distribution of the routing-and-int8-permute workload."""
    name: str
    N: int
    H: int
    E: int
    K: int
    zipf_s: float
    outlier_frac: float
    outlier_mult: float
    seed_index: int = 1


# The workloads: a tiny full layer, routing-only, and the full layer at the TP8-local
# shape H=3584, I=384, E=896, top-16 for decode, mid and prefill batches.
TINY = LayerConfig("tiny_T4_H256_I64_E16_k4", T=4, H=256, I=64, E=16, k=4, w_std=0.05,
                   seed_index=0)
ROUTE_8K = RouteConfig("route_N8192_H7168_E256_K8_zipf1.1_int8", N=8192, H=7168, E=256, K=8,
                       zipf_s=1.1, outlier_frac=0.01, outlier_mult=20.0, seed_index=1)
DECODE_16 = LayerConfig("layer_T16_H3584_I384_E896_k16_uniform", T=16, H=3584, I=384, E=896,
                        k=16, w_std=0.02, seed_index=2)
# The mid and prefill batches use the decode workload's expert weights.
MID_1024 = LayerConfig("layer_T1024_H3584_I384_E896_k16_zipf1.0", T=1024, H=3584, I=384,
                       E=896, k=16, zipf_s=1.0, w_std=0.02, seed_index=3, weight_seed_index=2)
PREFILL_16K = LayerConfig("layer_T16384_H3584_I384_E896_k16_uniform_situE", T=16384, H=3584,
                          I=384, E=896, k=16, w_std=0.02, outlier_frac=0.005,
                          outlier_mult=30.0, per_expert_situ=True, seed_index=4,
                          weight_seed_index=2)

# The edges of the two target bands: the largest decode batch (T=64, uniform picks, as the
# T=16 batch) and the smallest prefill batch (T=4096, as the T=16384 batch).
DECODE_64 = LayerConfig("layer_T64_H3584_I384_E896_k16_uniform", T=64, H=3584, I=384, E=896,
                        k=16, w_std=0.02, seed_index=5, weight_seed_index=2)
PREFILL_4K = LayerConfig("layer_T4096_H3584_I384_E896_k16_uniform_situE", T=4096, H=3584,
                         I=384, E=896, k=16, w_std=0.02, outlier_frac=0.005,
                         outlier_mult=30.0, per_expert_situ=True, seed_index=6,
                         weight_seed_index=2)

LAYER_CONFIGS = {c.name: c for c in (TINY, DECODE_16, MID_1024, PREFILL_16K, DECODE_64,
                                     PREFILL_4K)}


def _rng(seed_index, tag, index=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [BASE_SEED + seed_index, tag, index])))


def f32_to_bf16_bits(a):
    """Round fp32 to BF16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def draw_tokens(n, H, seed_index, outlier_frac=0.0, outlier_mult=1.0):
    """BF16 bits [n, H] of N(0,1) tokens with optional outlier columns."""
    x = _rng(seed_index, _TAG_X).standard_normal((n, H), dtype=np.float32)
    n_out = int(round(outlier_frac * H))
    if n_out:
        cols = _rng(seed_index, _TAG_OUTLIER).choice(H, size=n_out, replace=False)
        x[:, cols] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


def draw_expert_ids(n, E, k, seed_index, zipf_s=0.0):
    """int32 [n, k]: top-k without replacement from p_e ~ (e+1)^-s, Gumbel-top-k."""
    rng = _rng(seed_index, _TAG_IDS)
    logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
    out = np.empty((n, k), np.int32)
    chunk = 2048
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        keys = logp[None, :] + rng.gumbel(size=(m, E))
        top = np.argpartition(-keys, k - 1, axis=1)[:, :k]
        order = np.argsort(-np.take_along_axis(keys, top, axis=1), axis=1, kind="stable")
        out[s:s + m] = np.take_along_axis(top, order, axis=1)
    return out


def draw_route_weights(n, k, seed_index):
    """BF16 bits [n, k]: softmax over the k picks of N(0,1) logits (fp32)."""
    z = _rng(seed_index, _TAG_LOGITS).standard_normal((n, k), dtype=np.float32)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    return f32_to_bf16_bits(p.astype(np.float32))


def draw_expert_weights(cfg: LayerConfig, e):
    """BF16 bits of expert e: W13 [2I, H] (gate rows, then up rows) and W2 [H, I]."""
    w13 = _rng(cfg.wseed, _TAG_W13, e).standard_normal((2 * cfg.I, cfg.H), dtype=np.float32)
    w13 *= np.float32(cfg.w_std)
    w2 = _rng(cfg.wseed, _TAG_W2, e).standard_normal((cfg.H, cfg.I), dtype=np.float32)
    w2 *= np.float32(cfg.w_std)
    return f32_to_bf16_bits(w13), f32_to_bf16_bits(w2)


def draw_all_expert_weights(cfg: LayerConfig, experts=None, threads=None):
    """Stacked BF16 bits W13 [n, 2I, H], W2 [n, H, I] for the listed experts (default all),
    drawn in parallel threads (numpy releases the GIL while filling)."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    n = len(experts)
    w13 = np.empty((n, 2 * cfg.I, cfg.H), np.uint16)
    w2 = np.empty((n, cfg.H, cfg.I), np.uint16)

    def one(i):
        w13[i], w2[i] = draw_expert_weights(cfg, experts[i])

    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(n)))
    return w13, w2


def draw_situ_params(cfg: LayerConfig):
    """(beta [E], lambda [E]) float32, or (None, None) for the default 4 / 25."""
    if not cfg.per_expert_situ:
        return None, None
    rng = _rng(cfg.seed_index, _TAG_SITU)
    beta = rng.uniform(3.0, 5.0, cfg.E).astype(np.float32)
    lam = rng.uniform(20.0, 30.0, cfg.E).astype(np.float32)
    return beta, lam


def draw_layer_tokens(cfg: LayerConfig):
    """x bits [T, H], expert ids [T, k], route-weight bits [T, k] of a layer workload."""
    x = draw_tokens(cfg.T, cfg.H, cfg.seed_index, cfg.outlier_frac, cfg.outlier_mult)
    ids = draw_expert_ids(cfg.T, cfg.E, cfg.k, cfg.seed_index, cfg.zipf_s)
    rw = draw_route_weights(cfg.T, cfg.k, cfg.seed_index)
    return x, ids, rw


def draw_route_inputs(cfg: RouteConfig):
    """x bits [N, H] and expert ids [N, K] of the routing workload."""
    x = draw_tokens(cfg.N, cfg.H, cfg.seed_index, cfg.outlier_frac, cfg.outlier_mult)
    ids = draw_expert_ids(cfg.N, cfg.E, cfg.K, cfg.seed_index, cfg.zipf_s)
    return x, ids
