"""GPU parity at the full TP8-local shape (H=3584, I=384, E=896, top-16) for every batch
the benchmark times, in its launch configuration: decode (T=16: the fused small-batch
kernel), T=64 (small tiles, separate FC1 and FC2), mid (T=1024, Zipf 1.0: both FC1 tile
lists in one launch), T=4096 (per-expert SiTU: code-staged FC1, token-resident FC2 on big
tiles) and prefill (T=16384, per-expert SiTU, outliers: weight-stationary FC2).

Routing is compared bit for bit in full.  The oracle then evaluates routed rows chosen by
their position in the expert-sorted order (the GEMMs' token tiles are runs of 16-row blocks
of one expert's rows, so these cover every position a row can take in a tile):
  * every row of a few experts: the most loaded one, up to three whose row count leaves
    a ragged last 16-row block, a median one and the least loaded one -- their
    intermediate NVFP4 codes and their FC2 output rows are compared row by row;
  * the whole output of 64 tokens: those of the first and last row of every 16-row block
    of the two most loaded experts, then the first and last token (all 16 at T=16), with
    the input codes of those tokens and the codes and FC2 rows of all their picks.
The T=1024, T=4096 and T=16384 batches take a per-expert qA (each expert calibrated on
its own rows of the calibration tokens), the decode batches one shared qA."""

import sys

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import (DECODE_16, DECODE_64, MID_1024, PREFILL_4K, PREFILL_16K,
                        draw_all_expert_weights)
from tests.problem import build_full_problem, oracle_pairs
from tests.gpu_harness import dev, host, quantize_on_gpu, prepare, DeviceLayer
from tests import compare

pytestmark = pytest.mark.gpu

N_TOKENS = 64


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def full_weights():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    cfg = DECODE_16
    _say("drawing full-shape expert weights")
    w13_bits, w2_bits = draw_all_expert_weights(cfg)
    wscales = oracle.calibrate_weights(w13_bits) + oracle.calibrate_weights(w2_bits)
    dW13, qW13, dW2, qW2 = wscales
    E, H, I = cfg.E, cfg.H, cfg.I
    _say("quantizing expert weights on the GPU")
    w = dev(w13_bits)
    c13, s13 = quantize_on_gpu(w, E, 2 * I, H, dev(qW13))
    del w
    w = dev(w2_bits)
    c2, s2 = quantize_on_gpu(w, E, H, I, dev(qW2))
    del w
    prepared = prepare(cfg, c13, s13, c2, s2)
    torch.cuda.synchronize()
    yield dict(w13_bits=w13_bits, w2_bits=w2_bits, wscales=wscales, c13=c13, s13=s13, c2=c2,
               s2=s2, prepared=prepared)
    torch.cuda.synchronize()


def selection(cfg):
    """select(ids) for build_full_problem: (pairs checked row by row, tokens checked)."""
    def select(ids):
        T, k, E = cfg.T, cfg.k, cfg.E
        if T <= N_TOKENS:
            t, j = np.meshgrid(np.arange(T), np.arange(k), indexing="ij")
            return np.stack([t.ravel(), j.ravel()], 1), np.arange(T)
        r = oracle.route(ids, E)
        counts = r["counts"].astype(np.int64)
        start = r["cumsum"].astype(np.int64) - counts
        order = np.argsort(-counts, kind="stable")
        nz = [int(e) for e in order if counts[e] > 0]
        chosen = [nz[0]]
        chosen += [e for e in nz[1:] if counts[e] % 16 and counts[e] > 16][:3]
        chosen += [e for e in (nz[len(nz) // 2], nz[-1]) if e not in chosen]
        rows = np.concatenate([np.arange(start[e], start[e] + counts[e]) for e in chosen])
        tok = []
        for e in nz[:2]:
            for b0 in range(0, int(counts[e]), 16):
                for pos in (b0, min(b0 + 15, int(counts[e]) - 1)):
                    tok.append(int(r["sorted_row_idx"][start[e] + pos]) // k)
        tok = list(dict.fromkeys(tok))                   # first occurrences, in order
        half = N_TOKENS // 2 - 1
        # as many from each of the two experts' blocks, then the first and last token
        in_first = set((r["sorted_row_idx"][start[nz[0]]:start[nz[0]] + counts[nz[0]]] // k).tolist())
        first = [t for t in tok if t in in_first]
        second = [t for t in tok if t not in in_first]
        tokens = list(dict.fromkeys(first[:half] + second[:half] + [0, T - 1]))
        # top up to N_TOKENS: the remaining block-edge tokens, then the tokens of the
        # experts compared row by row, then evenly spaced ones (a batch whose two most
        # loaded experts have few blocks, T=4096, needs all three)
        extra = tok + (r["sorted_row_idx"][rows] // k).tolist() + \
            np.linspace(0, T - 1, N_TOKENS).astype(np.int64).tolist()
        for t in extra:
            if len(tokens) >= N_TOKENS:
                break
            if t not in tokens:
                tokens.append(int(t))
        tokens = np.array(tokens[:N_TOKENS])
        flat = r["sorted_row_idx"][rows].astype(np.int64)
        tj = np.stack([flat // k, flat % k], 1)
        t2, j2 = np.meshgrid(tokens, np.arange(k), indexing="ij")
        tj = np.concatenate([tj, np.stack([t2.ravel(), j2.ravel()], 1)])
        return np.unique(tj, axis=0), tokens
    return select


CASES = [(DECODE_16, False), (DECODE_64, False), (MID_1024, True), (PREFILL_4K, True),
         (PREFILL_16K, True)]


# the oracle side of one case takes one to two minutes of host time (hundreds of experts)
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,per_expert_qa", CASES,
                         ids=[f"{c.name}{'_qa_per_expert' if q else ''}" for c, q in CASES])
def test_full_layer_parity(full_weights, cfg, per_expert_qa):
    fw = full_weights
    E, H, I, k, T = cfg.E, cfg.H, cfg.I, cfg.k, cfg.T
    _say(f"full layer {cfg.name}: building oracle problem")
    p = build_full_problem(cfg, fw["w13_bits"], fw["w2_bits"], selection(cfg),
                           wscales=fw["wscales"], per_expert_qa=per_expert_qa)
    if per_expert_qa:
        assert len(np.unique(p["qA"])) > 16
    pairs, tokens = p["pairs"], p["tokens"]
    assert tokens.size == min(T, N_TOKENS)
    # the GPU-quantized weights of every expert the oracle touches equal the oracle's
    ex = np.array(p["store"].experts)
    sel = torch.from_numpy(ex).cuda()
    g13 = host(fw["c13"].view(E, 2 * I, H // 2)[sel])
    g13s = host(fw["s13"].view(E, 2 * I, H // 16)[sel])
    g2 = host(fw["c2"].view(E, H, I // 2)[sel])
    g2s = host(fw["s2"].view(E, H, I // 16)[sel])
    for n, e in enumerate(ex):
        assert np.array_equal(g13[n], p["w13"][e]) and np.array_equal(g13s[n], p["w13_sf"][e])
        assert np.array_equal(g2[n], p["w2"][e]) and np.array_equal(g2s[n], p["w2_sf"][e])
    _say(f"full layer {cfg.name}: moe_forward on the GPU")
    L = DeviceLayer(p, fw["prepared"])
    out = host(L.forward(), np.uint16)
    torch.cuda.synchronize()
    inter = L.intermediates()
    # routing: bit-exact in full
    r = oracle.route(p["ids"], E)
    for key in ("sorted_ids", "sorted_row_idx", "expanded_row_idx", "counts", "cumsum"):
        assert np.array_equal(inter[key], r[key]), key
    _say(f"  oracle on {pairs.shape[0]} routed rows over {ex.size} experts, "
         f"{tokens.size} whole tokens")
    ref = oracle_pairs(p, pairs)
    # input codes of the tokens involved
    assert np.array_equal(inter["x_codes"][ref["tokens"]], oracle.pack_nibbles(ref["x_codes"]))
    assert np.array_equal(inter["x_scales"][ref["tokens"]], ref["x_scales"])
    if T * k < compare.x_dec_max_rows():
        assert np.array_equal(inter["x_dec"][ref["tokens"]].astype(np.float64),
                              oracle.dequantize_nvfp4(ref["x_codes"], ref["x_scales"]))
    # intermediate codes, row by row
    flat = pairs[:, 0] * k + pairs[:, 1]
    pos = inter["expanded_row_idx"][flat]
    gc = compare.unpack(inter["a_codes"][pos])
    gs = inter["a_scales"][pos]
    st = compare.code_diff_stats(gc, gs, ref["a_codes"], ref["a_scales"])
    _say(f"  intermediate code diffs {st['n_diff']}/{st['n_codes']}")
    assert st["max_step_same_scale"] <= 1, st
    assert st["frac"] <= compare.CODE_DIFF_FRAC, st
    dO = np.zeros((pairs.shape[0], H))
    for i in st["rows_with_diff"]:
        e = int(p["ids"][pairs[i, 0], pairs[i, 1]])
        _, w2d = oracle.expert_weights_decoded(p["w13"], p["w13_sf"], p["w2"], p["w2_sf"], e)
        dO[i] = compare.flip_effect(gc[i], gs[i], ref["a_codes"][i], ref["a_scales"][i], w2d,
                                    p["alpha2"][e])
    # FC2 output rows, row by row.  Each row is stored as f16(O * 2^s) with its expert's
    # exponent s = clamp(141 - E, -126, 126), E the fp32 exponent of |alpha2| * I * 2688^2
    # (from the bound |FC2 sum| <= I * 2688^2, so that every stored value is below 2^15)
    s_row = inter["o_exp"][flat].astype(np.int64)
    assert np.array_equal(s_row, compare.out_exponents(p["alpha2"], I)[p["ids"][pairs[:, 0], pairs[:, 1]]])
    # 11 significant bits of the 32-column segment's largest value (fp32 accumulation and
    # scaling add less than another 2^-11 of it), down to f16's subnormal quantum
    o_gpu = inter["o_rows"][flat]
    seg = np.repeat(np.max(np.abs(ref["o"]).reshape(-1, H // 32, 32), axis=2), 32, axis=1)
    err = np.abs(o_gpu - ref["o"])
    tol = 2.0 ** -10 * seg + np.ldexp(1.0, -24 - s_row)[:, None] + np.abs(dO)
    assert np.all(err <= tol), (f"{int((err > tol).sum())} FC2 output values off; "
                                f"worst row {int(np.argmax((err > tol).sum(1)))}")
    # whole-token outputs against the oracle's unrounded finalization
    index = {(int(t), int(j)): i for i, (t, j) in enumerate(pairs)}
    rows_tk = np.array([[index[(int(t), j)] for j in range(k)] for t in tokens])
    want = oracle.combine(ref["o"][rows_tk], p["rw"][tokens])
    wts = oracle.bf16_bits_to_f32(p["rw"][tokens]).astype(np.float64)
    dy = np.einsum("nk,nkh->nh", wts, dO[rows_tk])
    res = compare.check_output(out[tokens], want, dy)
    _say(f"  {compare.fmt(res)}")
