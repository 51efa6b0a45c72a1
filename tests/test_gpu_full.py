"""GPU parity at the full TP8-local shape (H=3584, I=384, E=896, top-16) for the decode
(T=16), mid (T=1024, Zipf 1.0) and prefill (T=16384, per-expert SiTU, outliers) batches,
in the launch configuration the benchmark times.  Routing is compared bit for bit in full;
the layer output, the input codes and the intermediate codes on sampled tokens that the
oracle evaluates one by one (first, second, middle, last two)."""

import sys

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import DECODE_16, MID_1024, PREFILL_16K, draw_all_expert_weights
from tests.problem import build_full_problem, oracle_dense
from tests.gpu_harness import dev, host, quantize_on_gpu, prepare, DeviceLayer
from tests import compare

pytestmark = pytest.mark.gpu


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


def _samples(T):
    return np.unique(np.array([0, 1, T // 2, T - 2, T - 1])) if T > 16 else np.arange(T)


@pytest.mark.parametrize("cfg", [DECODE_16, MID_1024, PREFILL_16K], ids=lambda c: c.name)
def test_full_layer_parity(full_weights, cfg):
    fw = full_weights
    sample = _samples(cfg.T)
    _say(f"full layer {cfg.name}: building oracle problem")
    p = build_full_problem(cfg, fw["w13_bits"], fw["w2_bits"], sample, np.arange(min(8, cfg.T)),
                           wscales=fw["wscales"])
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.k
    # the GPU-quantized weights of every expert the oracle touches equal the oracle's
    ex = np.array(p["store"].experts)
    g13 = host(fw["c13"].view(E, 2 * I, H // 2)[torch.from_numpy(ex).cuda()])
    g13s = host(fw["s13"].view(E, 2 * I, H // 16)[torch.from_numpy(ex).cuda()])
    g2 = host(fw["c2"].view(E, H, I // 2)[torch.from_numpy(ex).cuda()])
    g2s = host(fw["s2"].view(E, H, I // 16)[torch.from_numpy(ex).cuda()])
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
    for key, rk in (("sorted_ids", "sorted_ids"), ("sorted_row_idx", "sorted_row_idx"),
                    ("expanded_row_idx", "expanded_row_idx"), ("counts", "counts"),
                    ("cumsum", "cumsum")):
        assert np.array_equal(inter[key], r[rk]), key
    # oracle on the sampled tokens
    _say(f"full layer {cfg.name}: oracle on tokens {sample.tolist()}")
    ref = oracle_dense(p, sample, weight_cache=p["weight_cache"])
    assert np.array_equal(inter["x_codes"][sample], oracle.pack_nibbles(ref["x_codes"]))
    assert np.array_equal(inter["x_scales"][sample], ref["x_scales"])
    if cfg.T * k < compare.X_DEC_MAX_ROWS:
        assert np.array_equal(inter["x_dec"][sample].astype(np.float64),
                              oracle.dequantize_nvfp4(ref["x_codes"], ref["x_scales"]))
    pos = inter["expanded_row_idx"].reshape(cfg.T, k)[sample]            # [n, k]
    gc = compare.unpack(inter["a_codes"][pos.ravel()])
    gs = inter["a_scales"][pos.ravel()]
    rc = ref["a_codes"].reshape(-1, I)
    rs = ref["a_scales"].reshape(-1, I // 16)
    st = compare.code_diff_stats(gc, gs, rc, rs)
    _say(f"  intermediate code diffs {st['n_diff']}/{st['n_codes']}")
    assert st["max_step_same_scale"] <= 1, st
    assert st["frac"] <= compare.CODE_DIFF_FRAC, st
    dy = np.zeros((sample.size, H))
    for row in st["rows_with_diff"]:
        n, j = divmod(int(row), k)
        e = int(p["ids"][sample[n], j])
        w2d = p["weight_cache"][e][1]
        dO = compare.flip_effect(gc[row], gs[row], rc[row], rs[row], w2d, p["alpha2"][e])
        dy[n] += float(oracle.bf16_bits_to_f32(p["rw"][sample[n], j])) * dO
    ratio = compare.check_output(out[sample], ref["out"], dy)
    _say(f"  worst err/(2e-2 rms) {ratio:.3f}")
