"""GPU parity of the HIP library against the CPU oracle: quantization, routing, the int8
routing primitive, and the whole layer at small shapes and edge cases.  Every call goes
through the C ABI (routed_moe_layer_amd)."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_moe_layer_amd as rm
from moe_inputs import (TINY, ROUTE_8K, LayerConfig, draw_expert_ids, draw_route_inputs,
                        f32_to_bf16_bits)
from tests.problem import build_layer_problem, constant_weight_problem, oracle_forward
from tests.gpu_harness import (dev, host, empty_bytes, check_guard, quantize_on_gpu, prepare,
                               DeviceLayer)
from tests import compare

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    yield
    torch.cuda.synchronize()


def _wide_rows(seed, n, K):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((n, K)).astype(np.float32)
    v *= np.exp(rng.uniform(-10, 6, (n, 1))).astype(np.float32)
    v[rng.random((n, K)) < 0.03] = 0.0
    v[rng.random((n, K)) < 0.01] *= -1e-6
    return f32_to_bf16_bits(v)


@pytest.mark.parametrize("groups,rows,K", [(1, 1, 16), (1, 37, 256), (3, 50, 3584), (5, 7, 384)])
def test_quantize_nvfp4_bit_exact(groups, rows, K):
    _say(f"quantize groups={groups} rows={rows} K={K}")
    bits = _wide_rows(groups * 1000 + rows, groups * rows, K)
    q = np.exp(np.random.default_rng(K).uniform(-3, 9, groups)).astype(np.float32)
    codes, scales = quantize_on_gpu(dev(bits), groups, rows, K, dev(q))
    torch.cuda.synchronize()
    qrow = np.repeat(q, rows)
    want_c, want_s = oracle.quantize_nvfp4(oracle.bf16_bits_to_f32(bits), qrow)
    assert np.array_equal(host(scales), want_s)
    assert np.array_equal(host(codes), oracle.pack_nibbles(want_c))


def test_quantize_nvfp4_ties_and_neighbours_bit_exact():
    """Blocks whose amax is 6 with q within 2^-20 of 1 get the scale 1.0 and an encode
    factor equal to q, so v*enc lands exactly on every E2M1 tie (q = 1) or one to a few
    fp32 ulps on either side of it."""
    _say("quantize ties")
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0],
                    np.float32)
    row = np.concatenate([[6.0], ties, [0.0]]).astype(np.float32)
    rows = np.stack([row, -row, row[::-1].copy()])
    qs = np.array([1.0, 1 + 2 ** -20, 1 - 2 ** -20, 1 + 2 ** -23, 1 - 2 ** -24, 1 + 3 * 2 ** -23],
                  np.float32)
    bits = np.tile(f32_to_bf16_bits(rows), (len(qs), 1))
    codes, scales = quantize_on_gpu(dev(bits), len(qs), rows.shape[0], 16, dev(qs))
    torch.cuda.synchronize()
    want_c, want_s = oracle.quantize_nvfp4(oracle.bf16_bits_to_f32(bits), np.repeat(qs, 3))
    assert np.all(want_s == 0x38)
    assert np.array_equal(host(scales), want_s)
    assert np.array_equal(host(codes), oracle.pack_nibbles(want_c))


def _route_on_gpu(ids, E):
    n, K = ids.shape
    H = 8
    x = np.zeros((n, H), np.uint16)
    R = n * K
    ex = torch.empty((R, H), dtype=torch.int16, device="cuda")
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    cs = torch.empty(E, dtype=torch.int32, device="cuda")
    sid = torch.empty(R, dtype=torch.int32, device="cuda")
    sri = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = empty_bytes(rm.moe_route_workspace_size(n, K, E), fill=0xFF)
    rm.moe_route(rm.MoeDims(H, 0, E, K), n, dev(x), dev(ids.astype(np.int32)),
                 rm.MOE_QUANT_NONE, None, sid, sri, eri, cs, ex, None, ws)
    torch.cuda.synchronize()
    return {"expanded_row_idx": host(eri), "cumsum": host(cs), "sorted_ids": host(sid),
            "sorted_row_idx": host(sri)}


ROUTE_CASES = [
    ("T1_k16_E896", 1, 16, 896, 0.0),
    ("T4_k4_E16", 4, 4, 16, 0.0),
    ("T16_k16_E896", 16, 16, 896, 0.0),
    ("T33_k3_E5_zipf", 33, 3, 5, 1.5),
    ("T1000_k8_E256_zipf1.1", 1000, 8, 256, 1.1),
    ("T1024_k16_E896_zipf1.0", 1024, 16, 896, 1.0),
    ("T16384_k16_E896", 16384, 16, 896, 0.0),
    ("T700_k1_E1", 700, 1, 1, 0.0),
    ("T300_k64_E4096", 300, 64, 4096, 0.5),
    # boundary of the single-workgroup router (at most 1024 ids) and just past it
    ("T64_k16_E896", 64, 16, 896, 0.8),
    ("T65_k16_E896", 65, 16, 896, 0.8),
    ("T16_k64_E3000", 16, 64, 3000, 0.3),
]


@pytest.mark.parametrize("name,T,k,E,zipf", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_bit_exact(name, T, k, E, zipf):
    _say(f"route {name}")
    ids = draw_expert_ids(T, E, k, seed_index=900 + T, zipf_s=zipf)
    got = _route_on_gpu(ids, E)
    want = oracle.route(ids, E)
    for key in ("expanded_row_idx", "cumsum", "sorted_ids", "sorted_row_idx"):
        assert np.array_equal(got[key], want[key]), key


def test_route_with_duplicates_and_one_hot_expert():
    _say("route duplicates")
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 4, (2000, 6)).astype(np.int32)
    ids[::7] = 2                                        # rows entirely on one expert
    got = _route_on_gpu(ids, 10)
    want = oracle.route(ids, 10)
    for key in want:
        if key in got:
            assert np.array_equal(got[key], want[key]), key


@pytest.mark.parametrize("T", [20, 300], ids=["one_workgroup", "tiled"])
def test_route_drops_out_of_range_ids(T):
    """Ids outside [0, E) break the caller's contract; the library documents that they
    are dropped (gather-map entry -1) and the valid ids are sorted stably among
    themselves.  Expected values: a stable argsort of the valid subset."""
    _say(f"route out-of-range ids T={T}")
    E, K = 40, 16
    rng = np.random.default_rng(77 + T)
    ids = rng.integers(0, E, (T, K)).astype(np.int32)
    bad = rng.random((T, K)) < 0.1
    ids[bad] = rng.choice(np.array([-1, E, E + 7, -100], np.int32), size=int(bad.sum()))
    got = _route_on_gpu(ids, E)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    nv = order.size
    assert np.array_equal(got["sorted_row_idx"][:nv], order)
    assert np.array_equal(got["sorted_ids"][:nv], flat[order])
    assert np.all(got["sorted_row_idx"][nv:] == -1) and np.all(got["sorted_ids"][nv:] == -1)
    want = np.full(flat.size, -1, np.int64)
    want[order] = np.arange(nv)
    assert np.array_equal(got["expanded_row_idx"], want)
    assert np.array_equal(got["cumsum"], np.cumsum(np.bincount(flat[valid], minlength=E)))


def test_route_more_than_2_21_ids():
    """2.56 M routed rows: the expert scan's packed row totals need more than 21 bits."""
    _say("route 40000 x 64 ids")
    ids = draw_expert_ids(40000, 256, 64, seed_index=1400, zipf_s=1.2)
    got = _route_on_gpu(ids, 256)
    want = oracle.route(ids, 256)
    for key in ("expanded_row_idx", "cumsum", "sorted_ids", "sorted_row_idx"):
        assert np.array_equal(got[key], want[key]), key


def test_route_int8_full_size_bit_exact():
    cfg = ROUTE_8K
    _say(f"route int8 {cfg.name}")
    x, ids = draw_route_inputs(cfg)
    N, K, E, H = cfg.N, cfg.K, cfg.E, cfg.H
    R = N * K
    ex = torch.empty((R, H), dtype=torch.int8, device="cuda")
    esc = torch.empty(R, dtype=torch.float32, device="cuda")
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    cs = torch.empty(E, dtype=torch.int32, device="cuda")
    sid = torch.empty(R, dtype=torch.int32, device="cuda")
    sri = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = empty_bytes(rm.moe_route_workspace_size(N, K, E))
    rm.moe_route(rm.MoeDims(H, 0, E, K), N, dev(x), dev(ids), rm.MOE_QUANT_INT8_ROW_DYNAMIC, None,
                 sid, sri, eri, cs, ex, esc, ws)
    torch.cuda.synchronize()
    want = oracle.route_int8(oracle.bf16_bits_to_f32(x), ids, E)
    assert np.array_equal(host(eri), want["expanded_row_idx"])
    assert np.array_equal(host(cs), want["cumsum"])
    assert np.array_equal(host(sid), want["sorted_ids"])
    assert np.array_equal(host(sri), want["sorted_row_idx"])
    assert np.array_equal(host(esc), want["expanded_scale"])
    assert np.array_equal(host(ex), want["expanded_x"])


@pytest.mark.parametrize("case", ["route_N8192_H7168_E256_K8", "layer_T16384_H3584_E896_k16"])
def test_route_nvfp4_full_size_bit_exact(case):
    """moe_route with the layer's group-16 NVFP4 quantization: every token quantized once
    with qX and its codes and E4M3 scales moved to its k expert-sorted rows.  Expected: the
    oracle's quantize_nvfp4 of each token and its route(), bit for bit."""
    from moe_inputs import PREFILL_16K, draw_layer_tokens
    _say(f"route nvfp4 {case}")
    if case.startswith("route"):
        x, ids = draw_route_inputs(ROUTE_8K)
        E = ROUTE_8K.E
    else:
        x, ids, _ = draw_layer_tokens(PREFILL_16K)
        E = PREFILL_16K.E
    N, H = x.shape
    K = ids.shape[1]
    R = N * K
    _, qX = oracle.calibrate_tokens(x)
    d = rm.MoeDims(H, 0, E, K)
    ex = torch.empty((R, H // 2), dtype=torch.uint8, device="cuda")
    esf = torch.empty((R, H // 16), dtype=torch.uint8, device="cuda")
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    cs = torch.empty(E, dtype=torch.int32, device="cuda")
    sid = torch.empty(R, dtype=torch.int32, device="cuda")
    sri = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = empty_bytes(rm.moe_workspace_size(d, N, rm.MOE_QUANT_NONE), fill=0xFF)
    rm.moe_route(d, N, dev(x), dev(ids), rm.MOE_QUANT_NVFP4_G16,
                 dev(np.array([qX], np.float32)), sid, sri, eri, cs, ex, esf, ws)
    torch.cuda.synchronize()
    check_guard(ws)
    r = oracle.route(ids, E)
    for key, got in (("sorted_ids", sid), ("sorted_row_idx", sri), ("expanded_row_idx", eri),
                     ("cumsum", cs)):
        assert np.array_equal(host(got), r[key]), key
    codes, scales = oracle.quantize_nvfp4(oracle.bf16_bits_to_f32(x), np.float32(qX))
    tok = r["sorted_row_idx"] // K
    assert np.array_equal(host(esf), scales[tok])
    assert np.array_equal(host(ex), oracle.pack_nibbles(codes)[tok])


def test_route_bf16_copy_mode():
    _say("route bf16 copy")
    rng = np.random.default_rng(4)
    N, K, E, H = 300, 4, 7, 136
    x = f32_to_bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    ids = draw_expert_ids(N, E, K, seed_index=44)
    ex = torch.empty((N * K, H), dtype=torch.int16, device="cuda")
    eri = torch.empty(N * K, dtype=torch.int32, device="cuda")
    cs = torch.empty(E, dtype=torch.int32, device="cuda")
    ws = empty_bytes(rm.moe_route_workspace_size(N, K, E))
    rm.moe_route(rm.MoeDims(H, 0, E, K), N, dev(x), dev(ids), rm.MOE_QUANT_NONE, None, None,
                 None, eri, cs, ex, None, ws)
    torch.cuda.synchronize()
    r = oracle.route(ids, E)
    assert np.array_equal(host(eri), r["expanded_row_idx"])
    assert np.array_equal(host(ex, np.uint16), x[r["sorted_row_idx"] // K])


# ------------------------------------------------------------------------------ layer
def _run_layer(p, prepared=None):
    cfg = p["cfg"]
    if prepared is None:
        prepared = prepare(cfg, p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    L = DeviceLayer(p, prepared)
    out = L.forward()
    L.check_guards()
    return L, host(out, np.uint16), L.intermediates()


def test_layer_tiny_parity():
    _say(f"layer {TINY.name}")
    p = build_layer_problem(TINY)
    ref = oracle_forward(p)
    _, out, inter = _run_layer(p)
    st, res = compare.check_layer(p, out, inter, ref)
    _say(f"  code diffs {st['n_diff']}/{st['n_codes']}, {compare.fmt(res)}")


def _edge(name, **kw):
    base = dict(name=name, T=4, H=256, I=64, E=16, k=4, w_std=0.05, seed_index=30)
    base.update(kw)
    return LayerConfig(**base)


EDGE = [
    ("T1", _edge("edge_T1", T=1, seed_index=31), None),
    ("one_expert_many_rows", _edge("edge_E2", T=90, E=2, k=2, seed_index=32), None),
    ("ragged_tiles", _edge("edge_ragged", T=70, E=3, k=3, H=384, I=128, seed_index=33), None),
    ("all_on_expert_5", _edge("edge_same", T=40, E=8, k=4, seed_index=34), "same"),
    ("duplicate_ids", _edge("edge_dup", T=24, E=16, k=4, seed_index=35), "dup"),
    ("per_expert_situ", _edge("edge_situ", T=32, E=16, k=4, per_expert_situ=True,
                              seed_index=36), None),
    ("outliers", _edge("edge_out", T=32, E=16, k=4, outlier_frac=0.05, outlier_mult=30.0,
                       seed_index=37), None),
    ("wide_H", _edge("edge_wideH", T=8, H=1024, I=192, E=16, k=6, seed_index=38), None),
    # several 100-row big tiles per expert through the 64-row-per-wave FC1 (2I % 256 == 0)
    ("big_tiles", _edge("edge_big", T=300, E=4, k=4, H=256, I=128, seed_index=39), None),
    # T*k = 65536 routed rows: FC2 big tiles take the LDS-resident kernel
    ("resident_fc2", _edge("edge_res", T=16384, E=16, k=4, H=256, I=128, seed_index=40),
     None),
    # 65536 routed rows, Zipf-skewed: the weight-stationary FC2 on two slabs and two
    # 128-wide chunks, with runs split inside hot experts and ragged last passes
    ("stationary_fc2_skewed", _edge("edge_stat", T=8192, E=64, k=8, H=512, I=256,
                                    zipf_s=1.0, seed_index=41), None),
    # 65536 routed rows over 1024 experts (64 rows each on average): the token-resident
    # FC2 on 256-column slabs, big tiles split into 64-row sub-tiles
    ("resident_fc2_short_runs", _edge("edge_short", T=8192, E=1024, k=8, H=256, I=128,
                                      seed_index=42), None),
    # 65536 routed rows, Zipf 1.2 over 512 experts: 241 small tiles staged as codes (no f16
    # copy of x at this size) beside a 4081-row expert
    ("many_rows_small_tiles", _edge("edge_many_small", T=4096, E=512, k=16, H=256, I=128,
                                    zipf_s=1.2, seed_index=43), None),
    # 65536 routed rows with H not a multiple of 256 and I not of 128: the token-resident
    # FC2 on 128-column slabs, FC2's reduction padded from 192 to 256
    ("many_rows_fallback_shapes", _edge("edge_fallback", T=16384, E=16, k=4, H=384, I=192,
                                        seed_index=44), None),
    # I > 384: FC2 through the grouped kernel for both tile lists; I=576 pads FC2's
    # reduction to 640 (zero codes and scales past I)
    ("wide_I_small_tiles", _edge("edge_wideI_s", T=64, E=64, k=4, H=256, I=576,
                                 seed_index=45), None),
    ("wide_I_big_tiles", _edge("edge_wideI_b", T=300, E=8, k=4, H=384, I=512,
                               seed_index=46), None),
    # at most 1024 routed rows the tiles are all small ones: an expert with 90 rows is
    # split into 32-row tiles, and no big-tile kernel is launched
    ("small_batch_split_experts", _edge("edge_split", T=90, E=4, k=2, H=256, I=128,
                                        seed_index=47), None),
    # at most one routed row per compute unit with H a multiple of 512 and I of 128: FC1
    # and FC2 fused in one workgroup per small tile (I = 128, 256, 384: 2, 4, 6 row groups
    # per wave in FC1, one to three K chunks in FC2), with ragged tiles, an expert split
    # over several tiles, duplicate ids and a qA per expert
    ("fused_small_I128", _edge("edge_fused_a", T=8, E=16, k=4, H=512, I=128, seed_index=53),
     None),
    ("fused_small_I256_ragged", _edge("edge_fused_b", T=16, E=8, k=8, H=1024, I=256,
                                      seed_index=54), None),
    ("fused_small_I384_qa", _edge("edge_fused_c", T=8, E=32, k=16, H=512, I=384,
                                  seed_index=55), "qa"),
    ("fused_small_one_expert_many_tiles", _edge("edge_fused_d", T=40, E=2, k=2, H=512,
                                                I=128, seed_index=56), None),
    ("fused_small_duplicate_ids", _edge("edge_fused_e", T=24, E=16, k=4, H=512, I=256,
                                        seed_index=57), "dup"),
    # tokens whose x is all zero (after calibration, so the scales stay those of the
    # random batch): zero block scales and codes for x, zero FC1 and SiTU rows, zero
    # intermediate scales and an exact zero output row, in every kernel instance --
    # separate small tiles, the fused small-batch kernel, big tiles, the 65536-row kernels
    # -- and a batch that is zero throughout (every expert's amax 0)
    ("zero_tokens_small", _edge("edge_zero_s", T=24, E=16, k=4, seed_index=58), "zero_rows"),
    ("zero_tokens_fused", _edge("edge_zero_f", T=16, E=8, k=8, H=1024, I=256,
                                seed_index=59), "zero_rows"),
    ("zero_tokens_big", _edge("edge_zero_b", T=300, E=4, k=4, H=256, I=128, seed_index=60),
     "zero_rows"),
    ("zero_tokens_many_rows", _edge("edge_zero_m", T=4096, E=64, k=16, H=256, I=128,
                                    seed_index=61), "zero_rows"),
    ("zero_batch", _edge("edge_zero_all", T=300, E=4, k=4, H=256, I=128, seed_index=62),
     "zero_all"),
    # a qA per expert (each expert's scale from its own rows): the requantization must use
    # the scale of the row's expert in every kernel instance -- small tiles, big tiles with
    # 2 and 4 row groups per wave, and the 65536-row kernels
    ("qa_per_expert_small", _edge("edge_qa_s", T=24, E=16, k=4, seed_index=48), "qa"),
    ("qa_per_expert_big", _edge("edge_qa_b", T=300, E=4, k=4, H=256, I=128, seed_index=49),
     "qa"),
    ("qa_per_expert_mid", _edge("edge_qa_m", T=400, E=8, k=4, H=384, I=128, seed_index=50),
     "qa"),
    ("qa_per_expert_many_rows", _edge("edge_qa_many", T=8192, E=64, k=8, H=512, I=256,
                                      zipf_s=1.0, seed_index=51), "qa"),
]


def test_fc2_sums_at_their_bound():
    """FC2 sums equal to the bound I * 2688^2 the row exponent is taken from (constant
    weights, a qA per expert; tests.problem.constant_weight_problem): those rows' stored
    f16 values sit in the top binade [2^14, 2^15] and must neither overflow nor lose bits;
    the whole layer meets the parity bar."""
    cfg = _edge("edge_bound", T=32, E=4, k=2, H=256, I=64, seed_index=52)
    _say("layer edge fc2_sums_at_their_bound")
    p = constant_weight_problem(cfg)
    ref = oracle_forward(p)
    _, out, inter = _run_layer(p)
    st, res = compare.check_layer(p, out, inter, ref)
    flat = ref["sorted_row_idx"]
    o_gpu = inter["o_rows"][flat]
    assert np.all(np.isfinite(o_gpu))
    # rows whose intermediate codes match the oracle's: f16 keeps 11 significant bits of
    # each value (plus one fp32 rounding of the scaled sum)
    same = np.ones(len(flat), bool)
    same[st["rows_with_diff"]] = False
    ref_o = ref["o"].astype(np.float64)
    assert np.all(np.abs(o_gpu - ref_o)[same] <= 2.0 ** -10 * np.abs(ref_o)[same])
    s_row = inter["o_exp"][flat].astype(np.int64)
    stored = np.abs(o_gpu) * np.ldexp(1.0, s_row)[:, None]
    assert 2.0 ** 14 <= stored.max() <= 2.0 ** 15
    _say(f"  largest stored value {stored.max():.1f}; {compare.fmt(res)}")


@pytest.mark.parametrize("name,cfg,mod", EDGE, ids=[c[0] for c in EDGE])
def test_layer_edge_cases(name, cfg, mod):
    _say(f"layer edge {name}")
    p = build_layer_problem(cfg, per_expert_qa=(mod == "qa"))
    if mod == "qa":
        assert len(np.unique(p["qA"])) == cfg.E
    if mod == "same":
        p["ids"] = p["ids"].copy()
        p["ids"][:, 0] = 5                   # every token's first pick is expert 5
    elif mod == "dup":
        p["ids"] = p["ids"].copy()
        p["ids"][:, 1] = p["ids"][:, 0]
    elif mod in ("zero_rows", "zero_all"):
        p["x"] = p["x"].copy()
        zero = slice(None) if mod == "zero_all" else slice(None, None, 3)
        p["x"][zero] = 0
    ref = oracle_forward(p)
    _, out, inter = _run_layer(p)
    st, res = compare.check_layer(p, out, inter, ref)
    if mod in ("zero_rows", "zero_all"):
        # the bound is 0 on a zero row: its output must be exactly zero
        assert not np.any(ref["out_f64"][zero])
        assert not np.any(out[zero] & 0x7FFF)
    _say(f"  code diffs {st['n_diff']}/{st['n_codes']}, {compare.fmt(res)}")


def test_layer_dropped_ids_many_tokens():
    """Out-of-range expert ids are dropped: their rows add nothing to the output, and a
    token whose picks are all dropped gets exact zeros.  4096 tokens, so that the
    finalization runs its persistent form.  The reference is the oracle on the original
    (valid) ids with the dropped picks' route weights set to zero: 0 * o adds nothing to
    the float64 sum, and every other row's value does not depend on the dropped ones."""
    _say("layer dropped ids, 4096 tokens")
    cfg = _edge("edge_drop", T=4096, E=64, k=8, H=256, I=128, seed_index=63)
    p = build_layer_problem(cfg)
    drop = np.zeros(p["ids"].shape, bool)
    drop[::3, 2] = True
    drop[5, :] = True                        # every pick of token 5
    drop[7, 0] = drop[7, 7] = True
    ref = oracle_forward(dict(p, rw=np.where(drop, np.uint16(0), p["rw"]).astype(np.uint16)))
    gpu_p = dict(p, ids=np.where(drop, np.int32(cfg.E), p["ids"]).astype(np.int32))
    _, out, inter = _run_layer(gpu_p)
    assert np.array_equal(inter["expanded_row_idx"].reshape(drop.shape) < 0, drop)
    # the kept rows' intermediate codes, in the reference's row order (a dropped row keeps
    # the reference's codes: its weight there is zero), then the output bound widened by
    # the exact effect of differing codes, as for every layer case
    pos = inter["expanded_row_idx"][ref["sorted_row_idx"]]
    keep = pos >= 0
    gc, gs = ref["a_codes"].copy(), ref["a_scales"].copy()
    gc[keep] = compare.unpack(inter["a_codes"])[pos[keep]]
    gs[keep] = inter["a_scales"][pos[keep]]
    st = compare.code_diff_stats(gc, gs, ref["a_codes"], ref["a_scales"])
    assert st["max_step_same_scale"] <= 1 and st["frac"] <= compare.CODE_DIFF_FRAC, st
    ref_p = dict(p, rw=np.where(drop, np.uint16(0), p["rw"]).astype(np.uint16))
    res = compare.check_output(out, ref["out_f64"],
                               compare.flip_widening(ref_p, gc, gs, ref, st["rows_with_diff"]))
    assert not np.any(out[5] & 0x7FFF)
    _say(f"  {int(drop.sum())} dropped picks; {compare.fmt(res)}")


def test_layer_determinism_poisoned_workspace_and_reuse():
    _say("layer determinism / poisoned workspace")
    p = build_layer_problem(_edge("edge_det", T=48, E=16, k=4, seed_index=40))
    prepared = prepare(p["cfg"], p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    L = DeviceLayer(p, prepared)
    a = host(L.forward().clone(), np.uint16)
    ws2 = empty_bytes(L.ws_bytes, fill=0xFF)
    out2 = torch.full_like(L.out, -1)
    b = host(L.forward(workspace=ws2, out=out2), np.uint16)
    c = host(L.forward(), np.uint16)
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.array_equal(a, c)
    # a workspace sized for more tokens serves a smaller call
    big = empty_bytes(rm.moe_workspace_size(L.dims, 4096), fill=0x5A)
    d = host(L.forward(workspace=big), np.uint16)
    assert np.array_equal(a, d)


@pytest.mark.parametrize("shape", ["separate_gemms", "fused_gemms"])
def test_layer_graph_capture_replay(shape):
    _say(f"layer hipGraph capture/replay ({shape})")
    cfg = (_edge("edge_graph", T=20, E=16, k=4, seed_index=41) if shape == "separate_gemms"
           else _edge("edge_graph_fused", T=16, E=32, k=8, H=512, I=256, seed_index=58))
    p = build_layer_problem(cfg)
    prepared = prepare(p["cfg"], p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    L = DeviceLayer(p, prepared)
    eager = host(L.forward().clone(), np.uint16)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        L.forward(stream=s)
    for i in range(5):
        L.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(L.out, np.uint16), eager), f"replay {i}"
        L.forward()                     # eager work between replays
        torch.cuda.synchronize()
