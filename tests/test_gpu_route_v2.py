"""GPU parity of moe_route_v2 (the routing primitive's options: scatter index, count and
key_value histograms, active expert range, static int8, drop/pad, active_num, per-row
scale) against oracle.route_v2, bit for bit, through the C ABI.

Every output buffer starts filled with a sentinel: the defined entries must equal the
oracle's, and the rows past the valid ones must still hold the sentinel (no stray
writes)."""

import sys

import numpy as np
import pytest
import torch

import oracle
import routed_moe_layer_amd as rm
from moe_inputs import ROUTE_8K, draw_expert_ids, draw_route_inputs, draw_tokens, f32_to_bf16_bits
from tests.gpu_harness import dev, host, empty_bytes

pytestmark = pytest.mark.gpu

SENT_BYTE = 0x5A
SENT_I32 = 0x5A5A5A5A
STATIC_SCALE = np.float32(17.3)
STATIC_OFFSET = np.float32(-0.6)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    yield
    torch.cuda.synchronize()


def _rows(N, K, E, opts):
    if opts.get("drop_pad_mode", 0):
        return E * opts["expert_capacity"]
    a = opts.get("active_num", -1)
    return N * K if a <= 0 else min(a, N * K)


def run_v2(x_bits, ids, E, opts, row_scale=None):
    """One moe_route_v2 call; returns the host copies of every output."""
    N, K = ids.shape
    H = x_bits.shape[1]
    q = opts.get("quant_mode", -1)
    rows = _rows(N, K, E, opts)
    elem = 2 if q == -1 else 1
    ex = torch.full((rows * H * elem,), SENT_BYTE, dtype=torch.uint8, device="cuda")
    eri = torch.full((N * K,), SENT_I32, dtype=torch.int32, device="cuda")
    start, end = opts.get("expert_start", 0), opts.get("expert_end", 0)
    e_act = (end - start) if end else E
    tok_shape = (E, 2) if opts.get("expert_tokens_num_type", 0) == 2 else (e_act,)
    tok = torch.full(tok_shape, SENT_I32, dtype=torch.int32, device="cuda")
    esc = torch.full((max(rows, 1),), SENT_I32, dtype=torch.int32, device="cuda")
    avail = torch.full((1,), SENT_I32, dtype=torch.int32, device="cuda")
    scale = offset = None
    if q == 0:
        scale = dev(np.array([STATIC_SCALE], np.float32))
        offset = dev(np.array([STATIC_OFFSET], np.float32))
    elif q == -1 and row_scale is not None:
        scale = dev(row_scale)
    want_scale = q == 1 or (q == -1 and row_scale is not None)
    ws = empty_bytes(rm.moe_route_workspace_size(N, K, E), fill=0xFF)
    rm.moe_route_v2(N, H, E, K, dev(x_bits), dev(ids.astype(np.int32)), rm.MoeRouteOptions(**opts),
                    ex, eri, expert_tokens=tok, expanded_scale=esc if want_scale else None,
                    available_idx_num=avail, scale=scale, offset=offset, workspace=ws)
    torch.cuda.synchronize()
    ex_h = host(ex)
    ex_h = ex_h.view(np.uint16) if elem == 2 else ex_h.view(np.int8)
    return {"expanded_x": ex_h.reshape(rows, H), "expanded_row_idx": host(eri),
            "expert_tokens": host(tok), "expanded_scale": host(esc).view(np.float32)[:rows],
            "expanded_scale_bits": host(esc)[:rows], "available_idx_num": int(host(avail)[0]),
            "has_scale": want_scale}


def oracle_v2(x_bits, ids, E, opts, row_scale=None):
    o = dict(opts)
    start, end = o.pop("expert_start", 0), o.pop("expert_end", 0)
    rng_ = None if (start, end) == (0, 0) else (start, end)
    q = o.get("quant_mode", -1)
    scale = offset = None
    if q == 0:
        scale, offset = STATIC_SCALE, STATIC_OFFSET
    elif row_scale is not None:
        scale = row_scale
    return oracle.route_v2(oracle.bf16_bits_to_f32(x_bits), ids, E, expert_range=rng_,
                           scale=scale, offset=offset, **o)


def check_v2(got, want, opts):
    assert got["available_idx_num"] == want["available_idx_num"]
    assert np.array_equal(got["expanded_row_idx"], want["expanded_row_idx"])
    assert np.array_equal(got["expert_tokens"], want["expert_tokens"])
    q = opts.get("quant_mode", -1)
    wx = want["expanded_x"]
    rows = got["expanded_x"].shape[0]
    wx = wx.reshape(rows, -1)
    if q == -1:
        wx = f32_to_bf16_bits(wx)
    v = want["valid_rows"]
    gx = got["expanded_x"]
    bad = np.nonzero(np.any(gx[:v] != wx[:v], axis=1))[0]
    assert bad.size == 0, f"{bad.size} expanded rows differ, first {bad[:5]}"
    if v < rows:                                   # rows past the valid ones: untouched
        assert np.all(gx[v:].view(np.uint8) == SENT_BYTE)
    if got["has_scale"]:
        ws_ = want["expanded_scale"].reshape(-1)
        assert np.array_equal(got["expanded_scale"][:v].view(np.uint32),
                              ws_[:v].astype(np.float32).view(np.uint32))
        if v < rows:
            assert np.all(got["expanded_scale_bits"][v:] == SENT_I32)


# name, N, K, E, H, zipf, options, per-row scale
V2_CASES = [
    ("scatter_one_workgroup", 16, 16, 896, 64, 0.0, dict(row_idx_type=1), False),
    ("scatter_tiled_count", 300, 8, 64, 64, 1.1, dict(row_idx_type=1, expert_tokens_num_type=1),
     False),
    ("range_gather_count_dynamic", 500, 8, 256, 136, 1.1,
     dict(expert_start=3, expert_end=40, expert_tokens_num_type=1, quant_mode=1), False),
    ("range_scatter_kv_static", 500, 8, 256, 136, 0.5,
     dict(expert_start=100, expert_end=228, row_idx_type=1, expert_tokens_num_type=2,
          quant_mode=0), False),
    ("range_one_expert", 200, 4, 16, 64, 0.0, dict(expert_start=15, expert_end=16), False),
    ("range_one_workgroup_kv", 60, 16, 896, 64, 1.0,
     dict(expert_start=400, expert_end=896, expert_tokens_num_type=2, quant_mode=1), False),
    # the page's low-latency case: one token, K=8, 256 experts, dynamic quant, key_value
    ("one_token_kv_dynamic", 1, 8, 256, 7168, 0.0,
     dict(expert_start=0, expert_end=256, quant_mode=1, expert_tokens_num_type=2), False),
    # the page's large-batch case: K=8, 256 experts, a range of 32, no quant, scatter, count
    ("large_batch_range32", 2048, 8, 256, 7168, 1.1,
     dict(expert_start=64, expert_end=96, quant_mode=-1, row_idx_type=1,
          expert_tokens_num_type=1), False),
    ("droppad_c1_dynamic", 200, 4, 16, 64, 1.3,
     dict(drop_pad_mode=1, expert_capacity=1, quant_mode=1), False),
    ("droppad_c37_static_kv", 300, 8, 64, 136, 1.1,
     dict(drop_pad_mode=1, expert_capacity=37, quant_mode=0, expert_tokens_num_type=2), False),
    ("droppad_nothing_dropped_bf16", 40, 4, 8, 64, 0.0,
     dict(drop_pad_mode=1, expert_capacity=160, quant_mode=-1), False),
    ("droppad_one_workgroup", 16, 16, 896, 64, 0.0,
     dict(drop_pad_mode=1, expert_capacity=2, quant_mode=1, expert_tokens_num_type=1), False),
    ("active_num_cut_dynamic", 300, 8, 64, 64, 1.1, dict(active_num=1000, quant_mode=1), False),
    ("active_num_range_static", 300, 8, 64, 64, 1.1,
     dict(active_num=50, expert_start=10, expert_end=30, quant_mode=0), False),
    ("active_num_above_rows", 30, 4, 8, 64, 0.0, dict(active_num=100000, quant_mode=-1), False),
    ("row_scale_bf16", 300, 8, 64, 72, 0.5, dict(quant_mode=-1), True),
    ("row_scale_range_scatter", 300, 8, 64, 72, 0.5,
     dict(quant_mode=-1, expert_start=5, expert_end=50, row_idx_type=1), True),
    ("row_scale_droppad", 100, 4, 8, 72, 1.0,
     dict(quant_mode=-1, drop_pad_mode=1, expert_capacity=20), True),
    # rows longer than the permute kernel's register chunk (8192 BF16): several chunks
    ("dynamic_two_chunks", 50, 4, 16, 8200, 0.5, dict(quant_mode=1), False),
    ("static_three_chunks_range", 20, 4, 16, 16392, 0.0,
     dict(quant_mode=0, expert_start=2, expert_end=9), False),
    ("bf16_two_chunks_droppad", 30, 2, 4, 9000, 0.0,
     dict(drop_pad_mode=1, expert_capacity=5, quant_mode=-1), False),
    # at most 8 tokens: routing and movement in one workgroup
    ("few_tokens_dynamic_long_rows", 3, 8, 256, 16392, 0.0,
     dict(quant_mode=1, expert_tokens_num_type=2), False),
    ("few_tokens_droppad_static", 8, 8, 64, 136, 1.0,
     dict(drop_pad_mode=1, expert_capacity=2, quant_mode=0), False),
    ("few_tokens_range_scatter_row_scale", 5, 4, 16, 72, 0.0,
     dict(quant_mode=-1, expert_start=3, expert_end=11, row_idx_type=1, active_num=9), True),
    # the page's expert_num limits: 10240 experts (the scatter ranks its waves in turn
    # against one running histogram above 4096), 5120 with the key_value histogram
    ("experts_10240_dynamic", 3000, 8, 10240, 64, 0.7, dict(quant_mode=1), False),
    ("experts_10240_range_scatter_count", 2000, 8, 10240, 64, 0.3,
     dict(expert_start=100, expert_end=9000, row_idx_type=1, expert_tokens_num_type=1,
          quant_mode=-1), False),
    ("experts_10240_droppad", 1500, 8, 10240, 64, 1.2,
     dict(drop_pad_mode=1, expert_capacity=3, quant_mode=0), False),
    ("experts_5120_kv", 3000, 8, 5120, 64, 0.5,
     dict(expert_tokens_num_type=2, quant_mode=1), False),
    ("experts_10240_one_tile", 40, 8, 10240, 64, 0.0, dict(quant_mode=1), False),
]


@pytest.mark.parametrize("name,N,K,E,H,zipf,opts,rs", V2_CASES, ids=[c[0] for c in V2_CASES])
def test_route_v2_bit_exact(name, N, K, E, H, zipf, opts, rs):
    _say(f"route_v2 {name}")
    seed = 1200 + N + H
    ids = draw_expert_ids(N, E, K, seed_index=seed, zipf_s=zipf)
    x = draw_tokens(N, H, seed_index=seed)
    x = f32_to_bf16_bits(oracle.bf16_bits_to_f32(x) * np.float32(3.0))
    row_scale = (np.random.default_rng(seed).standard_normal(N).astype(np.float32)
                 if rs else None)
    got = run_v2(x, ids, E, opts, row_scale)
    want = oracle_v2(x, ids, E, opts, row_scale)
    check_v2(got, want, opts)


def test_route_v2_full_size_scatter_kv_dynamic():
    """The int8 routing workload (N=8192, H=7168, E=256, K=8) through the options path."""
    cfg = ROUTE_8K
    _say(f"route_v2 {cfg.name} scatter kv dynamic")
    x, ids = draw_route_inputs(cfg)
    opts = dict(row_idx_type=1, expert_tokens_num_type=2, quant_mode=1)
    got = run_v2(x, ids, cfg.E, opts)
    want = oracle_v2(x, ids, cfg.E, opts)
    check_v2(got, want, opts)


def test_route_v2_defaults_equal_moe_route():
    """With default options moe_route_v2 computes what moe_route does."""
    _say("route_v2 defaults vs moe_route")
    N, K, E, H = 700, 8, 128, 64
    ids = draw_expert_ids(N, E, K, seed_index=1300, zipf_s=1.0)
    x = draw_tokens(N, H, seed_index=1300)
    got = run_v2(x, ids, E, dict(quant_mode=1))
    ex = torch.empty((N * K, H), dtype=torch.int8, device="cuda")
    esc = torch.empty(N * K, dtype=torch.float32, device="cuda")
    eri = torch.empty(N * K, dtype=torch.int32, device="cuda")
    cs = torch.empty(E, dtype=torch.int32, device="cuda")
    ws = empty_bytes(rm.moe_route_workspace_size(N, K, E))
    rm.moe_route(rm.MoeDims(H, 0, E, K), N, dev(x), dev(ids), rm.MOE_QUANT_INT8_ROW_DYNAMIC, None,
                 None, None, eri, cs, ex, esc, ws)
    torch.cuda.synchronize()
    assert np.array_equal(got["expanded_x"], host(ex))
    assert np.array_equal(got["expanded_scale"], host(esc))
    assert np.array_equal(got["expanded_row_idx"], host(eri))
    assert np.array_equal(got["expert_tokens"], host(cs))


def _random_case(rng):
    E = int(rng.choice([1, 3, 16, 64, 256, 897, 4096]))
    K = int(rng.integers(1, min(E, 16) + 1))
    N = int(rng.choice([1, 2, 7, 31, 128, 300, 1000]))
    H = int(rng.choice([8, 64, 136, 2048, 8200]))
    if N * H > 2_000_000:
        H = 64
    opts = {"row_idx_type": int(rng.integers(0, 2)),
            "expert_tokens_num_type": int(rng.integers(0, 3)),
            "quant_mode": int(rng.integers(-1, 2))}
    if rng.random() < 0.3 and opts["row_idx_type"] == 0:
        opts["drop_pad_mode"] = 1
        opts["expert_capacity"] = int(rng.integers(1, min(N * K, max(2, N * K // E * 2)) + 1))
    else:
        if rng.random() < 0.5:
            s = int(rng.integers(0, E))
            opts["expert_start"], opts["expert_end"] = s, int(rng.integers(s + 1, E + 1))
        if rng.random() < 0.3:
            opts["active_num"] = int(rng.integers(1, N * K + 5))
    zipf = float(rng.choice([0.0, 1.0, 1.5]))
    row_scale = opts["quant_mode"] == -1 and rng.random() < 0.5
    return N, K, E, H, zipf, opts, row_scale


@pytest.mark.parametrize("seed", range(40))
def test_route_v2_random_options_bit_exact(seed):
    """Seeded random shapes and option combinations (expert range, index type, histogram
    mode, quant mode, drop/pad capacity, active_num, per-row scale)."""
    rng = np.random.default_rng(9000 + seed)
    N, K, E, H, zipf, opts, rs = _random_case(rng)
    _say(f"route_v2 random {seed}: N={N} K={K} E={E} H={H} zipf={zipf} {opts} row_scale={rs}")
    ids = draw_expert_ids(N, E, K, seed_index=2000 + seed, zipf_s=zipf)
    x = draw_tokens(N, H, seed_index=2000 + seed)
    row_scale = rng.standard_normal(N).astype(np.float32) if rs else None
    got = run_v2(x, ids, E, opts, row_scale)
    want = oracle_v2(x, ids, E, opts, row_scale)
    check_v2(got, want, opts)


def test_route_v2_drop_pad_kv_many_ids():
    """Drop/pad with key_value counts past 2^21 routed rows (several router tiles and the
    26-bit row fields of the expert scan)."""
    _say("route_v2 drop/pad, 2.4 M ids")
    N, K, E, H = 300_000, 8, 64, 8
    ids = draw_expert_ids(N, E, K, seed_index=2100, zipf_s=1.2)
    x = draw_tokens(N, H, seed_index=2100)
    opts = dict(drop_pad_mode=1, expert_capacity=20_000, quant_mode=1, expert_tokens_num_type=2)
    got = run_v2(x, ids, E, opts)
    want = oracle_v2(x, ids, E, opts)
    check_v2(got, want, opts)


def test_route_v2_graph_capture_replay():
    """moe_route_v2 (drop/pad with its zero-fill launch, key_value histogram, dynamic int8)
    captured into a graph and replayed with eager work between the replays; every replay
    must equal the eager call."""
    _say("route_v2 graph capture/replay")
    N, K, E, H = 300, 8, 64, 136
    ids = draw_expert_ids(N, E, K, seed_index=2200, zipf_s=1.1)
    x = draw_tokens(N, H, seed_index=2200)
    opts = rm.MoeRouteOptions(drop_pad_mode=1, expert_capacity=40, quant_mode=1,
                              expert_tokens_num_type=2)
    xd, idd = dev(x), dev(ids)
    rows = E * 40
    ex = torch.zeros((rows, H), dtype=torch.int8, device="cuda")
    eri = torch.zeros(N * K, dtype=torch.int32, device="cuda")
    tok = torch.zeros((E, 2), dtype=torch.int32, device="cuda")
    esc = torch.zeros(rows, dtype=torch.float32, device="cuda")
    ws = empty_bytes(rm.moe_route_workspace_size(N, K, E))

    def call(stream=None):
        rm.moe_route_v2(N, H, E, K, xd, idd, opts, ex, eri, expert_tokens=tok,
                        expanded_scale=esc, workspace=ws, stream=stream)

    call()
    torch.cuda.synchronize()
    want = [host(t).copy() for t in (ex, eri, tok, esc)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(stream=s)
    for rep in range(4):
        for t in (ex, eri, tok, esc):
            t.fill_(-1 if t.dtype != torch.float32 else float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in (ex, eri, tok, esc)]
        for a, b in zip(got, want):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"replay {rep}"
        call()                                          # eager work between replays
        torch.cuda.synchronize()
