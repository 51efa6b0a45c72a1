"""Pins of the oracle's routing options (scatter index, count / key_value histograms,
active expert range, static int8 quant, drop/pad, active_num): a brute force that counts
instead of sorting, hand-worked values, and invariants.

The brute force places flat id f at position #{g in range: id[g] < id[f]} +
#{g in range: id[g] == id[f], g < f} (the definition of a stable sort), independently of
the oracle's argsort."""

import numpy as np
import pytest

from oracle import routing as oroute
from moe_inputs import draw_expert_ids


def _brute(ids, expert_num, start, end, C=None):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    inr = [start <= e < end for e in flat]
    pos = {}
    for f, e in enumerate(flat):
        if inr[f]:
            pos[f] = sum(1 for g, d in enumerate(flat) if inr[g] and (d < e or (d == e and g < f)))
    counts = [sum(1 for e in flat if e == x) for x in range(start, end)]
    rank = {}
    for f, e in enumerate(flat):
        if inr[f]:
            rank[f] = sum(1 for g, d in enumerate(flat) if inr[g] and d == e and g < f)
    return flat, pos, counts, rank


CASES = [(5, 3, 8, None), (9, 4, 16, (3, 11)), (1, 8, 256, (0, 256)), (12, 2, 6, (5, 6)),
         (17, 5, 12, (0, 1))]


@pytest.mark.parametrize("N,K,E,rng_", CASES)
@pytest.mark.parametrize("row_idx_type", [0, 1])
def test_index_outputs_match_brute_force(N, K, E, rng_, row_idx_type):
    ids = draw_expert_ids(N, E, K, seed_index=300 + N, zipf_s=1.0)
    start, end = (0, E) if rng_ is None else rng_
    r = oroute.route_v2(None, ids, E, expert_range=rng_, row_idx_type=row_idx_type)
    flat, pos, counts, _ = _brute(ids, E, start, end)
    avail = len(pos)
    assert r["available_idx_num"] == avail
    if row_idx_type == 0:
        want = [pos.get(f, -1) for f in range(len(flat))]
    else:
        want = [-1] * len(flat)
        for f, p in pos.items():
            want[p] = f
    assert r["expanded_row_idx"].tolist() == want
    assert r["expert_tokens"].tolist() == list(np.cumsum(counts))


@pytest.mark.parametrize("N,K,E,rng_", CASES)
def test_histogram_modes_match_brute_force(N, K, E, rng_):
    ids = draw_expert_ids(N, E, K, seed_index=400 + N, zipf_s=1.3)
    start, end = (0, E) if rng_ is None else rng_
    _, _, counts, _ = _brute(ids, E, start, end)
    r1 = oroute.route_v2(None, ids, E, expert_range=rng_, expert_tokens_num_type=1)
    assert r1["expert_tokens"].tolist() == counts
    r2 = oroute.route_v2(None, ids, E, expert_range=rng_, expert_tokens_num_type=2)
    kv = r2["expert_tokens"]
    assert kv.shape == (E, 2)
    pairs = [[start + i, c] for i, c in enumerate(counts) if c > 0]
    assert kv[:len(pairs)].tolist() == pairs
    assert np.all(kv[len(pairs):] == 0)


def test_key_value_hand_example():
    # experts 1 and 3 used, 0 and 2 empty
    ids = np.array([[3, 1], [3, 3]], np.int32)
    kv = oroute.route_v2(None, ids, 4, expert_tokens_num_type=2)["expert_tokens"]
    assert kv.tolist() == [[1, 1], [3, 3], [0, 0], [0, 0]]


@pytest.mark.parametrize("C", [1, 2, 5])
def test_drop_pad_matches_brute_force(C):
    N, K, E = 11, 3, 5
    ids = draw_expert_ids(N, E, K, seed_index=500 + C, zipf_s=1.5)
    rng = np.random.default_rng(C)
    x = rng.integers(-50, 50, (N, 8)).astype(np.float32)
    r = oroute.route_v2(x, ids, E, drop_pad_mode=1, expert_capacity=C, quant_mode=-1)
    flat, pos, counts, rank = _brute(ids, E, 0, E)
    want_idx = [(flat[f] * C + rank[f]) if rank[f] < C else -1 for f in range(len(flat))]
    assert r["expanded_row_idx"].tolist() == want_idx
    ex = r["expanded_x"]
    assert ex.shape == (E, C, 8)
    for e in range(E):
        for s in range(C):
            src = [f for f in range(len(flat)) if flat[f] == e and rank[f] == s]
            if src:
                assert np.array_equal(ex[e, s], x[src[0] // K])
            else:
                assert np.all(ex[e, s] == 0)
    # the histogram counts rows before the drop
    assert r["expert_tokens"].tolist() == list(np.cumsum(counts))


def test_static_quant_hand_values():
    x = np.array([1.5, -2.5, 0.5, 100.0, -100.0, 200.0, -200.0, 127.5, -128.5], np.float32)
    assert oroute.int8_static_quant(x, 1.0, 0.0).tolist() == \
        [2, -2, 0, 100, -100, 127, -128, 127, -128]
    # 1*2 + 0.5 = 2.5 -> 2 (half to even); 3*2 + 0.5 = 6.5 -> 6; -1*2 - 0.5 = -2.5 -> -2
    assert oroute.int8_static_quant(np.array([1, 3, -1], np.float32), 2.0, 0.5).tolist()[:2] \
        == [2, 6]
    assert oroute.int8_static_quant(np.array([-1.0], np.float32), 2.0, -0.5).tolist() == [-2]


def test_static_quant_rounds_the_product_in_fp32():
    # fp32(0.1) = 0.100000001490116...; 5 * that = 0.5000000075 exactly, which fp32 rounds
    # to 0.5 (half an ulp at 0.5 is 2.98e-8), and 0.5 rounds to 0.  In exact arithmetic
    # the value exceeds 0.5 and would round to 1.
    s = np.float32(0.1)
    assert float(s) * 5.0 > 0.5
    assert oroute.int8_static_quant(np.array([5.0], np.float32), s, 0.0).tolist() == [0]


def test_static_mode_moves_quantized_rows():
    ids = np.array([[1, 0], [0, 1]], np.int32)
    x = np.array([[1.0, 2.0], [3.0, 4.0]], np.float32)
    r = oroute.route_v2(x, ids, 2, quant_mode=0, scale=np.float32(1.5), offset=np.float32(0.25))
    # sorted: f=1 (t0, e0), f=2 (t1, e0), f=0 (t0, e1), f=3 (t1, e1)
    q0 = [2, 3]      # 1.75 -> 2, 3.25 -> 3
    q1 = [5, 6]      # 4.75 -> 5, 6.25 -> 6
    assert r["expanded_x"].tolist() == [q0, q1, q0, q1]
    assert "expanded_scale" not in r


def test_active_num_truncates_only_the_moved_rows():
    ids = draw_expert_ids(20, 8, 4, seed_index=600, zipf_s=0.0)
    x = np.random.default_rng(1).standard_normal((20, 16)).astype(np.float32)
    full = oroute.route_v2(x, ids, 8, quant_mode=1)
    cut = oroute.route_v2(x, ids, 8, quant_mode=1, active_num=7)
    assert cut["expanded_x"].shape == (7, 16) and cut["valid_rows"] == 7
    assert np.array_equal(cut["expanded_x"], full["expanded_x"][:7])
    assert np.array_equal(cut["expanded_scale"], full["expanded_scale"][:7])
    assert np.array_equal(cut["expanded_row_idx"], full["expanded_row_idx"])
    assert np.array_equal(cut["expert_tokens"], full["expert_tokens"])
    big = oroute.route_v2(x, ids, 8, quant_mode=1, active_num=1000)
    assert big["expanded_x"].shape == (80, 16)


def test_range_gather_and_scatter_move_the_same_rows():
    """Step 5 moves by the scatter index on the full range and by the gather index
    otherwise; on a range the two definitions must agree, which this checks by moving
    rows through the scatter form independently."""
    N, K, E = 13, 4, 10
    ids = draw_expert_ids(N, E, K, seed_index=700, zipf_s=0.5)
    x = np.random.default_rng(2).standard_normal((N, 12)).astype(np.float32)
    r = oroute.route_v2(x, ids, E, expert_range=(2, 7), quant_mode=-1,
                        scale=np.arange(N, dtype=np.float32))
    sc = oroute.route_v2(None, ids, E, expert_range=(2, 7), row_idx_type=1)
    avail = r["available_idx_num"]
    for i in range(avail):
        f = sc["expanded_row_idx"][i]
        assert np.array_equal(r["expanded_x"][i], x[f // K])
        assert r["expanded_scale"][i] == f // K


def test_full_range_defaults_agree_with_route():
    ids = draw_expert_ids(30, 16, 4, seed_index=800, zipf_s=1.0)
    a = oroute.route(ids, 16)
    b = oroute.route_v2(None, ids, 16)
    assert np.array_equal(a["expanded_row_idx"], b["expanded_row_idx"])
    assert np.array_equal(a["cumsum"], b["expert_tokens"])


def test_bad_options_raise():
    ids = np.array([[0, 1]], np.int32)
    with pytest.raises(ValueError):
        oroute.route_v2(None, ids, 2, expert_range=(1, 1))
    with pytest.raises(ValueError):
        oroute.route_v2(None, ids, 2, drop_pad_mode=1, expert_capacity=1, expert_range=(0, 1))
    with pytest.raises(ValueError):
        oroute.route_v2(None, ids, 2, drop_pad_mode=1, expert_capacity=1, row_idx_type=1)
