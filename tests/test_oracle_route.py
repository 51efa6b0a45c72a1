"""Pins of the oracle's routing and int8 token movement: brute force and invariants."""

import numpy as np
import pytest
import torch

from oracle import routing as oroute
from moe_inputs import draw_expert_ids


def _insertion_sort_route(ids, E):
    """Brute-force stable sort by repeated insertion (pure Python, tiny inputs only)."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    order = []
    for f, e in enumerate(flat):
        pos = len(order)
        while pos > 0 and flat[order[pos - 1]] > e:
            pos -= 1
        order.insert(pos, f)
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    return order, counts


@pytest.mark.parametrize("T,k,E,zipf", [(4, 4, 16, 0.0), (7, 3, 5, 1.5), (1, 8, 256, 0.0),
                                        (33, 16, 40, 1.0)])
def test_route_matches_insertion_sort(T, k, E, zipf):
    ids = draw_expert_ids(T, E, k, seed_index=50 + T, zipf_s=zipf)
    r = oroute.route(ids, E)
    order, counts = _insertion_sort_route(ids, E)
    assert r["sorted_row_idx"].tolist() == order
    assert r["counts"].tolist() == counts
    assert r["cumsum"].tolist() == list(np.cumsum(counts))
    for i, f in enumerate(order):
        assert r["expanded_row_idx"][f] == i
        assert r["sorted_ids"][i] == ids.reshape(-1)[f]


def test_route_invariants_with_duplicates_and_empty_experts():
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 3, (100, 6)).astype(np.int32)        # duplicates within tokens
    E = 9                                                      # experts 3..8 empty
    r = oroute.route(ids, E)
    n = ids.size
    assert r["counts"].sum() == n and r["cumsum"][-1] == n
    assert np.all(r["counts"][3:] == 0)
    assert np.array_equal(r["sorted_row_idx"][r["expanded_row_idx"]], np.arange(n))
    assert np.array_equal(r["expanded_row_idx"][r["sorted_row_idx"]], np.arange(n))
    assert np.all(np.diff(r["sorted_ids"]) >= 0)
    same = np.diff(r["sorted_ids"]) == 0
    assert np.all(np.diff(r["sorted_row_idx"])[same] > 0)     # stable: f increases


def test_route_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oroute.route(np.array([[0, 5]], np.int32), 5)


def test_int8_quant_matches_torch_round_half_even():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-3, 3, (64, 1)))).astype(np.float32)
    x[3] = 0.0
    q, scale = oroute.int8_row_quant(x)
    tx = torch.from_numpy(x)
    tscale = (tx.abs().amax(dim=1) / 127.0)
    assert np.array_equal(tscale.numpy(), scale)
    quot = torch.where(tscale[:, None] == 0, torch.zeros_like(tx), tx / tscale[:, None])
    tq = torch.clamp(torch.round(quot), -127, 127).to(torch.int8).numpy()
    assert np.array_equal(tq, q)


def test_int8_quant_invariants():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((200, 300)).astype(np.float32)
    x[5] = 0.0
    q, scale = oroute.int8_row_quant(x)
    nz = scale > 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)
    assert np.all(q[~nz] == 0) and scale[5] == 0
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * scale[:, None])
    assert np.all(err[nz] <= scale[nz, None] / 2 * (1 + 2 ** -20))


def test_half_way_quotients_round_to_even():
    # row max 127 gives scale 1 exactly, so x/scale = x; x.5 values tie.
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.0]], np.float32)
    q, scale = oroute.int8_row_quant(x)
    assert scale[0] == 1.0
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 3]


def test_route_int8_moves_token_rows_by_the_scatter_index():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((6, 32)).astype(np.float32)
    ids = draw_expert_ids(6, 5, 3, seed_index=77)
    r = oroute.route_int8(x, ids, 5)
    q, scale = oroute.int8_row_quant(x)
    for f in range(ids.size):
        i = r["expanded_row_idx"][f]
        assert np.array_equal(r["expanded_x"][i], q[f // 3])
        assert r["expanded_scale"][i] == scale[f // 3]
