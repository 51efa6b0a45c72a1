"""Pins of the oracle's top-k selection and softmax route weights: a pure-Python selection
by repeated maximum (with ties), torch.topk on distinct logits, and closed forms of the
weights (k = 1, equal logits, the two-expert sigmoid)."""

import math

import numpy as np
import pytest
import torch

from oracle import router as orouter
from oracle.codecs import bf16_bits_to_f32


def _select(row, k):
    taken, out = set(), []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:          # strict: the lower id wins ties
                best = e
        taken.add(best)
        out.append(best)
    return out


@pytest.mark.parametrize("T,E,k", [(5, 8, 3), (7, 16, 4), (3, 64, 16), (4, 5, 5)])
def test_selection_matches_repeated_maximum_with_ties(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    z = rng.integers(-3, 4, (T, E)).astype(np.float32)   # many ties
    ids, _ = orouter.topk_softmax(z, k)
    for t in range(T):
        assert ids[t].tolist() == _select(z[t].tolist(), k)


def test_selection_matches_torch_topk_on_distinct_logits():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 896)).astype(np.float32)
    ids, _ = orouter.topk_softmax(z, 16)
    tk = torch.topk(torch.from_numpy(z), 16, dim=1, sorted=True).indices.numpy()
    assert np.array_equal(ids, tk)


def test_weight_closed_forms():
    z = np.array([[0.3, -1.0, 2.5, 0.0]], np.float32)
    _, w = orouter.topk_softmax(z, 1)
    assert w.tolist() == [[0x3F80]]                                   # 1.0
    _, w = orouter.topk_softmax(np.full((1, 6), 0.7, np.float32), 4)
    assert np.all(bf16_bits_to_f32(w) == np.float32(0.25))
    ids, w = orouter.topk_softmax(z, 2)
    a, b = 2.5, 0.3                                                   # experts 2 then 0
    assert ids.tolist() == [[2, 0]]
    s = 1.0 / (1.0 + math.exp(b - np.float64(np.float32(a))))
    exp_hi = bf16_bits_to_f32(w)[0]
    assert abs(exp_hi[0] - s) <= 2.0 ** -9 and abs(exp_hi[1] - (1 - s)) <= 2.0 ** -9


def test_weights_are_decreasing_and_sum_to_one():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((200, 256)).astype(np.float32) * 3
    ids, w = orouter.topk_softmax(z, 8)
    wf = bf16_bits_to_f32(w).astype(np.float64)
    assert np.all(np.diff(wf, axis=1) <= 0)
    # each weight is within half a BF16 ulp (2^-9 relative) of its exact value
    assert np.all(np.abs(wf.sum(axis=1) - 1.0) <= 8 * 2.0 ** -9)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        orouter.topk_softmax(np.zeros((2, 4), np.float32), 5)
