"""GPU parity of moe_topk_softmax (top-k expert selection with softmax route weights over
the picks) against oracle.topk_softmax: the expert ids bit for bit (the selection only
compares fp32 logits), the BF16 weights equal or one BF16 step apart (fp32 softmax on the
GPU against float64 in the oracle can round differently only next to a rounding tie)."""

import sys

import numpy as np
import pytest
import torch

import oracle
import routed_moe_layer_amd as rm
from tests.gpu_harness import dev, host

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


def _run(z, k):
    T, E = z.shape
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), -7, dtype=torch.int16, device="cuda")
    rm.moe_topk_softmax(T, E, k, dev(z), ids, w)
    torch.cuda.synchronize()
    return host(ids), host(w, np.uint16)


CASES = [("T16_E896_k16", 16, 896, 16, "normal"), ("T1_E256_k8", 1, 256, 8, "normal"),
         ("T1000_E896_k16", 1000, 896, 16, "normal"), ("T37_E16_k4", 37, 16, 4, "normal"),
         ("T50_E4096_k64", 50, 4096, 64, "normal"), ("T20_E5_k5", 20, 5, 5, "normal"),
         ("T64_E3_k1", 64, 3, 1, "normal"), ("T200_E64_k8_ties", 200, 64, 8, "ties"),
         ("T9_E1000_k2_wide", 9, 1000, 2, "wide")]


@pytest.mark.parametrize("name,T,E,k,kind", CASES, ids=[c[0] for c in CASES])
def test_topk_softmax_matches_oracle(name, T, E, k, kind):
    _say(f"topk {name}")
    rng = np.random.default_rng(T * 7 + E)
    if kind == "ties":
        z = rng.integers(-2, 3, (T, E)).astype(np.float32)
        z[rng.random((T, E)) < 0.2] = -0.0                # equal to +0.0
    elif kind == "wide":
        z = (rng.standard_normal((T, E)) * 30).astype(np.float32)
    else:
        z = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = _run(z, k)
    want_ids, want_w = oracle.topk_softmax(z, k)
    assert np.array_equal(ids, want_ids)
    step = np.abs(w.astype(np.int32) - want_w.astype(np.int32))
    assert step.max() <= 1, f"weights differ by {step.max()} BF16 steps"
    assert (step == 0).mean() >= 0.99


def test_topk_feeds_the_layer_layout():
    """The outputs are the [T, k] ids and BF16 weights moe_forward takes: distinct ids per
    token and weights summing to one within BF16 rounding."""
    _say("topk layout")
    rng = np.random.default_rng(11)
    z = rng.standard_normal((300, 896)).astype(np.float32)
    ids, w = _run(z, 16)
    assert all(len(set(r)) == 16 for r in ids.tolist())
    wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
    assert np.all(np.abs(wf.sum(1) - 1) <= 16 * 2.0 ** -9)


def test_topk_graph_capture_replay():
    _say("topk graph capture/replay")
    rng = np.random.default_rng(12)
    z = dev(rng.standard_normal((64, 896)).astype(np.float32))
    ids = torch.zeros((64, 16), dtype=torch.int32, device="cuda")
    w = torch.zeros((64, 16), dtype=torch.int16, device="cuda")
    rm.moe_topk_softmax(64, 896, 16, z, ids, w)
    torch.cuda.synchronize()
    want_i, want_w = host(ids).copy(), host(w).copy()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rm.moe_topk_softmax(64, 896, 16, z, ids, w, stream=s)
    for rep in range(3):
        ids.fill_(-1)
        w.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ids), want_i) and np.array_equal(host(w), want_w), rep
        rm.moe_topk_softmax(64, 896, 16, z, ids, w)
        torch.cuda.synchronize()
