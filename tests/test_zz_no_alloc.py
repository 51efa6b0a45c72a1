"""moe_forward_noalloc (the layer for callers that cannot allocate: its workspace is a
fixed array in the GPU's memory) against moe_forward with a caller workspace: the same
kernels, so the outputs must be identical bit for bit -- on two calls in a row, the second
with fewer tokens, and on a later call after other work used the array."""

import sys

import numpy as np
import pytest
import torch

import routed_moe_layer_amd as rm
from moe_inputs import LayerConfig
from tests.problem import build_layer_problem
from tests.gpu_harness import host, prepare, DeviceLayer

pytestmark = pytest.mark.gpu

CFG = LayerConfig(name="noalloc_T96_H512_I128_E32_k4", T=96, H=512, I=128, E=32, k=4,
                  w_std=0.05, seed_index=90)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(L, out):
    rm.moe_forward_noalloc(L.dims, L.T, L.x, L.ids, L.rw, L.prepared, L.qx, L.alpha1, L.qa,
                           L.alpha2, L.beta, L.lam, out)


def test_noalloc_equals_moe_forward_on_two_calls_the_second_smaller():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    _say(f"noalloc {CFG.name}")
    p = build_layer_problem(CFG)
    prepared = prepare(CFG, p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    for T in (CFG.T, 17):                           # the second call has fewer tokens
        L = DeviceLayer(p, prepared, T=T)
        want = host(L.forward().clone(), np.uint16)
        out = torch.full_like(L.out, -1)
        _noalloc(L, out)
        torch.cuda.synchronize()
        got = host(out, np.uint16)
        assert np.array_equal(got, want), f"T={T}: {int((got != want).sum())} outputs differ"
        _say(f"  T={T}: identical to moe_forward")
    # the array keeps the last call's contents; a call on the full batch again is unaffected
    L = DeviceLayer(p, prepared)
    out = torch.full_like(L.out, -1)
    _noalloc(L, out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out, np.uint16), host(L.forward(), np.uint16))


def test_noalloc_rejects_batches_beyond_its_array():
    d = rm.MoeDims(3584, 384, 896, 16)
    assert rm.moe_workspace_size(d, 262) <= rm.MOE_NOALLOC_SCRATCH_BYTES
    assert rm.moe_workspace_size(d, 263) > rm.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(rm.MoeError) as ei:
        rm.moe_forward_noalloc(d, 263, 4096, 8192, 8192, 1 << 20, 256, 512, 768, 1024, None,
                               None, 1 << 22, stream=0)
    assert ei.value.status == -2                       # unsupported: before any GPU work
