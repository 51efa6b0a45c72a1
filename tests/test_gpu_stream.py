"""GPU tests of the chunk-streamed front end (moe_ring_*, moe_forward_streamed, and
moe_forward_absorb + moe_forward_seal).

The streamed layer runs each token chunk as a layer call of its own; every token's result
is computed exactly as in a whole-batch call (same kernels' per-row arithmetic, same K
order), so the streamed output must equal moe_forward's bit for bit, and that output is
itself checked against the oracle here.  Cases: chunk sizes from 1 token to more than the
batch (partial last chunk), serialized production then consumption, produce/consume
alternating on a one-slot ring (repeated ring wrap), producer and consumer on two streams,
graph capture and replay, and the bounded waits' time-out status (forced from the host
with a tiny time limit: every kernel still exits normally)."""

import sys

import numpy as np
import pytest
import torch

import routed_moe_layer_amd as rm
from moe_inputs import LayerConfig
from tests.problem import build_layer_problem, oracle_forward
from tests.gpu_harness import dev, host, empty_bytes, prepare, DeviceLayer, check_guard
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


CFG = LayerConfig(name="stream_T200_H256_I128_E16_k4", T=200, H=256, I=128, E=16, k=4,
                  w_std=0.05, seed_index=60)


@pytest.fixture(scope="module")
def layer():
    p = build_layer_problem(CFG)
    prepared = prepare(CFG, p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    L = DeviceLayer(p, prepared)
    batch = host(L.forward().clone(), np.uint16)
    L.check_guards()
    # the batch output is the oracle-checked reference of every streamed run
    st, res = compare.check_layer(p, batch, L.intermediates(), oracle_forward(p))
    _say(f"batch vs oracle: code diffs {st['n_diff']}/{st['n_codes']}, {compare.fmt(res)}")
    return p, L, batch


class Ring:
    def __init__(self, L, slots, C):
        self.L, self.S, self.C = L, slots, C
        self.lay = rm.moe_ring_layout(L.dims, slots, C)
        self.buf = torch.zeros(self.lay["total"] + 4096, dtype=torch.uint8, device="cuda")
        self.buf[self.lay["total"]:].fill_(0xA5)                      # guard
        self.ring = rm.make_ring((self.buf.data_ptr(), self.lay["total"]), slots, C)
        H, k = CFG.H, CFG.k
        b = self.buf
        self.x = b[self.lay["x"]:self.lay["x"] + slots * C * H * 2].view(torch.int16).view(slots, C, H)
        self.ids = b[self.lay["expert_ids"]:self.lay["expert_ids"] + slots * C * k * 4].view(
            torch.int32).view(slots, C, k)
        self.rw = b[self.lay["route_weights"]:self.lay["route_weights"] + slots * C * k * 2].view(
            torch.int16).view(slots, C, k)
        self.ws = empty_bytes(rm.moe_workspace_size(L.dims, C))
        self.sws = empty_bytes(rm.moe_sealed_workspace_size(L.dims, CFG.T))
        self.out = torch.full((CFG.T, CFG.H), -1, dtype=torch.int16, device="cuda")
        rm.moe_ring_init(L.dims, self.ring)

    def chunks(self, T):
        return (T + self.C - 1) // self.C

    def produce(self, n, T, src=None, stream=None, timeout_us=0, parts=("route", "layout")):
        L = self.L
        x, ids, rw = (L.x, L.ids, L.rw) if src is None else src
        s, C = n % self.S, self.C
        lo, hi = n * C, min(T, (n + 1) * C)
        st = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(st):
            if "route" in parts:
                rm.moe_ring_acquire(L.dims, self.ring, s, rm.MOE_RING_ROUTE, timeout_us, stream=st)
                self.ids[s, :hi - lo].copy_(ids[lo:hi])
                self.rw[s, :hi - lo].copy_(rw[lo:hi])
                rm.moe_ring_publish(L.dims, self.ring, s, rm.MOE_RING_ROUTE, stream=st)
            if "layout" in parts:
                rm.moe_ring_acquire(L.dims, self.ring, s, rm.MOE_RING_LAYOUT, timeout_us, stream=st)
                self.x[s, :hi - lo].copy_(x[lo:hi])
                rm.moe_ring_publish(L.dims, self.ring, s, rm.MOE_RING_LAYOUT, stream=st)

    def consume(self, T, first, num, stream=None, timeout_us=0):
        L = self.L
        rm.moe_forward_streamed(L.dims, self.ring, T, first, num, L.prepared, L.qx, L.alpha1,
                                L.qa, L.alpha2, L.beta, L.lam, self.ws, self.out,
                                timeout_us=timeout_us, stream=stream)

    def absorb(self, T, first, num, stream=None, timeout_us=0):
        rm.moe_forward_absorb(self.L.dims, self.ring, T, first, num, self.L.qx, self.sws,
                              timeout_us=timeout_us, stream=stream)

    def seal(self, T, stream=None):
        L = self.L
        rm.moe_forward_seal(L.dims, T, L.prepared, L.alpha1, L.qa, L.alpha2, L.beta, L.lam,
                            self.sws, self.out, stream=stream)

    def status(self):
        torch.cuda.synchronize()
        st = self.lay["status"]
        return int(self.buf[st:st + 4].view(torch.int32).item())

    def check(self):
        torch.cuda.synchronize()
        assert torch.all(self.buf[self.lay["total"]:] == 0xA5), "ring guard overwritten"
        check_guard(self.ws)
        check_guard(self.sws)


@pytest.mark.parametrize("C", [1, 7, 64, 200, 256])
def test_streamed_serialized_equals_batch(layer, C):
    """All chunks produced into a ring with a slot per chunk, then consumed: one stream."""
    _say(f"streamed serialized C={C}")
    p, L, batch = layer
    n = (CFG.T + C - 1) // C
    R = Ring(L, n, C)
    for i in range(n):
        R.produce(i, CFG.T)
    R.consume(CFG.T, 0, n)
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_streamed_one_slot_alternating(layer):
    """Produce and consume alternate chunk by chunk on one stream through a single slot:
    the slot is reused (and its generations advanced) for every chunk."""
    _say("streamed one slot alternating")
    p, L, batch = layer
    R = Ring(L, 1, 16)
    n = R.chunks(CFG.T)
    for i in range(n):
        R.produce(i, CFG.T, parts=("layout", "route") if i % 2 else ("route", "layout"))
        R.consume(CFG.T, i, 1)
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_streamed_producer_and_consumer_on_two_streams(layer):
    """Producer and consumer on two streams through a two-slot ring, enqueued chunk by
    chunk (produce chunk i, then consume chunk i): every wait then needs only publishes
    enqueued before it, which is valid whether the runtime puts the two streams on
    different hardware queues (they overlap; the producer's wait for a free slot depends
    on the consumer's stream) or on one (they run in enqueue order)."""
    _say("streamed two streams")
    p, L, batch = layer
    R = Ring(L, 2, 16)
    n = R.chunks(CFG.T)
    torch.cuda.synchronize()
    cons, prod = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(n):
        R.produce(i, CFG.T, stream=prod, timeout_us=10_000_000)
        R.consume(CFG.T, i, 1, stream=cons, timeout_us=10_000_000)
    torch.cuda.synchronize()
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_streamed_all_chunks_produced_first_on_another_stream(layer):
    """A ring with a slot per chunk, every chunk produced on one stream and then the
    whole stream consumed on another: the consumer's waits depend on the other stream's
    publishes only."""
    _say("streamed produce-all then consume, two streams")
    p, L, batch = layer
    R = Ring(L, 7, 32)
    n = R.chunks(CFG.T)
    torch.cuda.synchronize()
    cons, prod = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(n):
        R.produce(i, CFG.T, stream=prod, timeout_us=10_000_000)
    R.consume(CFG.T, 0, n, stream=cons, timeout_us=10_000_000)
    torch.cuda.synchronize()
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_streamed_graph_replay(layer):
    """Production and consumption of all chunks (two-slot ring, alternating) captured into
    one graph; every replay advances the device-side generations, reads the current
    source tokens and must equal a batch call on them."""
    _say("streamed graph replay")
    p, L, batch = layer
    R = Ring(L, 2, 32)
    n = R.chunks(CFG.T)
    src_x = L.x.clone()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(n):
            R.produce(i, CFG.T, src=(src_x, L.ids, L.rw), stream=s)
            if i >= 1:
                R.consume(CFG.T, i - 1, 1, stream=s)
        R.consume(CFG.T, n - 1, 1, stream=s)
    rng = np.random.default_rng(5)
    for rep in range(4):
        if rep % 2:
            perm = torch.from_numpy(rng.permutation(CFG.T)).cuda()
            src_x.copy_(L.x[perm])
        else:
            src_x.copy_(L.x)
        R.out.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert R.status() == rm.MOE_RING_OK, f"replay {rep}"
        got = host(R.out, np.uint16)
        # a batch call on the same tokens (eager work between replays)
        ref_out = torch.empty_like(L.out)
        rm.moe_forward(L.dims, CFG.T, src_x, L.ids, L.rw, L.prepared, L.qx, L.alpha1, L.qa,
                       L.alpha2, L.beta, L.lam, L.workspace, ref_out)
        torch.cuda.synchronize()
        assert np.array_equal(got, host(ref_out, np.uint16)), f"replay {rep}"
    R.check()


@pytest.mark.parametrize("C", [1, 7, 64, 200, 256])
def test_sealed_serialized_equals_batch(layer, C):
    """Scheduling option 2: all chunks produced into a ring with a slot per chunk,
    absorbed in one call, then sealed: the batch call's result bit for bit."""
    _say(f"sealed serialized C={C}")
    p, L, batch = layer
    n = (CFG.T + C - 1) // C
    R = Ring(L, n, C)
    for i in range(n):
        R.produce(i, CFG.T)
    R.absorb(CFG.T, 0, n)
    R.seal(CFG.T)
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_sealed_one_slot_alternating(layer):
    """Produce and absorb alternate chunk by chunk through one slot (the slot is released
    by every absorb before the stream ends), then one seal."""
    _say("sealed one slot alternating")
    p, L, batch = layer
    R = Ring(L, 1, 16)
    n = R.chunks(CFG.T)
    for i in range(n):
        R.produce(i, CFG.T, parts=("layout", "route") if i % 2 else ("route", "layout"))
        R.absorb(CFG.T, i, 1)
    R.seal(CFG.T)
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_sealed_producer_and_consumer_on_two_streams(layer):
    """Producer and consumer on two streams through a two-slot ring, enqueued chunk by
    chunk (the progress rule), the seal on the consumer's stream."""
    _say("sealed two streams")
    p, L, batch = layer
    R = Ring(L, 2, 16)
    n = R.chunks(CFG.T)
    torch.cuda.synchronize()
    cons, prod = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(n):
        R.produce(i, CFG.T, stream=prod, timeout_us=10_000_000)
        R.absorb(CFG.T, i, 1, stream=cons, timeout_us=10_000_000)
    R.seal(CFG.T, stream=cons)
    torch.cuda.synchronize()
    assert R.status() == rm.MOE_RING_OK
    R.check()
    assert np.array_equal(host(R.out, np.uint16), batch)


def test_sealed_graph_replay(layer):
    """Production, absorption and the seal of all chunks captured into one graph (two-slot
    ring); every replay must equal a batch call on the current source tokens."""
    _say("sealed graph replay")
    p, L, batch = layer
    R = Ring(L, 2, 32)
    n = R.chunks(CFG.T)
    src_x = L.x.clone()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(n):
            R.produce(i, CFG.T, src=(src_x, L.ids, L.rw), stream=s)
            R.absorb(CFG.T, i, 1, stream=s)
        R.seal(CFG.T, stream=s)
    rng = np.random.default_rng(6)
    for rep in range(4):
        if rep % 2:
            perm = torch.from_numpy(rng.permutation(CFG.T)).cuda()
            src_x.copy_(L.x[perm])
        else:
            src_x.copy_(L.x)
        R.out.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert R.status() == rm.MOE_RING_OK, f"replay {rep}"
        got = host(R.out, np.uint16)
        ref_out = torch.empty_like(L.out)
        rm.moe_forward(L.dims, CFG.T, src_x, L.ids, L.rw, L.prepared, L.qx, L.alpha1, L.qa,
                       L.alpha2, L.beta, L.lam, L.workspace, ref_out)
        torch.cuda.synchronize()
        assert np.array_equal(got, host(ref_out, np.uint16)), f"replay {rep}"
    R.check()


def test_wait_timeouts_set_status_and_return(layer):
    """Time-outs forced from the host with a 2 ms limit: a consumer waiting on a slot
    nobody publishes, and a producer re-acquiring a slot the consumer never freed."""
    _say("streamed wait time-outs")
    p, L, _ = layer
    R = Ring(L, 1, 16)
    R.produce(0, CFG.T, parts=("route",))          # the layout part is never published
    R.consume(CFG.T, 0, 1, timeout_us=2000)
    assert R.status() == rm.MOE_RING_CONSUMER_TIMEOUT
    # the expired chunk computed nothing from the slot: its output rows are zero, the rows
    # of the chunks never consumed keep their fill value
    out = host(R.out, np.uint16)
    assert np.all(out[:16] == 0) and np.all(out[16:] == 0xFFFF)
    # so is a chunk consumed later while the failure stands, even with its data published
    R.out.fill_(-1)
    R.produce(0, CFG.T, parts=("layout",))
    R.consume(CFG.T, 0, 1, timeout_us=2000)
    assert np.all(host(R.out, np.uint16)[:16] == 0)
    # the sealed front end likewise drops an expired chunk's ids
    rm.moe_ring_init(L.dims, R.ring)
    R.produce(0, CFG.T, parts=("route",))
    R.absorb(CFG.T, 0, 1, timeout_us=2000)
    assert R.status() == rm.MOE_RING_CONSUMER_TIMEOUT
    torch.cuda.synchronize()
    ids_tail = R.sws[rm.moe_workspace_size(L.dims, CFG.T):].view(torch.int32)[:16 * CFG.k]
    assert bool((ids_tail == -1).all())
    rm.moe_ring_init(L.dims, R.ring)
    assert R.status() == rm.MOE_RING_OK
    R.produce(0, CFG.T, parts=("route",))
    R.produce(1, CFG.T, parts=("route",), timeout_us=2000)   # slot 0 not consumed yet
    assert R.status() == rm.MOE_RING_PRODUCER_TIMEOUT
    R.check()


def test_streamed_chunks_take_other_kernels_than_the_batch():
    """T*k = 65536 routed rows: the batch call takes the many-rows FC1 and the resident FC2
    kernels, its chunks of 5000 tokens (20000 rows) the others; the per-row arithmetic
    is the same, so the outputs must agree bit for bit."""
    _say("streamed vs batch across kernel variants")
    cfg = LayerConfig(name="stream_T16384_H256_I128_E16_k4", T=16384, H=256, I=128, E=16, k=4,
                      w_std=0.05, seed_index=61)
    p = build_layer_problem(cfg, calib_tokens=np.arange(8))
    prepared = prepare(cfg, p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    L = DeviceLayer(p, prepared)
    batch = host(L.forward().clone(), np.uint16)
    C = 5000
    n = (cfg.T + C - 1) // C
    lay = rm.moe_ring_layout(L.dims, 2, C)
    buf = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    ring = rm.make_ring(buf, 2, C)
    rm.moe_ring_init(L.dims, ring)
    x = buf[lay["x"]:].view(torch.int16)[:2 * C * cfg.H].view(2, C, cfg.H)
    ids = buf[lay["expert_ids"]:].view(torch.int32)[:2 * C * cfg.k].view(2, C, cfg.k)
    rw = buf[lay["route_weights"]:].view(torch.int16)[:2 * C * cfg.k].view(2, C, cfg.k)
    ws = empty_bytes(rm.moe_workspace_size(L.dims, C))
    out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device="cuda")
    for i in range(n):
        s, lo, hi = i % 2, i * C, min(cfg.T, (i + 1) * C)
        for role, parts in ((rm.MOE_RING_ROUTE, ((ids, L.ids), (rw, L.rw))),
                            (rm.MOE_RING_LAYOUT, ((x, L.x),))):
            rm.moe_ring_acquire(L.dims, ring, s, role)
            for dst, src in parts:
                dst[s, :hi - lo].copy_(src[lo:hi])
            rm.moe_ring_publish(L.dims, ring, s, role)
        rm.moe_forward_streamed(L.dims, ring, cfg.T, i, 1, L.prepared, L.qx, L.alpha1, L.qa,
                                L.alpha2, L.beta, L.lam, ws, out)
    torch.cuda.synchronize()
    st = lay["status"]
    assert int(buf[st:st + 4].view(torch.int32).item()) == rm.MOE_RING_OK
    check_guard(ws)
    got = host(out, np.uint16)
    diff = np.nonzero(np.any(got != batch, axis=1))[0]
    assert diff.size == 0, f"{diff.size} rows differ, first {diff[:5]}"


def test_sealed_many_rows_equals_batch():
    """T*k = 65536 routed rows sealed from chunks of 5000 tokens through a two-slot ring:
    the seal takes the many-rows kernels (no f16 copy of x), like the batch call, and must
    equal it bit for bit."""
    _say("sealed many rows")
    cfg = LayerConfig(name="stream_T16384_H256_I128_E16_k4", T=16384, H=256, I=128, E=16, k=4,
                      w_std=0.05, seed_index=61)
    p = build_layer_problem(cfg, calib_tokens=np.arange(8))
    prepared = prepare(cfg, p["w13"], p["w13_sf"], p["w2"], p["w2_sf"])
    L = DeviceLayer(p, prepared)
    batch = host(L.forward().clone(), np.uint16)
    C = 5000
    n = (cfg.T + C - 1) // C
    lay = rm.moe_ring_layout(L.dims, 2, C)
    buf = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    ring = rm.make_ring(buf, 2, C)
    rm.moe_ring_init(L.dims, ring)
    x = buf[lay["x"]:].view(torch.int16)[:2 * C * cfg.H].view(2, C, cfg.H)
    ids = buf[lay["expert_ids"]:].view(torch.int32)[:2 * C * cfg.k].view(2, C, cfg.k)
    rw = buf[lay["route_weights"]:].view(torch.int16)[:2 * C * cfg.k].view(2, C, cfg.k)
    ws = empty_bytes(rm.moe_sealed_workspace_size(L.dims, cfg.T))
    out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device="cuda")
    for i in range(n):
        s, lo, hi = i % 2, i * C, min(cfg.T, (i + 1) * C)
        for role, parts in ((rm.MOE_RING_ROUTE, ((ids, L.ids), (rw, L.rw))),
                            (rm.MOE_RING_LAYOUT, ((x, L.x),))):
            rm.moe_ring_acquire(L.dims, ring, s, role)
            for dst, src in parts:
                dst[s, :hi - lo].copy_(src[lo:hi])
            rm.moe_ring_publish(L.dims, ring, s, role)
        rm.moe_forward_absorb(L.dims, ring, cfg.T, i, 1, L.qx, ws)
    rm.moe_forward_seal(L.dims, cfg.T, L.prepared, L.alpha1, L.qa, L.alpha2, L.beta, L.lam, ws,
                        out)
    torch.cuda.synchronize()
    st = lay["status"]
    assert int(buf[st:st + 4].view(torch.int32).item()) == rm.MOE_RING_OK
    check_guard(ws)
    got = host(out, np.uint16)
    diff = np.nonzero(np.any(got != batch, axis=1))[0]
    assert diff.size == 0, f"{diff.size} rows differ, first {diff[:5]}"
