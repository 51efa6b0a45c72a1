"""CPU checks of the chunk-streamed front end: the ring layout and argument validation of
the C ABI (no GPU needed: validation returns before any HIP call), and a model of the
ring's counter rules run under random interleavings of two producers and the consumer.

The model restates the documented rules (the device kernels implement the same ones):
  producer p, chunk n, slot s = n % S:
      acquire: wait until consumed[s] >= seq_p[s]
      write its payload part, then seq_p[s] += 1; ready_p[s] = seq_p[s]
  consumer, chunk n: want = cseq[s] + 1; wait until ready_route[s] >= want and
      ready_layout[s] >= want; read the slot; cseq[s] = want; consumed[s] = want
and checks safety (the consumer reads exactly chunk n's parts; no part is overwritten
before it is consumed) and progress (every schedule finishes), also over repeated runs
without re-initialization (graph replay)."""

import random

import pytest

import routed_moe_layer_amd as rm

D = rm.MoeDims(256, 64, 16, 4)


def test_ring_layout_sizes_and_alignment():
    lay = rm.moe_ring_layout(D, 3, 10)
    assert lay["x"] == 0
    assert lay["expert_ids"] >= 3 * 10 * 256 * 2
    assert lay["route_weights"] >= lay["expert_ids"] + 3 * 10 * 4 * 4
    assert lay["counters"] >= lay["route_weights"] + 3 * 10 * 4 * 2
    assert lay["status"] >= lay["counters"] + 3 * 64
    assert lay["total"] >= lay["status"] + 4
    assert all(v % 256 == 0 for v in lay.values())


@pytest.mark.parametrize("S,C", [(0, 4), (4097, 4), (2, 0), (2, rm.MOE_MAX_TOKENS + 1)])
def test_ring_layout_rejects_bad_shapes(S, C):
    with pytest.raises(rm.MoeError) as ei:
        rm.moe_ring_layout(D, S, C)
    assert ei.value.status == -1


def test_ring_calls_validate_before_any_hip_call():
    lay = rm.moe_ring_layout(D, 2, 8)
    good = rm.MoeRing(1 << 20, lay["total"], 2, 8)
    cases = [
        (lambda: rm.moe_ring_init(D, rm.MoeRing(None, lay["total"], 2, 8), stream=0), -1),
        (lambda: rm.moe_ring_init(D, rm.MoeRing((1 << 20) + 16, lay["total"], 2, 8), stream=0), -1),
        (lambda: rm.moe_ring_init(D, rm.MoeRing(1 << 20, lay["total"] - 1, 2, 8), stream=0), -3),
        (lambda: rm.moe_ring_acquire(D, good, 2, rm.MOE_RING_ROUTE, stream=0), -1),
        (lambda: rm.moe_ring_acquire(D, good, -1, rm.MOE_RING_ROUTE, stream=0), -1),
        (lambda: rm.moe_ring_acquire(D, good, 0, 7, stream=0), -1),
        (lambda: rm.moe_ring_publish(D, good, 5, rm.MOE_RING_LAYOUT, stream=0), -1),
        (lambda: rm.moe_ring_publish(D, good, 0, 2, stream=0), -1),
    ]
    ws = rm.moe_workspace_size(D, 8)
    fwd = dict(dims=D, ring=good, total_tokens=20, first_chunk=0, num_chunks=3, prepared=1 << 24,
               qx=256, alpha1=512, qa=768, alpha2=1024, situ_beta=None, situ_linear_beta=None,
               workspace=1 << 26, out=1 << 28, workspace_bytes=ws, stream=0)
    for kw, code in ((dict(num_chunks=4), -1), (dict(first_chunk=3, num_chunks=1), -1),
                     (dict(total_tokens=0), -1), (dict(num_chunks=0), -1),
                     (dict(workspace_bytes=ws - 1), -3), (dict(out=(1 << 28) + 8), -1),
                     (dict(dims=rm.MoeDims(200, 64, 16, 4)), -2)):
        a = dict(fwd); a.update(kw)
        cases.append((lambda a=a: rm.moe_forward_streamed(**a), code))
    for fn, code in cases:
        with pytest.raises(rm.MoeError) as ei:
            fn()
        assert ei.value.status == code


def test_sealed_calls_validate_before_any_hip_call():
    """moe_forward_absorb / moe_forward_seal (scheduling option 2) reject bad arguments on
    the host; the sealed workspace holds the layer's workspace for the whole stream plus
    its expert ids and route weights."""
    T, k = 20, D.top_k
    ws = rm.moe_sealed_workspace_size(D, T)
    assert ws >= rm.moe_workspace_size(D, T) + T * k * 4 + T * k * 2
    assert rm.moe_sealed_workspace_size(D, 2 * T) > ws
    for bad in (0, rm.MOE_MAX_TOKENS + 1):
        with pytest.raises(rm.MoeError) as ei:
            rm.moe_sealed_workspace_size(D, bad)
        assert ei.value.status == -1
    lay = rm.moe_ring_layout(D, 2, 8)
    good = rm.MoeRing(1 << 20, lay["total"], 2, 8)
    absorb = dict(dims=D, ring=good, total_tokens=T, first_chunk=0, num_chunks=3, qx=256,
                  workspace=1 << 26, workspace_bytes=ws, stream=0)
    seal = dict(dims=D, total_tokens=T, prepared=1 << 24, alpha1=512, qa=768, alpha2=1024,
                situ_beta=None, situ_linear_beta=None, workspace=1 << 26, out=1 << 28,
                workspace_bytes=ws, stream=0)
    cases = []
    for kw, code in ((dict(num_chunks=4), -1), (dict(first_chunk=3, num_chunks=1), -1),
                     (dict(total_tokens=0), -1), (dict(qx=None), -1),
                     (dict(workspace_bytes=ws - 1), -3), (dict(workspace=(1 << 26) + 16), -1),
                     (dict(ring=rm.MoeRing(1 << 20, lay["total"] - 1, 2, 8)), -3),
                     (dict(dims=rm.MoeDims(200, 64, 16, 4)), -2)):
        a = dict(absorb); a.update(kw)
        cases.append((lambda a=a: rm.moe_forward_absorb(**a), code))
    for kw, code in ((dict(total_tokens=0), -1), (dict(workspace_bytes=ws - 1), -3),
                     (dict(workspace=None), -1), (dict(out=(1 << 28) + 8), -1),
                     (dict(prepared=None), -1), (dict(dims=rm.MoeDims(200, 64, 16, 4)), -2)):
        a = dict(seal); a.update(kw)
        cases.append((lambda a=a: rm.moe_forward_seal(**a), code))
    for fn, code in cases:
        with pytest.raises(rm.MoeError) as ei:
            fn()
        assert ei.value.status == code


class RingModel:
    def __init__(self, S):
        self.S = S
        self.ready = {"route": [0] * S, "layout": [0] * S}
        self.seq = {"route": [0] * S, "layout": [0] * S}
        self.consumed = [0] * S
        self.cseq = [0] * S
        self.payload = {"route": [None] * S, "layout": [None] * S}


def _programs(n_chunks, S):
    """Each actor's list of steps; a step is (kind, chunk)."""
    prod = {p: [s for n in range(n_chunks) for s in (("acquire", n), ("write", n), ("publish", n))]
            for p in ("route", "layout")}
    cons = [s for n in range(n_chunks) for s in (("wait", n), ("read", n), ("done", n))]
    return prod, cons


def _run(model, n_chunks, rng, run_id, read_log):
    S = model.S
    prod, cons = _programs(n_chunks, S)
    pc = {"route": 0, "layout": 0, "consumer": 0}
    progs = {"route": prod["route"], "layout": prod["layout"], "consumer": cons}
    while any(pc[a] < len(progs[a]) for a in pc):
        enabled = []
        for a, prog in progs.items():
            if pc[a] >= len(prog):
                continue
            kind, n = prog[pc[a]]
            s = n % S
            if kind == "acquire" and model.consumed[s] < model.seq[a][s]:
                continue
            if kind == "wait":
                want = model.cseq[s] + 1
                if model.ready["route"][s] < want or model.ready["layout"][s] < want:
                    continue
            enabled.append(a)
        assert enabled, "deadlock"
        a = rng.choice(enabled)
        kind, n = progs[a][pc[a]]
        s = n % S
        if kind == "write":
            old = model.payload[a][s]
            # never overwrite a part the consumer has not read yet
            assert old is None or old in read_log, (a, n, old)
            model.payload[a][s] = (run_id, a, n)
        elif kind == "publish":
            model.seq[a][s] += 1
            model.ready[a][s] = model.seq[a][s]
        elif kind == "read":
            got = (model.payload["route"][s], model.payload["layout"][s])
            assert got == ((run_id, "route", n), (run_id, "layout", n)), (n, got)
            read_log.update(got)
        elif kind == "done":
            model.cseq[s] += 1
            model.consumed[s] = model.cseq[s]
        pc[a] += 1


@pytest.mark.parametrize("S,n_chunks", [(1, 9), (2, 9), (3, 7), (5, 5), (8, 3)])
def test_protocol_model_is_safe_and_live_under_random_schedules(S, n_chunks):
    for seed in range(200):
        rng = random.Random(seed * 31 + S)
        model = RingModel(S)
        read_log = set()
        for run in range(3):                     # replays without re-initialization
            _run(model, n_chunks, rng, run, read_log)


def test_protocol_model_serialized_orders():
    """Serialized on one stream: all production first is valid when every chunk has its
    own slot; alternating production and consumption is valid with any slot count."""
    def serial(S, n_chunks, order):
        model = RingModel(S)
        prod, cons = _programs(n_chunks, S)
        steps = []
        if order == "all_first":
            steps = [("route", x) for x in prod["route"]] + [("layout", x) for x in prod["layout"]] \
                + [("consumer", x) for x in cons]
        else:
            for n in range(n_chunks):
                steps += [("route", x) for x in prod["route"][3 * n:3 * n + 3]]
                steps += [("layout", x) for x in prod["layout"][3 * n:3 * n + 3]]
                steps += [("consumer", x) for x in cons[3 * n:3 * n + 3]]
        for a, (kind, n) in steps:
            s = n % S
            if kind == "acquire" and model.consumed[s] < model.seq[a][s]:
                return False                      # would wait forever on one stream
            if kind == "wait":
                want = model.cseq[s] + 1
                if model.ready["route"][s] < want or model.ready["layout"][s] < want:
                    return False
            if kind == "publish":
                model.seq[a][s] += 1
                model.ready[a][s] = model.seq[a][s]
            if kind == "done":
                model.cseq[s] += 1
                model.consumed[s] = model.cseq[s]
        return True

    assert serial(6, 6, "all_first")
    assert not serial(2, 6, "all_first")
    for S in (1, 2, 5):
        assert serial(S, 7, "alternate")
