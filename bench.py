#!/usr/bin/env python3
"""Throughput of the routed-MoE layer on one MI355X, with its roofline and the CPU oracle.

One step = one moe_forward call (NVFP4 quantization of x, routing, FC1 + SiTU +
requantization, FC2, finalization) over one batch of seeded synthetic tokens at the
TP8-local shape H=3584, I=384, E=896, top-16, with every input already resident in HBM.

The headline line reports the prefill batch (T=16384, per-expert SiTU parameters, 0.5%
outlier channels x30): tokens/s, and the roofline of its dominant kernel (the FC1 grouped
GEMM, bound by the f16 MFMA).  The decode (T=16), mid (T=1024, Zipf 1.0) batches and the
band edges T=64 (decode) and T=4096 (prefill) are reported under "workloads" with their
HBM rooflines, per-step medians and spreads (at least 50 timed steps each) and the same
step captured into a graph and replayed; and the routing-and-int8-permute
primitive (moe_route, N=8192, H=7168, E=256, K=8) under "routing_primitive" with its
routed rows/s and HBM fraction, and two cases of its options (moe_route_v2) under
"routing_primitive.options", and the layer through the chunk-streamed front end
(moe_forward_streamed fed by a producer on a second stream) under "streamed".  Per-stage times come from HIP events recorded between
the stages on the launch stream (moe_forward_timed).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workloads prefill,decode,mid,decode64,prefill4k,route,stream]
                       [--summarize DIR]
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-MoE tokens/s at T=16/1024/16384; % peak HBM GB/s or MFMA util"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_F16_TFLOPS = 2500.0       # MI355X dense f16/bf16 MFMA
FC1_BYTES_PER_EXPERT = 768 * 1792 + 768 * 224          # codes + E4M3 scales
FC2_BYTES_PER_EXPERT = 3584 * 192 + 3584 * 24
STAGES = ("quantize_x", "route", "fc1_situ_requant", "fc2", "finalize")
MIN_SUB_STEPS = 50             # timed steps of every batch but the headline one
CSRC = os.path.join(ROOT, "routed_moe_layer_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def build_weights(cfg, torch, rm):
    """Draw every expert's BF16 weights, calibrate per-expert scales on the GPU, quantize with
    moe_quantize_nvfp4 and re-lay with moe_prepare_weights.  Returns prepared weights and
    the per-expert dequantization scales dW13, dW2 (device)."""
    from moe_inputs import draw_expert_weights
    from concurrent.futures import ThreadPoolExecutor
    E, H, I = cfg.E, cfg.H, cfg.I
    dims = rm.MoeDims(H, I, E, cfg.k)
    c13 = torch.empty((E * 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    s13 = torch.empty((E * 2 * I, H // 16), dtype=torch.uint8, device="cuda")
    c2 = torch.empty((E * H, I // 2), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((E * H, I // 16), dtype=torch.uint8, device="cuda")
    d13 = torch.empty(E, dtype=torch.float32, device="cuda")
    d2 = torch.empty(E, dtype=torch.float32, device="cuda")
    chunk = 64
    t0 = time.time()
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for e0 in range(0, E, chunk):
            es = list(range(e0, min(E, e0 + chunk)))
            pairs = list(ex.map(lambda e: draw_expert_weights(cfg, e), es))
            w13 = torch.from_numpy(np.stack([p[0] for p in pairs]).view(np.int16)).cuda()
            w2 = torch.from_numpy(np.stack([p[1] for p in pairs]).view(np.int16)).cuda()
            n = len(es)
            for w, dst_d, dst_c, dst_s, R, K in ((w13, d13, c13, s13, 2 * I, H),
                                                 (w2, d2, c2, s2, H, I)):
                amax = w.view(torch.bfloat16).float().abs().amax(dim=(1, 2))
                d = torch.where(amax > 0, amax / 2688.0, torch.ones_like(amax))
                q = (1.0 / d).contiguous()
                dst_d[e0:e0 + n] = d
                rm.moe_quantize_nvfp4(w, n, R, K, q, dst_c[e0 * R:(e0 + n) * R],
                                      dst_s[e0 * R:(e0 + n) * R])
            torch.cuda.synchronize()
    prepared = torch.empty(rm.moe_prepared_weights_size(dims), dtype=torch.uint8, device="cuda")
    rm.moe_prepare_weights(dims, c13, s13, c2, s2, prepared)
    torch.cuda.synchronize()
    log(f"weights drawn, quantized and prepared in {time.time() - t0:.1f} s")
    del c13, s13, c2, s2
    return prepared, d13, d2


def layer_workload(cfg, torch, rm, prepared, d13, d2, steps, warmup, events, rotations):
    """Time `steps` moe_forward calls of one workload; returns its result dict."""
    from moe_inputs import (draw_tokens, draw_expert_ids, draw_route_weights, draw_situ_params,
                            LayerConfig)
    E, H, I, k, T = cfg.E, cfg.H, cfg.I, cfg.k, cfg.T
    dims = rm.MoeDims(H, I, E, k)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = dev(draw_tokens(T, H, cfg.seed_index, cfg.outlier_frac, cfg.outlier_mult).view(np.int16))
    rw = dev(draw_route_weights(T, k, cfg.seed_index).view(np.int16))
    ids_host = [draw_expert_ids(T, E, k, cfg.seed_index + 100 * r, cfg.zipf_s)
                for r in range(rotations)]
    ids = [dev(a) for a in ids_host]
    beta, lam = draw_situ_params(cfg)
    beta = None if beta is None else dev(beta)
    lam = None if lam is None else dev(lam)
    # calibration (model preparation): dX from the batch, dA from one calibration call
    amax_x = x.view(torch.bfloat16).float().abs().amax()
    dX = torch.where(amax_x > 0, amax_x / 2688.0, torch.ones_like(amax_x))
    qx = (1.0 / dX).reshape(1).contiguous()
    alpha1 = (dX * d13).contiguous()
    ones = torch.ones(E, dtype=torch.float32, device="cuda")
    ws_bytes = rm.moe_workspace_size(dims, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    lay = rm.moe_workspace_layout(dims, T)
    rm.moe_forward(dims, T, x, ids[0], rw, prepared, qx, alpha1, ones, ones, beta, lam, ws, out)
    a_amax = ws[lay["a_amax"]: lay["a_amax"] + 4 * E].view(torch.float32).amax()
    dA = torch.where(a_amax > 0, a_amax / 2688.0, torch.ones_like(a_amax))
    qa = torch.full((E,), 1.0, dtype=torch.float32, device="cuda") / dA
    alpha2 = (dA * d2).contiguous()
    torch.cuda.synchronize()

    def call(i, evs=None):
        args = (dims, T, x, ids[i % rotations], rw, prepared, qx, alpha1, qa, alpha2, beta, lam,
                ws, out)
        if evs is None:
            rm.moe_forward(*args)
        else:
            rm.moe_forward_timed(*args, evs)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    nev = rm.MOE_FORWARD_STAGES + 1
    evs = [events.create(nev) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = np.zeros((steps, len(STAGES)))
    for i in range(steps):
        for s in range(len(STAGES)):
            stage_ms[i, s] = events.elapsed_ms(evs[i][s], evs[i][s + 1])
    gpu_ms = [events.elapsed_ms(evs[i][0], evs[i][-1]) for i in range(steps)]
    for e in evs:
        events.destroy(e)
    ms_per_step = wall * 1e3 / steps
    graph = graph_replay_ms(lambda i, stream: rm.moe_forward(
        dims, T, x, ids[i], rw, prepared, qx, alpha1, qa, alpha2, beta, lam, ws, out,
        stream=stream), rotations, torch, steps, warmup, events)
    # algorithmic work
    distinct = np.mean([len(np.unique(a)) for a in ids_host])
    weight_bytes = distinct * (FC1_BYTES_PER_EXPERT + FC2_BYTES_PER_EXPERT)
    act_bytes = T * H * 2 * 2 + T * k * (4 + 2)                  # x, out, ids, route weights
    R = T * k
    fc1_flops = 2.0 * R * 2 * I * H
    fc2_flops = 2.0 * R * H * I
    st = {name: float(np.mean(stage_ms[:, j])) for j, name in enumerate(STAGES)}
    res = {
        "workload": cfg.name, "T": T, "tokens_per_s": T / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step, "gpu_ms_per_step": float(np.mean(gpu_ms)),
        "steps": steps, "gpu_ms_step_stats": _stats(gpu_ms),
        "graph_replay_ms_step_stats": graph,
        "graph_replay_tokens_per_s": T / (graph["median"] * 1e-3),
        "stage_ms": st, "stage_ms_median": {name: float(np.median(stage_ms[:, j]))
                                            for j, name in enumerate(STAGES)},
        "distinct_experts": float(distinct),
        "algorithmic_bytes": float(weight_bytes + act_bytes),
        "hbm_frac_of_step": (weight_bytes + act_bytes) / (ms_per_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "flops": fc1_flops + fc2_flops,
        "mfma_frac_of_step": (fc1_flops + fc2_flops) / (ms_per_step * 1e-3) / (PEAK_F16_TFLOPS * 1e12),
        "fc1": {"flops": fc1_flops, "bytes": distinct * FC1_BYTES_PER_EXPERT + T * H * 9 / 16,
                "ms": st["fc1_situ_requant"]},
        "fc2": {"flops": fc2_flops, "bytes": distinct * FC2_BYTES_PER_EXPERT, "ms": st["fc2"]},
        "rotations": rotations,
    }
    # the library runs FC1 and FC2 as one launch when every routed row can have a compute
    # unit of its own (and the shapes suit it); both stage marks then follow that launch,
    # so FC1's stage holds the two GEMMs
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    if R <= cus and I % 128 == 0 and I <= 384 and H % 512 == 0:
        both = res["fc1"]["bytes"] + res["fc2"]["bytes"]
        res["fused_fc1_fc2"] = {"bytes": both, "flops": fc1_flops + fc2_flops,
                                "ms": st["fc1_situ_requant"] + st["fc2"],
                                "kernel": "layer_small_fused_kernel"}
    keep = dict(x=x, ids=ids_host[0], rw=rw, qx=qx, alpha1=alpha1, qa=qa, alpha2=alpha2,
                beta=beta, lam=lam)
    return res, keep


def _stats(ms):
    """Median, spread and extremes (ms) of per-step times."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "min": float(a.min()), "max": float(a.max()),
            "n": int(a.size)}


def graph_replay_ms(capture_call, rotations, torch, steps, warmup, events):
    """Per-step times (ms) of the layer call captured into a graph and replayed ("Cake SiTU
    backend", "Caller-owned execution": the caller may capture and replay): one graph per
    input rotation, replayed in turn, each replay bracketed by events on the launch stream."""
    side = torch.cuda.Stream()
    graphs = []
    torch.cuda.synchronize()
    for i in range(rotations):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            capture_call(i, side)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % rotations].replay()
    torch.cuda.synchronize()
    evs = [events.create(2) for _ in range(steps)]
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(steps):
        events.record(evs[i][0], stream)
        graphs[i % rotations].replay()
        events.record(evs[i][1], stream)
    torch.cuda.synchronize()
    ms = [events.elapsed_ms(e[0], e[1]) for e in evs]
    for e in evs:
        events.destroy(e)
    del graphs
    return _stats(ms)


# The chunk-streamed front end: (layer workload, tokens per slot, ring slots).
STREAM_CASES = {"prefill": (4096, 2), "mid": (256, 2)}


def streamed_workload(cfg, keep, torch, rm, prepared, chunk, slots, steps, warmup, events,
                      sealed=False):
    """Time the streamed layer on a layer workload's inputs: per step, a producer on a
    second stream fills a `slots`-slot ring chunk by chunk (copies of the resident ids,
    route weights and x into the slot, each part acquired and published) and the
    consumer runs on the launch stream, so production overlaps the consumer's work on
    earlier chunks.  The consumer is moe_forward_streamed (one chunk per call: chunk-local
    expert pools) or, when `sealed`, moe_forward_absorb per chunk and moe_forward_seal at
    the end of the stream (reservations across chunks)."""
    E, H, I, k, T = cfg.E, cfg.H, cfg.I, cfg.k, cfg.T
    dims = rm.MoeDims(H, I, E, k)
    x, rw = keep["x"], keep["rw"]
    ids = torch.from_numpy(np.ascontiguousarray(keep["ids"])).cuda()
    lay = rm.moe_ring_layout(dims, slots, chunk)
    buf = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    ring = rm.make_ring(buf, slots, chunk)
    rx = buf[lay["x"]:].view(torch.int16)[:slots * chunk * H].view(slots, chunk, H)
    rids = buf[lay["expert_ids"]:].view(torch.int32)[:slots * chunk * k].view(slots, chunk, k)
    rrw = buf[lay["route_weights"]:].view(torch.int16)[:slots * chunk * k].view(slots, chunk, k)
    ws_bytes = (rm.moe_sealed_workspace_size(dims, T) if sealed
                else rm.moe_workspace_size(dims, chunk))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    n = (T + chunk - 1) // chunk
    prod = torch.cuda.Stream()
    rm.moe_ring_init(dims, ring)
    torch.cuda.synchronize()

    def step():
        # chunk by chunk: produce chunk i on the producer stream, then consume it on the
        # launch stream; every wait needs only publishes enqueued before it, so the step
        # is valid whether or not the runtime gives the two streams separate queues
        for i in range(n):
            sl, lo, hi = i % slots, i * chunk, min(T, (i + 1) * chunk)
            with torch.cuda.stream(prod):
                rm.moe_ring_acquire(dims, ring, sl, rm.MOE_RING_ROUTE, stream=prod)
                rids[sl, :hi - lo].copy_(ids[lo:hi])
                rrw[sl, :hi - lo].copy_(rw[lo:hi])
                rm.moe_ring_publish(dims, ring, sl, rm.MOE_RING_ROUTE, stream=prod)
                rm.moe_ring_acquire(dims, ring, sl, rm.MOE_RING_LAYOUT, stream=prod)
                rx[sl, :hi - lo].copy_(x[lo:hi])
                rm.moe_ring_publish(dims, ring, sl, rm.MOE_RING_LAYOUT, stream=prod)
            if sealed:
                rm.moe_forward_absorb(dims, ring, T, i, 1, keep["qx"], ws)
            else:
                rm.moe_forward_streamed(dims, ring, T, i, 1, prepared, keep["qx"],
                                        keep["alpha1"], keep["qa"], keep["alpha2"],
                                        keep["beta"], keep["lam"], ws, out)
        if sealed:
            rm.moe_forward_seal(dims, T, prepared, keep["alpha1"], keep["qa"], keep["alpha2"],
                                keep["beta"], keep["lam"], ws, out)

    gpu_ms, wall_ms = _time_calls(step, torch, steps, warmup, events)
    torch.cuda.synchronize()
    status = int(buf[lay["status"]:lay["status"] + 4].view(torch.int32).item())
    if status != rm.MOE_RING_OK:
        raise RuntimeError(f"streamed run ended with ring status {status}")
    tag = "sealed" if sealed else "streamed"
    res = {"workload": f"{cfg.name}_{tag}_C{chunk}_S{slots}", "chunks": n,
           "tokens_per_s": T / (wall_ms * 1e-3), "ms_per_step": wall_ms,
           "gpu_ms_per_step": gpu_ms}
    if sealed:
        # the whole sealed step (production, absorption, seal) captured into one graph on
        # one stream and replayed, so the host's enqueue cost is out of the number
        def capture(i, st):
            for c in range(n):
                sl, lo, hi = c % slots, c * chunk, min(T, (c + 1) * chunk)
                rm.moe_ring_acquire(dims, ring, sl, rm.MOE_RING_ROUTE, stream=st)
                rids[sl, :hi - lo].copy_(ids[lo:hi])
                rrw[sl, :hi - lo].copy_(rw[lo:hi])
                rm.moe_ring_publish(dims, ring, sl, rm.MOE_RING_ROUTE, stream=st)
                rm.moe_ring_acquire(dims, ring, sl, rm.MOE_RING_LAYOUT, stream=st)
                rx[sl, :hi - lo].copy_(x[lo:hi])
                rm.moe_ring_publish(dims, ring, sl, rm.MOE_RING_LAYOUT, stream=st)
                rm.moe_forward_absorb(dims, ring, T, c, 1, keep["qx"], ws, stream=st)
            rm.moe_forward_seal(dims, T, prepared, keep["alpha1"], keep["qa"], keep["alpha2"],
                                keep["beta"], keep["lam"], ws, out, stream=st)
        g = graph_replay_ms(capture, 1, torch, steps, warmup, events)
        status = int(buf[lay["status"]:lay["status"] + 4].view(torch.int32).item())
        if status != rm.MOE_RING_OK:
            raise RuntimeError(f"graph-replayed sealed run ended with ring status {status}")
        res["graph_replay_ms_step_stats"] = g
        res["graph_replay_tokens_per_s"] = T / (g["median"] * 1e-3)
    return res


def _time_calls(call, torch, steps, warmup, events):
    """Mean HIP-event time (ms) of `call` over `steps` calls after `warmup`, and the wall
    time per call (ms)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [events.create(2) for _ in range(steps)]
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    for i in range(steps):
        events.record(evs[i][0], stream)
        call()
        events.record(evs[i][1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = float(np.mean([events.elapsed_ms(e[0], e[1]) for e in evs]))
    for e in evs:
        events.destroy(e)
    return gpu_ms, wall * 1e3 / steps


def route_workload(cfg, torch, rm, steps, warmup, events):
    """Time the routing-and-int8-permute primitive (moe_route) on its own workload: the
    stable sort by expert, the row maps, the per-expert cumsum and the expanded int8 rows
    with their dynamic scales.  Algorithmic bytes: x read once, ids, the expanded rows and
    scales and the three index arrays written once."""
    from moe_inputs import draw_route_inputs
    N, H, E, K = cfg.N, cfg.H, cfg.E, cfg.K
    xb, ids_h = draw_route_inputs(cfg)
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    ids = torch.from_numpy(np.ascontiguousarray(ids_h)).cuda()
    R = N * K
    ex = torch.empty((R, H), dtype=torch.int8, device="cuda")
    esc = torch.empty(R, dtype=torch.float32, device="cuda")
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    cs = torch.empty(E, dtype=torch.int32, device="cuda")
    sid = torch.empty(R, dtype=torch.int32, device="cuda")
    sri = torch.empty(R, dtype=torch.int32, device="cuda")
    ws = torch.empty(rm.moe_route_workspace_size(N, K, E), dtype=torch.uint8, device="cuda")

    def call():
        rm.moe_route(rm.MoeDims(H, 0, E, K), N, x, ids, rm.MOE_QUANT_INT8_ROW_DYNAMIC, None, sid,
                     sri, eri, cs, ex, esc, ws)

    gpu_ms, wall_ms = _time_calls(call, torch, steps, warmup, events)
    nbytes = N * H * 2 + R * 4 + R * H + R * 4 + 3 * R * 4 + E * 4
    res = {"workload": cfg.name, "N": N, "routed_rows_per_s": R / (gpu_ms * 1e-3),
           "ms_per_call": gpu_ms, "wall_ms_per_call": wall_ms,
           "algorithmic_bytes": float(nbytes),
           "hbm_frac": nbytes / (gpu_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)}
    # the same routing with the layer's NVFP4 quantization of the moved rows (qx from the
    # tokens' amax); bytes: x once, the ids, expanded codes and scales, three index arrays
    amax = x.view(torch.bfloat16).float().abs().amax()
    qx = (2688.0 / torch.where(amax > 0, amax, torch.ones_like(amax))).reshape(1).contiguous()
    exf = torch.empty((R, H // 2), dtype=torch.uint8, device="cuda")
    esf = torch.empty((R, H // 16), dtype=torch.uint8, device="cuda")

    def call_fp4():
        rm.moe_route(rm.MoeDims(H, 0, E, K), N, x, ids, rm.MOE_QUANT_NVFP4_G16, qx, sid, sri, eri,
                     cs, exf, esf, ws)

    g4, w4 = _time_calls(call_fp4, torch, steps, warmup, events)
    b4 = N * H * 2 + R * 4 + R * (H // 2 + H // 16) + 3 * R * 4 + E * 4
    res["nvfp4"] = {"workload": cfg.name.replace("_int8", "_nvfp4"), "ms_per_call": g4,
                    "wall_ms_per_call": w4, "routed_rows_per_s": R / (g4 * 1e-3),
                    "algorithmic_bytes": float(b4),
                    "hbm_frac": b4 / (g4 * 1e-3) / (PEAK_HBM_GBS * 1e9)}
    return res


# The routing page's two named fast cases, through moe_route_v2 on the routing workload's
# inputs: a large batch routed to one range of 32 experts (BF16 rows, scatter index,
# per-expert counts) and a single token (dynamic int8, key_value histogram).
ROUTE_OPTION_CASES = {
    "large_batch_range32": dict(N=8192, start=0, end=32,
                                opts=dict(expert_start=0, expert_end=32, quant_mode=-1,
                                          row_idx_type=1, expert_tokens_num_type=1)),
    "one_token_dynamic_kv": dict(N=1, start=0, end=256,
                                 opts=dict(expert_start=0, expert_end=256, quant_mode=1,
                                           expert_tokens_num_type=2)),
}


def route_options_workload(case, cfg, torch, rm, steps, warmup, events):
    """Time one moe_route_v2 case.  Algorithmic bytes: the ids, the x rows of tokens with
    at least one in-range id (read once), the expanded rows (and scales) of the in-range
    ids, the index output and the histogram, each once."""
    from moe_inputs import draw_route_inputs
    c = ROUTE_OPTION_CASES[case]
    xb, ids_h = draw_route_inputs(cfg)
    N, H, E, K = c["N"], cfg.H, cfg.E, cfg.K
    xb, ids_h = np.ascontiguousarray(xb[:N]), np.ascontiguousarray(ids_h[:N])
    opts = c["opts"]
    q = opts["quant_mode"]
    inr = (ids_h >= c["start"]) & (ids_h < c["end"])
    avail = int(inr.sum())
    tok_hit = int(inr.any(axis=1).sum())
    R = N * K
    elem = 2 if q == -1 else 1
    x = torch.from_numpy(xb.view(np.int16)).cuda()
    ids = torch.from_numpy(ids_h).cuda()
    ex = torch.empty((R, H * elem), dtype=torch.uint8, device="cuda")
    eri = torch.empty(R, dtype=torch.int32, device="cuda")
    kv = opts["expert_tokens_num_type"] == 2
    tok = torch.empty((E, 2) if kv else (c["end"] - c["start"],), dtype=torch.int32,
                      device="cuda")
    esc = torch.empty(R, dtype=torch.float32, device="cuda") if q == 1 else None
    ws = torch.empty(rm.moe_route_workspace_size(N, K, E), dtype=torch.uint8, device="cuda")
    o = rm.MoeRouteOptions(**opts)

    def call():
        rm.moe_route_v2(N, H, E, K, x, ids, o, ex, eri, expert_tokens=tok, expanded_scale=esc,
                        workspace=ws)

    gpu_ms, wall_ms = _time_calls(call, torch, steps, warmup, events)
    nbytes = (R * 4 + tok_hit * H * 2 + avail * (H * elem + (4 if q == 1 else 0)) + R * 4
              + tok.numel() * 4)
    return {"workload": f"{case}_N{N}_H{H}_E{E}_K{K}_experts{c['start']}-{c['end']}",
            "routed_rows": avail, "us_per_call": gpu_ms * 1e3, "wall_us_per_call": wall_ms * 1e3,
            "in_range_rows_per_s": avail / (gpu_ms * 1e-3), "algorithmic_bytes": float(nbytes),
            "hbm_frac": nbytes / (gpu_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)}


def topk_workload(T, E, k, torch, rm, steps, warmup, events):
    """Time moe_topk_softmax (router logits -> the layer's expert ids and route weights).
    Algorithmic bytes: the f32 logits read once, the ids and BF16 weights written once."""
    rng = np.random.default_rng(T + E)
    z = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.int16, device="cuda")

    def call():
        rm.moe_topk_softmax(T, E, k, z, ids, w)

    gpu_ms, wall_ms = _time_calls(call, torch, steps, warmup, events)
    nbytes = T * E * 4 + T * k * 6
    return {"workload": f"topk_softmax_T{T}_E{E}_k{k}", "us_per_call": gpu_ms * 1e3,
            "wall_us_per_call": wall_ms * 1e3, "algorithmic_bytes": float(nbytes),
            "hbm_frac": nbytes / (gpu_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)}


def cpu_baseline(cfg, keep, torch, n_tokens):
    """The oracle, as it stands, on a bounded sample of the same workload's tokens."""
    import oracle
    from tests.problem import ExpertStore
    from moe_inputs import draw_tokens, draw_route_weights
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    x = draw_tokens(cfg.T, cfg.H, cfg.seed_index, cfg.outlier_frac, cfg.outlier_mult)
    rw = draw_route_weights(cfg.T, cfg.k, cfg.seed_index)
    ids = keep["ids"]
    tokens = np.linspace(0, cfg.T - 1, n_tokens).astype(np.int64)
    h = lambda t: t.detach().cpu().numpy()
    a1, qa, a2 = h(keep["alpha1"]), h(keep["qa"]), h(keep["alpha2"])
    beta = None if keep["beta"] is None else h(keep["beta"])
    lam = None if keep["lam"] is None else h(keep["lam"])
    qx = np.float32(h(keep["qx"])[0])
    # canonical NVFP4 weights of the touched experts (weight preparation, not timed)
    from moe_inputs import draw_expert_weights
    used = np.unique(ids[tokens])
    qW13 = np.ones(cfg.E, np.float32)
    qW2 = np.ones(cfg.E, np.float32)
    for e in used:
        w13b, w2b = draw_expert_weights(cfg, int(e))
        qW13[e] = oracle.calibrate_weights(w13b[None])[1][0]
        qW2[e] = oracle.calibrate_weights(w2b[None])[1][0]
    store = ExpertStore(cfg, qW13, qW2, used)
    t0 = time.perf_counter()
    oracle.token_forward(tokens, x, ids, rw, store.w13, store.w13_sf, store.w2, store.w2_sf,
                         qx, a1, qa, a2, beta, lam)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_tokens} tokens of {cfg.name} ({n_tokens * cfg.k} routed rows, "
                      f"{len(used)} experts decoded), {dt:.1f} s"}


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    no summary exists or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            data = json.load(fh)
        entry = data.get(kernel)
        if not entry or entry.get("source_hash") != kernel_source_hash():
            return None
        return float(entry["bytes_per_launch"])
    except Exception:
        return None


# ---------------------------------------------------------------------------------------
# Profile summaries: turn the CSV output of the rocprofv3 runs (kernel trace per workload,
# FETCH_SIZE / WRITE_SIZE counters, and the plain-copy calibration) into the text
# summaries under profiles/ and the traffic table the roofline line reads.
PROFILE_WORKLOADS = {"prefill": "PREFILL_16K", "decode": "DECODE_16", "mid": "MID_1024",
                     "decode64": "DECODE_64", "prefill4k": "PREFILL_4K"}


def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _one(pattern):
    import glob
    hits = sorted(glob.glob(pattern))
    return hits[0] if hits else None


def _bench_line(log_path):
    """The JSON line a profiled bench.py run printed (None if absent)."""
    if not log_path or not os.path.exists(log_path):
        return None
    for ln in open(log_path, errors="replace"):
        ln = ln.strip()
        if ln.startswith("{") and '"metric"' in ln:
            return json.loads(ln)
    return None


def _short(name):
    n = name.replace("void ", "").replace("rmoe::", "")
    if n.startswith(("grouped_gemm_kernel", "grouped_gemm_pair_kernel", "fc2_kernel",
                     "fc2_stationary_kernel", "finalize",
                     "quantize", "route", "prepare", "topk", "layer_small_fused_kernel")):
        return n.split("(")[0]
    return n if len(n) <= 72 else n[:72] + "..."


def _role(name):
    n = _short(name)
    if n.startswith(("grouped_gemm_kernel<0", "grouped_gemm_pair_kernel<0")):
        return "fc1_kernel"
    if n.startswith(("grouped_gemm_kernel<1", "fc2_kernel", "fc2_stationary_kernel")):
        return "fc2_kernel"
    if n.startswith("finalize_kernel"):
        return "finalize_kernel"
    if n.startswith("layer_small_fused_kernel"):
        return "fused_kernel"
    return None


def summarize_profiles(src, out_dir):
    import moe_inputs
    os.makedirs(out_dir, exist_ok=True)
    cmd_trace = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace_{w} -o {w} "
                 "-- python3 <repo>/bench.py --workloads {w} --cpu-tokens 0 --steps 20 --warmup 5")
    cmd_pmc = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_{w}_{c} -o {w} -- python3 "
               "<repo>/bench.py --workloads {w} --cpu-tokens 0 --steps 3 --warmup 1")
    cmd_copy = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_copy_{c} -o copy -- python3 "
                "<repo>/bench.py --copy-calibration")
    # copy calibration: counter KiB per byte actually moved by a plain device copy
    factors = {}
    for c, key in (("FETCH_SIZE", "copy_bytes_read"), ("WRITE_SIZE", "copy_bytes_written")):
        f = _one(os.path.join(src, f"pmc_copy_{c}", "*counter_collection.csv"))
        if f is None:
            continue
        rows = [r for r in _read_csv(f) if "copy" in r["Kernel_Name"].lower()
                or "elementwise" in r["Kernel_Name"]]
        big = max(rows, key=lambda r: float(r["Counter_Value"]))
        kib = float(big["Counter_Value"])
        factors[c] = (1 << 30) / (kib * 1024.0)          # bytes moved per counted byte
    traffic = {"_copy_calibration": {
        "fetch_factor": factors.get("FETCH_SIZE"), "write_factor": factors.get("WRITE_SIZE"),
        "note": "bytes moved per counter byte, from a 1 GiB device-to-device copy"}}
    for w, cname in PROFILE_WORKLOADS.items():
        cfg = getattr(moe_inputs, cname)
        stats = _one(os.path.join(src, f"trace_{w}", "*kernel_stats.csv"))
        if stats is None:
            continue
        line = _bench_line(os.path.join(src, f"trace_{w}.log"))
        rows = _read_csv(stats)
        md = [f"# Kernel trace: routed-MoE layer, {cfg.name}", "",
              "Command (run from the repository root, after "
              "`cd /tmp && export TMPDIR=/tmp`):", "", "```", cmd_trace.format(w=w), "```", "",
              "Per-kernel statistics (`*_kernel_stats.csv`; all calls of the run: weight "
              "preparation, calibration, warmup and timed steps; `at::` kernels are the "
              "benchmark's own input setup):", "",
              "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
        for r in rows[:14]:
            md.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                      f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                      f"{float(r['Percentage']):.1f} |")
        if line:
            wl = line["workloads"][w]
            md += ["", "Stage times the same run measured with HIP events on the launch stream "
                   "(mean over the timed steps, ms): "
                   + ", ".join(f"{k} {v:.4f}" for k, v in wl["stage_ms"].items())
                   + f"; {wl['ms_per_step']:.3f} ms per step, {wl['tokens_per_s']:.0f} tokens/s. "
                   f"Kernel sources: `{line['kernel_source_hash']}`."]
        with open(os.path.join(out_dir, f"kernel_trace_T{cfg.T}.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
        # HBM bytes per launch from the counters, scaled by the copy calibration
        per = {}
        src_hash = None
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            f = _one(os.path.join(src, f"pmc_{w}_{c}", "*counter_collection.csv"))
            if f is None or c not in factors:
                continue
            pl = _bench_line(os.path.join(src, f"pmc_{w}_{c}.log"))
            if pl:
                src_hash = pl["kernel_source_hash"]
            for r in _read_csv(f):
                role = _role(r["Kernel_Name"])
                if role is None:
                    continue
                per.setdefault((role, _short(r["Kernel_Name"])), {}).setdefault(c, []).append(
                    float(r["Counter_Value"]) * 1024.0 * factors[c])
        if not per:
            continue
        md = [f"# HBM traffic per launch: {cfg.name}", "",
              "Commands (each counter in a run of its own; the copy calibration divides a "
              "1 GiB device copy's counter reading into the bytes it moved):", "", "```"]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            md.append(cmd_pmc.format(w=w, c=c))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            md.append(cmd_copy.format(c=c))
        md += ["```", "",
               f"Calibration: fetch factor {factors.get('FETCH_SIZE'):.4f}, write factor "
               f"{factors.get('WRITE_SIZE'):.4f} (bytes per counted byte).", "",
               "| kernel | launches | read MB/launch | written MB/launch |", "|---|---|---|---|"]
        best = {}
        for (role, kname), cs in sorted(per.items()):
            fr = cs.get("FETCH_SIZE", [0.0])
            wr = cs.get("WRITE_SIZE", [0.0])
            fb, wb = sum(fr) / len(fr), sum(wr) / len(wr)
            md.append(f"| `{kname}` | {len(fr)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
            if role not in best or fb + wb > best[role]["bytes_per_launch"]:
                best[role] = {"kernel": kname, "fetch_bytes_per_launch": fb,
                              "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
                              "source_hash": src_hash}
        for role, ent in best.items():
            traffic[f"{role}:{cfg.name}"] = ent
        md.append("")
        md.append(f"Kernel sources: `{src_hash}`.")
        with open(os.path.join(out_dir, f"hbm_traffic_T{cfg.T}.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
    _summarize_routing(src, out_dir, cmd_trace)
    with open(os.path.join(out_dir, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1)
        fh.write("\n")


def _summarize_routing(src, out_dir, cmd_trace):
    """Kernel trace of the routing-primitive run (moe_route and the moe_route_v2 cases)."""
    stats = _one(os.path.join(src, "trace_route", "*kernel_stats.csv"))
    if stats is None:
        return
    line = None
    log_path = os.path.join(src, "trace_route.log")
    if os.path.exists(log_path):
        for ln in open(log_path, errors="replace"):
            if ln.startswith("{") and '"routing_primitive"' in ln:
                line = json.loads(ln)["routing_primitive"]
    md = ["# Kernel trace: routing primitive", "",
          "Command (run from the repository root, after "
          "`cd /tmp && export TMPDIR=/tmp`):", "", "```", cmd_trace.format(w="route"), "```", "",
          "Per-kernel statistics (all calls of the run: moe_route on "
          "route_N8192_H7168_E256_K8_zipf1.1 with int8 and with NVFP4 rows, then the "
          "moe_route_v2 cases, each with its warmup and timed calls; `at::` kernels are the "
          "benchmark's own input setup):", "",
          "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in _read_csv(stats)[:14]:
        md.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                  f"{float(r['Percentage']):.1f} |")
    trace = _one(os.path.join(src, "trace_route", "*kernel_trace.csv"))
    if line and trace:
        # The cases run one after the other, each with warmup + steps calls: split the
        # library's kernels in dispatch order.
        kern = [r for r in _read_csv(trace) if "rmoe::route" in r["Kernel_Name"]]
        kern.sort(key=lambda r: int(r["Start_Timestamp"]))
        # one library call starts with the histogram launch, or is one fused small kernel
        starts = ("route_hist", "route_small", "route_permute_small", "quantize_route_small")
        calls = []
        for r in kern:
            if not calls or _short(r["Kernel_Name"]).startswith(starts):
                calls.append([])
            calls[-1].append(r)
        # dispatch order: moe_route (int8), moe_route (NVFP4), then the moe_route_v2 cases
        cases = [("moe_route", line)]
        if "nvfp4" in line:
            cases.append(("moe_route_nvfp4", line["nvfp4"]))
        cases += [(c, r) for c, r in line.get("options", {}).items()]
        names = sorted({_short(r["Kernel_Name"]) for r in kern})
        per_case = len(calls) // len(cases)
        md += ["", "Per case (kernel average µs over its calls; HIP-event time per call of "
               "the same run, which includes the gaps between launches):", "",
               "| case | " + " | ".join(f"`{n}`" for n in names) + " | event µs/call | HBM frac |",
               "|---|" + "---|" * (len(names) + 2)]
        for i, (case, r) in enumerate(cases):
            chunk = [k for c in calls[i * per_case:(i + 1) * per_case] for k in c]
            cells = []
            for n in names:
                d = [(int(c["End_Timestamp"]) - int(c["Start_Timestamp"])) / 1e3 for c in chunk
                     if _short(c["Kernel_Name"]) == n]
                cells.append(f"{sum(d) / len(d):.1f}" if d else "—")
            us = r["ms_per_call"] * 1e3 if case.startswith("moe_route") else r["us_per_call"]
            label = r["workload"]
            md.append(f"| {label} | " + " | ".join(cells) + f" | {us:.1f} | "
                      f"{100 * r['hbm_frac']:.1f}% |")
    with open(os.path.join(out_dir, "kernel_trace_routing.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads",
                    default="prefill,decode,mid,decode64,prefill4k,route,stream")
    ap.add_argument("--cpu-tokens", type=int, default=32,
                    help="tokens of the oracle's bounded CPU sample (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write profiles/ summaries from the rocprofv3 output under DIR (no GPU)")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize, os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer (one TP rank's work); the "
              "library has no multi-GPU path, so --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import routed_moe_layer_amd as rm
    from moe_inputs import DECODE_16, MID_1024, PREFILL_16K, ROUTE_8K, DECODE_64, PREFILL_4K

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    rm._lib()
    events = HipEvents()
    chosen = [w.strip() for w in args.workloads.split(",") if w.strip() and w.strip() != "stream"]
    if any(c != "route" for c in chosen):
        prepared, d13, d2 = build_weights(DECODE_16, torch, rm)
    cfgs = {"prefill": (PREFILL_16K, 1), "decode": (DECODE_16, 8), "mid": (MID_1024, 4),
            "decode64": (DECODE_64, 4), "prefill4k": (PREFILL_4K, 1)}
    results, keeps = {}, {}
    route_res = None
    if "route" in chosen:
        chosen = [c for c in chosen if c != "route"]
        log(f"timing {ROUTE_8K.name}: warmup {args.warmup}, steps {args.steps}")
        route_res = route_workload(ROUTE_8K, torch, rm, args.steps, args.warmup, events)
        log(f"  {route_res['routed_rows_per_s']:.3e} routed rows/s, {route_res['ms_per_call']:.3f} ms, "
            f"{100 * route_res['hbm_frac']:.1f}% of HBM peak")
        r4 = route_res["nvfp4"]
        log(f"  {r4['workload']}: {r4['ms_per_call']:.3f} ms, {100 * r4['hbm_frac']:.1f}% of HBM peak")
        route_res["topk"] = {}
        for T in (16384, 16):
            r = topk_workload(T, 896, 16, torch, rm, args.steps, args.warmup, events)
            route_res["topk"][f"T{T}"] = r
            log(f"  {r['workload']}: {r['us_per_call']:.1f} us/call, "
                f"{100 * r['hbm_frac']:.1f}% of HBM peak")
        route_res["options"] = {}
        for case in ROUTE_OPTION_CASES:
            r = route_options_workload(case, ROUTE_8K, torch, rm, args.steps, args.warmup,
                                       events)
            route_res["options"][case] = r
            log(f"  {r['workload']}: {r['us_per_call']:.1f} us/call, {r['routed_rows']} rows, "
                f"{100 * r['hbm_frac']:.1f}% of HBM peak")
    head = "prefill" if "prefill" in chosen else (chosen[0] if chosen else None)
    for name in chosen:
        cfg, rot = cfgs[name]
        # the headline batch times exactly --steps steps; the others at least 50 (cheap)
        steps = args.steps if name == head else max(args.steps, MIN_SUB_STEPS)
        log(f"timing {cfg.name}: warmup {args.warmup}, steps {steps}")
        results[name], keeps[name] = layer_workload(cfg, torch, rm, prepared, d13, d2,
                                                    steps, args.warmup, events, rot)
        r = results[name]
        log(f"  {r['tokens_per_s']:.1f} tokens/s, {r['ms_per_step']:.3f} ms/step "
            f"(median {r['gpu_ms_step_stats']['median']:.4f}, graph replay median "
            f"{r['graph_replay_ms_step_stats']['median']:.4f}), stages "
            + ", ".join(f"{k} {v:.4f}" for k, v in r["stage_ms_median"].items()))
    streamed = {}
    if "stream" in [w.strip() for w in args.workloads.split(",")]:
        for name, (chunk, slots) in STREAM_CASES.items():
            if name not in keeps:
                continue
            cfg = cfgs[name][0]
            for sealed in (False, True):
                tag = "sealed" if sealed else "streamed"
                log(f"timing {cfg.name} {tag} in chunks of {chunk} through {slots} slots")
                r = streamed_workload(cfg, keeps[name], torch, rm, prepared, chunk, slots,
                                      args.steps, args.warmup, events, sealed=sealed)
                r["batch_tokens_per_s"] = results[name]["tokens_per_s"]
                streamed[name + ("_sealed" if sealed else "")] = r
                extra = ""
                if "graph_replay_ms_step_stats" in r:
                    extra = (f", graph replay median "
                             f"{r['graph_replay_ms_step_stats']['median']:.3f} ms")
                log(f"  {r['tokens_per_s']:.1f} tokens/s, {r['ms_per_step']:.3f} ms/step "
                    f"(batch {results[name]['tokens_per_s']:.1f}){extra}")
    if not chosen:                      # routing primitive only
        print(json.dumps({"routing_primitive": route_res}), flush=True)
        return
    hr = results[head]
    hcfg = cfgs[head][0]
    fc1_ms = hr["fc1"]["ms"]
    if hcfg.T >= 4096:                 # the MFMA-bound band; smaller batches stream weights
        roof = {"bound": "mfma", "achieved": hr["fc1"]["flops"] / (fc1_ms * 1e-3) / 1e12,
                "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s"}
    elif "fused_fc1_fc2" in hr:
        fu = hr["fused_fc1_fc2"]
        roof = {"bound": "hbm", "achieved": fu["bytes"] / (fu["ms"] * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "hbm", "achieved": hr["fc1"]["bytes"] / (fc1_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = hr.get("fused_fc1_fc2", {}).get("kernel", "fc1_kernel")
    role = "fused_kernel" if "fused_fc1_fc2" in hr else "fc1_kernel"
    roof["traffic"] = traffic_from_profile(f"{role}:{hcfg.name}")
    cpu = None
    if args.cpu_tokens > 0:
        log(f"oracle CPU baseline on {args.cpu_tokens} tokens of {hcfg.name}")
        cpu = cpu_baseline(hcfg, keeps[head], torch, args.cpu_tokens)
    line = {
        "metric": METRIC, "value": hr["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": hr["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": hcfg.name, "T": hcfg.T, "H": hcfg.H, "I": hcfg.I, "E": hcfg.E,
                   "top_k": hcfg.k, "parallelism": "single GPU (one TP8 rank's share)"},
        "roofline": roof, "cpu_baseline": cpu, "workloads": results, "routing_primitive": route_res,
        "streamed": streamed or None,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
