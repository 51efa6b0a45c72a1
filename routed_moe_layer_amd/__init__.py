"""Python binding of the routed-MoE HIP library (include/routed_moe.h).

Argument marshalling only: each function has the C entry point's name, takes torch
tensors (or raw integer device addresses) for the device buffers, passes their addresses
and the current HIP stream to the library and raises ``MoeError`` on a non-zero status.
Every step of the layer runs in the library's HIP kernels; there is no other
implementation behind these names.  If the shared library has not been built, every call
raises -- nothing falls back to another path.
"""

import ctypes
import os

__all__ = [
    "MoeError", "MoeDims", "library_path", "moe_status_string", "moe_workspace_size",
    "moe_prepared_weights_size", "moe_workspace_layout", "moe_route_workspace_size",
    "moe_quantize_nvfp4", "moe_prepare_weights", "moe_route", "moe_route_v2",
    "MoeRouteOptions", "moe_forward", "moe_forward_timed", "MOE_FORWARD_STAGES",
    "MoeRing", "make_ring", "moe_ring_layout", "moe_ring_init", "moe_ring_acquire",
    "moe_ring_publish", "moe_forward_streamed", "moe_sealed_workspace_size",
    "moe_forward_absorb", "moe_forward_seal", "moe_topk_softmax", "moe_forward_noalloc",
    "MOE_NOALLOC_SCRATCH_BYTES", "MOE_RING_ROUTE",
    "MOE_RING_LAYOUT",
    "MOE_RING_OK", "MOE_RING_CONSUMER_TIMEOUT", "MOE_RING_PRODUCER_TIMEOUT",
    "MOE_QUANT_NONE", "MOE_QUANT_INT8_ROW_DYNAMIC", "MOE_QUANT_NVFP4_G16", "MOE_MAX_TOKENS",
    "EXPORTED",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "lib", "libroutedmoe.so")

MOE_QUANT_NONE = 0
MOE_QUANT_INT8_ROW_DYNAMIC = 1
MOE_QUANT_NVFP4_G16 = 2
MOE_MAX_TOKENS = 16384
MOE_FORWARD_STAGES = 5
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/routed_moe.h declares.
EXPORTED = ("moe_status_string", "moe_workspace_size", "moe_prepared_weights_size",
            "moe_workspace_layout", "moe_route_workspace_size", "moe_quantize_nvfp4",
            "moe_prepare_weights", "moe_route", "moe_route_v2", "moe_forward",
            "moe_forward_timed", "moe_ring_layout", "moe_ring_init", "moe_ring_acquire",
            "moe_ring_publish", "moe_forward_streamed", "moe_sealed_workspace_size",
            "moe_forward_absorb", "moe_forward_seal", "moe_topk_softmax",
            "moe_forward_noalloc")

MOE_RING_ROUTE = 0
MOE_RING_LAYOUT = 1
MOE_RING_OK = 0
MOE_RING_CONSUMER_TIMEOUT = 1
MOE_RING_PRODUCER_TIMEOUT = 2


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {_status_text(status)} ({status})")


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]

    def __init__(self, hidden, inter, num_experts, top_k):
        super().__init__(hidden, inter, num_experts, top_k)


class MoeRouteOptions(ctypes.Structure):
    """moe_route_options_t: the routing primitive's options (defaults: all experts, gather
    index, cumsum histogram, no quant, dropless, no capacity, no row limit)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "expert_start", "expert_end", "row_idx_type", "expert_tokens_num_type", "quant_mode",
        "drop_pad_mode", "expert_capacity", "active_num")]

    def __init__(self, expert_start=0, expert_end=0, row_idx_type=0, expert_tokens_num_type=0,
                 quant_mode=-1, drop_pad_mode=0, expert_capacity=-1, active_num=-1):
        super().__init__(expert_start, expert_end, row_idx_type, expert_tokens_num_type,
                         quant_mode, drop_pad_mode, expert_capacity, active_num)


class MoeRing(ctypes.Structure):
    """moe_ring_t: a caller-owned ring of token slots (device memory at `base`)."""
    _fields_ = [("base", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
                ("num_slots", ctypes.c_int32), ("tokens_per_slot", ctypes.c_int32)]


class _RingLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "x", "expert_ids", "route_weights", "counters", "status", "total")]


class _Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "x_codes", "x_scales", "x_dec", "sorted_ids", "sorted_row_idx", "expanded_row_idx",
        "expert_counts", "expert_cumsum", "a_codes", "a_scales", "o_rows", "o_exp", "a_amax",
        "total")]


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"routed-MoE HIP library not built ({library_path} missing); run "
                "`python -m routed_moe_layer_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(library_path)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        st = ctypes.c_int
        sig = {
            "moe_status_string": (ctypes.c_char_p, [st]),
            "moe_workspace_size": (st, [MoeDims, I32, ctypes.c_int, ctypes.POINTER(SZ)]),
            "moe_prepared_weights_size": (st, [MoeDims, ctypes.POINTER(SZ)]),
            "moe_workspace_layout": (st, [MoeDims, I32, ctypes.POINTER(_Layout)]),
            "moe_route_workspace_size": (st, [I32, I32, I32, ctypes.POINTER(SZ)]),
            "moe_quantize_nvfp4": (st, [P, I64, I64, I32, P, P, P, P]),
            "moe_prepare_weights": (st, [MoeDims, P, P, P, P, P, SZ, P]),
            "moe_route": (st, [MoeDims, I32, P, P, ctypes.c_int, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_route_v2": (st, [I32, I32, I32, I32, P, P, P, P,
                                  ctypes.POINTER(MoeRouteOptions), P, P, P, P, P, P, SZ, P]),
            "moe_forward": (st, [MoeDims, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P, P]),
            "moe_forward_timed": (st, [MoeDims, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P, P,
                                       ctypes.POINTER(P)]),
            "moe_ring_layout": (st, [MoeDims, I32, I32, ctypes.POINTER(_RingLayout)]),
            "moe_topk_softmax": (st, [I32, I32, I32, P, P, P, P]),
            "moe_ring_init": (st, [MoeDims, ctypes.POINTER(MoeRing), P]),
            "moe_ring_acquire": (st, [MoeDims, ctypes.POINTER(MoeRing), I32, ctypes.c_int,
                                      ctypes.c_uint32, P]),
            "moe_ring_publish": (st, [MoeDims, ctypes.POINTER(MoeRing), I32, ctypes.c_int, P]),
            "moe_forward_streamed": (st, [MoeDims, ctypes.POINTER(MoeRing), I32, I32, I32, P, P,
                                          P, P, P, P, P, ctypes.c_uint32, P, SZ, P, P]),
            "moe_sealed_workspace_size": (st, [MoeDims, I32, ctypes.POINTER(SZ)]),
            "moe_forward_absorb": (st, [MoeDims, ctypes.POINTER(MoeRing), I32, I32, I32, P,
                                        ctypes.c_uint32, P, SZ, P]),
            "moe_forward_seal": (st, [MoeDims, I32, P, P, P, P, P, P, P, SZ, P, P]),
            "moe_forward_noalloc": (st, [MoeDims, I32, P, P, P, P, P, P, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib_handle = lib
    return _lib_handle


def _status_text(status):
    try:
        return _lib().moe_status_string(status).decode()
    except Exception:  # the library itself failed to load
        return "status"


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t):
    """Device address of a tensor (or an int address; None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def moe_status_string(status):
    return _lib().moe_status_string(status).decode()


def moe_workspace_size(dims, max_tokens, quant=MOE_QUANT_NVFP4_G16):
    n = ctypes.c_size_t()
    _check("moe_workspace_size",
           _lib().moe_workspace_size(dims, max_tokens, quant, ctypes.byref(n)))
    return n.value


def moe_prepared_weights_size(dims):
    n = ctypes.c_size_t()
    _check("moe_prepared_weights_size", _lib().moe_prepared_weights_size(dims, ctypes.byref(n)))
    return n.value


def moe_workspace_layout(dims, T):
    lay = _Layout()
    _check("moe_workspace_layout", _lib().moe_workspace_layout(dims, T, ctypes.byref(lay)))
    return {name: getattr(lay, name) for name, _ in _Layout._fields_}


def moe_route_workspace_size(num_rows, top_k, num_experts):
    n = ctypes.c_size_t()
    _check("moe_route_workspace_size",
           _lib().moe_route_workspace_size(num_rows, top_k, num_experts, ctypes.byref(n)))
    return n.value


def moe_quantize_nvfp4(src, groups, rows_per_group, K, q, codes, scales, stream=None):
    _check("moe_quantize_nvfp4", _lib().moe_quantize_nvfp4(
        _ptr(src), groups, rows_per_group, K, _ptr(q), _ptr(codes), _ptr(scales),
        _stream(stream)))


def moe_prepare_weights(dims, w13, w13_sf, w2, w2_sf, prepared, prepared_bytes=None, stream=None):
    nb = _nbytes(prepared) if prepared_bytes is None else prepared_bytes
    _check("moe_prepare_weights", _lib().moe_prepare_weights(
        dims, _ptr(w13), _ptr(w13_sf), _ptr(w2), _ptr(w2_sf), _ptr(prepared), nb,
        _stream(stream)))


def moe_route(dims, T, x, expert_ids, quant, qx, sorted_expert_ids, sorted_row_idx,
              expanded_row_idx, expert_cumsum, expanded_x, expanded_sf_or_scale, workspace,
              workspace_bytes=None, stream=None):
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check("moe_route", _lib().moe_route(
        dims, T, _ptr(x), _ptr(expert_ids), quant, _ptr(qx), _ptr(sorted_expert_ids),
        _ptr(sorted_row_idx), _ptr(expanded_row_idx), _ptr(expert_cumsum), _ptr(expanded_x),
        _ptr(expanded_sf_or_scale), _ptr(workspace), nb, _stream(stream)))


def moe_route_v2(num_rows, hidden, num_experts, top_k, x, expert_idx, options, expanded_x,
                 expanded_row_idx, expert_tokens=None, expanded_scale=None,
                 available_idx_num=None, scale=None, offset=None, workspace=None,
                 workspace_bytes=None, stream=None):
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check("moe_route_v2", _lib().moe_route_v2(
        num_rows, hidden, num_experts, top_k, _ptr(x), _ptr(expert_idx), _ptr(scale),
        _ptr(offset), ctypes.byref(options), _ptr(expanded_x), _ptr(expanded_row_idx),
        _ptr(expert_tokens), _ptr(expanded_scale), _ptr(available_idx_num), _ptr(workspace),
        nb, _stream(stream)))


def moe_forward(dims, T, x, expert_ids, route_weights, prepared, qx, alpha1, qa, alpha2,
                situ_beta, situ_linear_beta, workspace, out, workspace_bytes=None, stream=None):
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check("moe_forward", _lib().moe_forward(
        dims, T, _ptr(x), _ptr(expert_ids), _ptr(route_weights), _ptr(prepared), _ptr(qx),
        _ptr(alpha1), _ptr(qa), _ptr(alpha2), _ptr(situ_beta), _ptr(situ_linear_beta),
        _ptr(workspace), nb, _ptr(out), _stream(stream)))


def moe_forward_noalloc(dims, T, x, expert_ids, route_weights, prepared, qx, alpha1, qa,
                        alpha2, situ_beta, situ_linear_beta, out, stream=None):
    _check("moe_forward_noalloc", _lib().moe_forward_noalloc(
        dims, T, _ptr(x), _ptr(expert_ids), _ptr(route_weights), _ptr(prepared), _ptr(qx),
        _ptr(alpha1), _ptr(qa), _ptr(alpha2), _ptr(situ_beta), _ptr(situ_linear_beta), _ptr(out),
        _stream(stream)))


def moe_forward_timed(dims, T, x, expert_ids, route_weights, prepared, qx, alpha1, qa, alpha2,
                      situ_beta, situ_linear_beta, workspace, out, events,
                      workspace_bytes=None, stream=None):
    """``events``: a sequence of MOE_FORWARD_STAGES + 1 raw hipEvent_t handles (ints)."""
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    ev = (ctypes.c_void_p * len(events))(*events)
    _check("moe_forward_timed", _lib().moe_forward_timed(
        dims, T, _ptr(x), _ptr(expert_ids), _ptr(route_weights), _ptr(prepared), _ptr(qx),
        _ptr(alpha1), _ptr(qa), _ptr(alpha2), _ptr(situ_beta), _ptr(situ_linear_beta),
        _ptr(workspace), nb, _ptr(out), _stream(stream), ev))


def moe_ring_layout(dims, num_slots, tokens_per_slot):
    lay = _RingLayout()
    _check("moe_ring_layout", _lib().moe_ring_layout(dims, num_slots, tokens_per_slot,
                                                     ctypes.byref(lay)))
    return {n: getattr(lay, n) for n, _ in _RingLayout._fields_}


def make_ring(buffer, num_slots, tokens_per_slot):
    """A MoeRing over a device byte buffer (a tensor or an int address with its size)."""
    if isinstance(buffer, tuple):
        base, nbytes = buffer
    else:
        base, nbytes = buffer.data_ptr(), _nbytes(buffer)
    return MoeRing(base, nbytes, num_slots, tokens_per_slot)


def moe_ring_init(dims, ring, stream=None):
    _check("moe_ring_init", _lib().moe_ring_init(dims, ctypes.byref(ring), _stream(stream)))


def moe_ring_acquire(dims, ring, slot, role, timeout_us=0, stream=None):
    _check("moe_ring_acquire", _lib().moe_ring_acquire(dims, ctypes.byref(ring), slot, role,
                                                       timeout_us, _stream(stream)))


def moe_ring_publish(dims, ring, slot, role, stream=None):
    _check("moe_ring_publish", _lib().moe_ring_publish(dims, ctypes.byref(ring), slot, role,
                                                       _stream(stream)))


def moe_forward_streamed(dims, ring, total_tokens, first_chunk, num_chunks, prepared, qx,
                         alpha1, qa, alpha2, situ_beta, situ_linear_beta, workspace, out,
                         timeout_us=0, workspace_bytes=None, stream=None):
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check("moe_forward_streamed", _lib().moe_forward_streamed(
        dims, ctypes.byref(ring), total_tokens, first_chunk, num_chunks, _ptr(prepared), _ptr(qx),
        _ptr(alpha1), _ptr(qa), _ptr(alpha2), _ptr(situ_beta), _ptr(situ_linear_beta),
        timeout_us, _ptr(workspace), nb, _ptr(out), _stream(stream)))


def moe_sealed_workspace_size(dims, total_tokens):
    n = ctypes.c_size_t()
    _check("moe_sealed_workspace_size",
           _lib().moe_sealed_workspace_size(dims, total_tokens, ctypes.byref(n)))
    return n.value


def moe_forward_absorb(dims, ring, total_tokens, first_chunk, num_chunks, qx, workspace,
                       timeout_us=0, workspace_bytes=None, stream=None):
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check("moe_forward_absorb", _lib().moe_forward_absorb(
        dims, ctypes.byref(ring), total_tokens, first_chunk, num_chunks, _ptr(qx), timeout_us,
        _ptr(workspace), nb, _stream(stream)))


def moe_forward_seal(dims, total_tokens, prepared, alpha1, qa, alpha2, situ_beta,
                     situ_linear_beta, workspace, out, workspace_bytes=None, stream=None):
    nb = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    _check("moe_forward_seal", _lib().moe_forward_seal(
        dims, total_tokens, _ptr(prepared), _ptr(alpha1), _ptr(qa), _ptr(alpha2),
        _ptr(situ_beta), _ptr(situ_linear_beta), _ptr(workspace), nb, _ptr(out),
        _stream(stream)))


def moe_topk_softmax(T, num_experts, top_k, logits, expert_ids, route_weights, stream=None):
    _check("moe_topk_softmax", _lib().moe_topk_softmax(
        T, num_experts, top_k, _ptr(logits), _ptr(expert_ids), _ptr(route_weights),
        _stream(stream)))
