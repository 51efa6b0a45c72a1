"""Device-side helpers of the GPU tests: upload inputs, call the library through its C ABI
(routed_moe_layer_amd), and read back outputs and the workspace intermediates."""

import numpy as np
import torch

import routed_moe_layer_amd as rm


def dev(a):
    """numpy -> device tensor with the same bytes (uint16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


GUARD = 1 << 16
GUARD_BYTE = 0xA5


def empty_bytes(n, fill=None):
    """A device byte buffer of n bytes followed by a guard region (see check_guard)."""
    n = max(int(n), 1)
    full = torch.empty(n + GUARD, dtype=torch.uint8, device="cuda")
    full[n:].fill_(GUARD_BYTE)
    t = full[:n]
    if fill is not None:
        t.fill_(fill)
    t._guard_full = full
    return t


def check_guard(t):
    """Assert that nothing was written past the end of a buffer from empty_bytes."""
    full = t._guard_full
    tail = full[t.numel():]
    assert bool((tail == GUARD_BYTE).all()), "write past the end of a library buffer"


def dims_of(cfg):
    return rm.MoeDims(cfg.H, cfg.I, cfg.E, cfg.k)


def quantize_on_gpu(bits_dev, groups, rows_per_group, K, q_dev):
    """moe_quantize_nvfp4 of a device BF16 tensor; returns (codes, scales) device tensors."""
    n = groups * rows_per_group
    codes = torch.empty((n, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, K // 16), dtype=torch.uint8, device="cuda")
    rm.moe_quantize_nvfp4(bits_dev, groups, rows_per_group, K, q_dev, codes, scales)
    return codes, scales


def prepare(cfg, w13, w13_sf, w2, w2_sf):
    """moe_prepare_weights from canonical device (or numpy) weight storage."""
    d = dims_of(cfg)
    prepared = empty_bytes(rm.moe_prepared_weights_size(d))
    args = [t if isinstance(t, torch.Tensor) else dev(t) for t in (w13, w13_sf, w2, w2_sf)]
    rm.moe_prepare_weights(d, *args, prepared)
    torch.cuda.synchronize()
    check_guard(prepared)
    return prepared


def _fc2_rows(vals, exps):
    """FC2 output rows [R, H] as float64 from the stored f16 values and the exponent s of
    each row (value = stored * 2^-s).  Rows of dropped ids are never written, so they may
    hold anything; no check reads them."""
    with np.errstate(invalid="ignore", over="ignore"):
        return vals.astype(np.float64) * np.ldexp(1.0, -exps.astype(np.int64))[:, None]


class DeviceLayer:
    """The inputs of one moe_forward call resident on the GPU."""

    def __init__(self, p, prepared, T=None):
        cfg = p["cfg"]
        self.cfg = cfg
        self.dims = dims_of(cfg)
        self.T = cfg.T if T is None else T
        self.x = dev(p["x"][: self.T])
        self.ids = dev(p["ids"][: self.T].astype(np.int32))
        self.rw = dev(p["rw"][: self.T])
        self.prepared = prepared
        self.qx = dev(np.array([p["qX"]], np.float32))
        self.alpha1 = dev(p["alpha1"])
        self.qa = dev(p["qA"])
        self.alpha2 = dev(p["alpha2"])
        self.beta = None if p["beta"] is None else dev(p["beta"])
        self.lam = None if p["lam"] is None else dev(p["lam"])
        self.ws_bytes = rm.moe_workspace_size(self.dims, self.T)
        self.workspace = empty_bytes(self.ws_bytes)
        self.out = torch.empty((self.T, cfg.H), dtype=torch.int16, device="cuda")

    def forward(self, workspace=None, out=None, stream=None):
        ws = self.workspace if workspace is None else workspace
        o = self.out if out is None else out
        rm.moe_forward(self.dims, self.T, self.x, self.ids, self.rw, self.prepared, self.qx,
                       self.alpha1, self.qa, self.alpha2, self.beta, self.lam, ws, o,
                       workspace_bytes=ws.numel(), stream=stream)
        return o

    def check_guards(self):
        torch.cuda.synchronize()
        check_guard(self.workspace)

    def intermediates(self, workspace=None):
        ws = self.workspace if workspace is None else workspace
        lay = rm.moe_workspace_layout(self.dims, self.T)
        cfg, T = self.cfg, self.T
        R = T * cfg.k
        raw = ws.cpu().numpy()

        def take(key, count, dtype, shape):
            b = np.dtype(dtype).itemsize * count
            return raw[lay[key]: lay[key] + b].view(dtype).reshape(shape)

        return {
            "x_codes": take("x_codes", T * cfg.H // 2, np.uint8, (T, cfg.H // 2)),
            "x_scales": take("x_scales", T * cfg.H // 16, np.uint8, (T, cfg.H // 16)),
            "x_dec": take("x_dec", T * cfg.H, np.float16, (T, cfg.H)),
            "sorted_ids": take("sorted_ids", R, np.int32, (R,)),
            "sorted_row_idx": take("sorted_row_idx", R, np.int32, (R,)),
            "expanded_row_idx": take("expanded_row_idx", R, np.int32, (R,)),
            "counts": take("expert_counts", cfg.E, np.int32, (cfg.E,)),
            "cumsum": take("expert_cumsum", cfg.E, np.int32, (cfg.E,)),
            "a_codes": take("a_codes", R * cfg.I // 2, np.uint8, (R, cfg.I // 2)),
            "a_scales": take("a_scales", R * cfg.I // 16, np.uint8, (R, cfg.I // 16)),
            "o_rows": _fc2_rows(take("o_rows", R * cfg.H, np.float16, (R, cfg.H)),
                                take("o_exp", R, np.int8, (R,))),
            "o_exp": take("o_exp", R, np.int8, (R,)).copy(),
            "a_amax": take("a_amax", cfg.E, np.float32, (cfg.E,)),
        }
