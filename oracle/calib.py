"""Global-scale calibration: d = amax / (6 * 448), q = 1 / d.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Cake SiTU backend", section "Prepared weights and scales": qX = 1/dX and qA = 1/dA;
FC1 dequantization uses dX*dW13 and FC2 uses dA*dW2, both float32 [E]; the caller does
this scale arithmetic during model preparation.  The tensor-to-scale rule amax/(6*448)
(6 = largest E2M1 magnitude, 448 = largest E4M3 scale) is the calibration the workload
description states; it puts the largest element of the tensor at code 6 under a
block scale of 448.

Reading taken: a tensor whose amax is 0 gets d = q = 1 (any positive value encodes zeros
as zeros; 1/0 would make the block-scale arithmetic produce NaN).
"""

import numpy as np

from .codecs import bf16_bits_to_f32

FP4_TIMES_E4M3_MAX = np.float32(6.0 * 448.0)   # 2688


def global_scale_from_amax(amax):
    """(d, q) float32 for an fp32 amax (scalar or array): d = amax/2688, q = 1/d."""
    a = np.asarray(amax, dtype=np.float32)
    d = np.where(a > 0, a / FP4_TIMES_E4M3_MAX, np.float32(1.0)).astype(np.float32)
    q = (np.float32(1.0) / d).astype(np.float32)
    return d, q


def calibrate_tokens(x_bits):
    """(dX, qX) float32 of BF16 token bits: one tensor-global scale."""
    return global_scale_from_amax(np.max(np.abs(bf16_bits_to_f32(x_bits))))


def calibrate_weights(w_bits):
    """(dW [E], qW [E]) float32 of stacked BF16 expert weights [E, N, K]: per-expert amax."""
    a = np.array([np.max(np.abs(bf16_bits_to_f32(w_bits[e]))) for e in range(w_bits.shape[0])],
                 np.float32)
    return global_scale_from_amax(a)


def calibrate_layer(x_bits, w13_bits, w2_bits):
    """Scales of the inputs that are known before the layer runs.

    x_bits   : BF16 bits [T, H] of the tokens (tensor-global dX).
    w13_bits : BF16 bits [E, 2I, H] (per-expert dW13), w2_bits: BF16 bits [E, H, I].
    Returns a dict of float32 arrays: dX, qX (scalars), dW13, qW13, dW2, qW2 ([E]).
    """
    out = {}
    out["dX"], out["qX"] = calibrate_tokens(x_bits)
    out["dW13"], out["qW13"] = calibrate_weights(w13_bits)
    out["dW2"], out["qW2"] = calibrate_weights(w2_bits)
    return out


def quantize_expert_stack(w_bits, q):
    """NVFP4-quantize stacked BF16 expert weights [E, N, K] along K with per-expert q[E].

    Returns canonical storage: packed codes uint8 [E, N, K/2] (element 2b in the low
    nibble of byte b) and E4M3 block scales uint8 [E, N, K/16].
    """
    from .nvfp4 import quantize_nvfp4, pack_nibbles
    w_bits = np.asarray(w_bits, np.uint16)
    E, N, K = w_bits.shape
    packed = np.empty((E, N, K // 2), np.uint8)
    scales = np.empty((E, N, K // 16), np.uint8)
    for e in range(E):
        c, s = quantize_nvfp4(bf16_bits_to_f32(w_bits[e]), np.asarray(q, np.float32)[e])
        packed[e], scales[e] = pack_nibbles(c), s
    return packed, scales
