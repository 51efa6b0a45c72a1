"""Group-16 NVFP4 block quantization, its inverse and nibble packing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Cake SiTU backend", intro: BF16 input is quantized to group-16 NVFP4, and the
intermediate is requantized to NVFP4; section "Prepared weights and scales": one fp32
activation encoding scale qX = 1/dX, per-expert qA = 1/dA, E4M3 block scales (one per
16 values: FC1 scales are [.., 3584/16], FC2 scales [.., 384/16]).  "Nvfp4 Tensor":
the global scale multiplies after block dequantization.

The pages do not give the block-scale arithmetic.  The reading taken (the plainest one that
fits those facts; every step in IEEE fp32, left to right):

    amax  = max |v_i|                      over the 16 values of the block
    s32   = fp32( fp32(amax * q) / 6 )     (6 = largest E2M1 magnitude)
    s     = E4M3( min(s32, 448) )          round to nearest even, saturating
    enc   = 0 if s == 0 else fp32(q / s)   one encode factor per block
    code  = E2M1( fp32(v_i * enc) )        round to nearest even, saturating at 6

The decoded block is code * s (a float64 here), and the real value is that times 1/q.
"""

import numpy as np

from .codecs import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode

GROUP = 16


def quantize_nvfp4(v, q):
    """Quantize the last axis of ``v`` in groups of 16.

    v : float32 array [..., K], K % 16 == 0 (BF16 inputs are first widened exactly).
    q : float32 global encoding scale; a scalar or an array broadcastable to v.shape[:-1].
    Returns (codes uint8 [..., K], one E2M1 code per element, unpacked;
             scales uint8 [..., K/16], E4M3 bytes).
    """
    v = np.asarray(v, dtype=np.float32)
    K = v.shape[-1]
    if K % GROUP:
        raise ValueError("last axis must be a multiple of 16")
    q = np.asarray(q, dtype=np.float32)
    blocks = v.reshape(v.shape[:-1] + (K // GROUP, GROUP))
    qb = np.broadcast_to(q[..., None], blocks.shape[:-1]).astype(np.float32)
    amax = np.max(np.abs(blocks), axis=-1)                                 # exact in fp32
    s32 = (amax * qb).astype(np.float32) / np.float32(6.0)                # fp32 * then fp32 /
    s32 = s32.astype(np.float32)
    scales = e4m3_encode(s32.astype(np.float64))                           # clamp + RNE
    s_val = e4m3_decode(scales).astype(np.float32)                         # exact in fp32
    with np.errstate(divide="ignore", invalid="ignore"):
        enc = np.where(s_val == 0, np.float32(0.0), qb / s_val).astype(np.float32)
    y = (blocks * enc[..., None]).astype(np.float32)                       # fp32 product
    codes = e2m1_encode(y.astype(np.float64))
    return codes.reshape(v.shape), scales


def dequantize_nvfp4(codes, scales):
    """float64 code * scale for unpacked codes [..., K] and E4M3 scales [..., K/16].

    Every result is an integer multiple of 2^-10 (E2M1 values are multiples of 1/2,
    E4M3 values multiples of 2^-9) and at most 6 * 448 in magnitude.
    """
    c = e2m1_decode(codes)
    s = e4m3_decode(scales)
    K = c.shape[-1]
    blocks = c.reshape(c.shape[:-1] + (K // GROUP, GROUP)) * s[..., None]
    return blocks.reshape(c.shape)


def pack_nibbles(codes):
    """Two codes per byte along the last axis: element 2b in the low nibble of byte b
    (a reading; "Nvfp4 Tensor" only says eight FP4 values share a 32-bit word)."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
