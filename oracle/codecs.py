"""Element codecs: FP4 E2M1, FP8 E4M3 (the "fn" flavour) and BF16 rounding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the formats but never spell them out: "Cake SiTU backend", intro and
section "Prepared weights and scales", say NVFP4 (FP4 values in groups of 16) with
float8_e4m3fn block scales; "Nvfp4 Tensor" (struct NVFP4Tensor) calls the 4-bit payload
E2M1 and the scales FP8 E4M3.  The definitions below are the standard ones for those
names (readings of those names):

  * E2M1: bit 3 = sign, bits 2..0 = magnitude index into {0, .5, 1, 1.5, 2, 3, 4, 6};
    no Inf/NaN.
  * E4M3 "fn": bit 7 = sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent
    field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; no Inf; largest finite 448.
  * Rounding to either grid is round-to-nearest, ties to the even code, saturating at
    the largest finite magnitude.

Everything is written as "nearest point of an enumerated grid", the definition itself,
not as bit tricks.
"""

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e4m3_magnitude_table():
    """Value of every non-negative E4M3 byte 0..126 (127 is NaN), by the format definition."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        exp_field, mant = code >> 3, code & 7
        if exp_field == 0:
            vals[code] = mant * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            vals[code] = (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return vals


E4M3_MAGNITUDES = _e4m3_magnitude_table()
E4M3_MAX = 448.0


def e2m1_decode(codes):
    """float64 value of each 4-bit code (low nibble of the input integers)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def _nearest_even(abs_vals, grid):
    """Index of the grid point nearest to each value; on a tie the even index wins.

    ``grid`` is sorted ascending and its indices are the codes, so "even index" is
    "even code" (the mantissa LSB is the code LSB).  Values above the top grid point go
    to the top point (saturation).
    """
    a = np.asarray(abs_vals, dtype=np.float64)
    hi = np.searchsorted(grid, a, side="left")            # first grid >= a
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = np.abs(a - grid[lo])
    d_hi = np.abs(grid[hi] - a)
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie & (lo != hi), np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= grid[-1], len(grid) - 1, pick)   # saturate (distances lose meaning far out)
    return pick.astype(np.int64)


def e2m1_encode(y):
    """4-bit E2M1 code of float values ``y`` (round to nearest, ties to even, saturate at 6).

    The sign bit is the sign bit of ``y``: a negative value that rounds to zero, or -0.0,
    gives code 0x8 (a reading: signed zeros are kept).
    """
    y = np.asarray(y, dtype=np.float64)
    mag_code = _nearest_even(np.abs(y), E2M1_MAGNITUDES)
    sign = np.signbit(y).astype(np.int64) << 3
    return (mag_code | sign).astype(np.uint8)


def e4m3_decode(codes):
    """float64 value of E4M3 bytes (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    mag_idx = c & 0x7F
    mag = np.where(mag_idx == 127, np.nan, E4M3_MAGNITUDES[np.minimum(mag_idx, 126)])
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(s):
    """E4M3 byte of non-negative float values: clamp to 448 first, then round to nearest,
    ties to even (a reading: saturating conversion, never NaN)."""
    s = np.asarray(s, dtype=np.float64)
    if np.any(s < 0) or np.any(np.isnan(s)):
        raise ValueError("e4m3_encode is only used on non-negative block scales")
    return _nearest_even(np.minimum(s, E4M3_MAX), E4M3_MAGNITUDES).astype(np.uint8)


def bf16_bits_to_f32(bits):
    """float32 value of BF16 bit patterns (exact: BF16 is the top half of FP32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f64_to_bf16_bits(v):
    """Round float64 values once, to nearest-even, onto the BF16 grid; return the bits.

    BF16 keeps 8 significant bits: write v = m * 2^e with 0.5 <= |m| < 1, round m*256 to
    an integer (half-even), rebuild.  Below 2^-126 the grid spacing is fixed at 2^-133.
    Finite inputs only; the layer never produces Inf/NaN on finite inputs.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value reached the BF16 rounding")
    m, e = np.frexp(v)
    normal = np.abs(v) >= 2.0 ** -126
    r_norm = np.ldexp(np.rint(m * 256.0), e - 8)
    r_sub = np.rint(v * 2.0 ** 133) * 2.0 ** -133
    r = np.where(normal, r_norm, r_sub)
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise ValueError("BF16 overflow")
    f32 = r.astype(np.float32)                     # exact: r is on the BF16 grid
    return (f32.view(np.uint32) >> 16).astype(np.uint16)
