"""Number formats: BF16, E2M1 (FP4), E4M3 (FP8) and E8M0 (CPU oracle; test only).

P1, PR description: a packed NVFP4 row holds E2M1 codes and E4M3 block scales.
P2, description: MXFP8 carries E4M3 data with E8M0 block scales.
The pages give no encoding details; the rules below are the standard formats
(OCP 8-bit floating point / OCP microscaling) with the readings stated.
"""

import numpy as np

# R2: the eight E2M1 magnitudes, index 0..7 (sign is bit 3 of the 4-bit code).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0


# ----------------------------------------------------------------------------- BF16
def bf16_to_f32(bits):
    """R1: a BF16 bit pattern is the upper half of an FP32 bit pattern."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """R1: FP32 -> BF16 by round-to-nearest-even on the bit pattern (finite inputs).

    Works unchanged for FP32 subnormals because their bit patterns are linear in
    the value.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------- E2M1
def e2m1_index(v):
    """R2: magnitude index of the nearest E2M1 grid point to v >= 0.

    Nearest in absolute distance; an exact tie goes to the even index
    (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
    5 -> 4); anything above 6 saturates to 6 (index 7).

    ``v`` may be float32 or float64.  The two distances are computed in
    float64 where they are exact (Sterbenz: the neighbours differ by at most
    a factor two), so the comparison decides ties exactly.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("e2m1_index expects finite magnitudes")
    lo = np.searchsorted(E2M1_GRID, v, side="right") - 1          # G[lo] <= v
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = v - E2M1_GRID[lo]
    d_hi = E2M1_GRID[hi] - v
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    idx = np.where(up, hi, lo)
    return idx.astype(np.uint8)


def e2m1_value(code):
    """Decode 4-bit E2M1 codes to float64 (sign bit 3, magnitude index bits 0..2)."""
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_GRID[code & 7]
    return np.where(code & 8, -mag, mag)


def pack_nibbles(codes):
    """Two 4-bit codes per byte along the last axis: element 2j low nibble, 2j+1 high."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & np.uint8(0x0F)
    out[..., 1::2] = packed >> np.uint8(4)
    return out


# ----------------------------------------------------------------------------- E4M3
def _e4m3_table():
    """All non-negative finite OCP E4M3FN values, indexed by code 0..126."""
    vals = np.empty(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_encode(y):
    """R3: OCP E4M3FN code of y >= 0: round-to-nearest-even of min(y, 448).

    Subnormals (multiples of 2^-9) are kept; the result is never NaN; an exact
    tie goes to the code with an even mantissa (even code).
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(y < 0) or np.any(np.isnan(y)):
        raise ValueError("e4m3_encode expects non-negative values")
    y = np.minimum(y, E4M3_MAX)
    lo = np.searchsorted(E4M3_VALUES, y, side="right") - 1
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = y - E4M3_VALUES[lo]
    d_hi = E4M3_VALUES[hi] - y
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    return np.where(up, hi, lo).astype(np.uint8)


def e4m3_decode(code):
    """Decode E4M3FN codes (sign bit 7) to float64; code 0x7F/0xFF (NaN) is rejected."""
    code = np.asarray(code, dtype=np.uint8)
    mag_code = code & np.uint8(0x7F)
    if np.any(mag_code == 0x7F):
        raise ValueError("E4M3 NaN code")
    mag = E4M3_VALUES[mag_code]
    return np.where(code & 0x80, -mag, mag)


# ----------------------------------------------------------------------------- E8M0
def e8m0_decode(code):
    """E8M0: code c (0..254) is the power of two 2^(c-127); 255 is NaN (rejected)."""
    code = np.asarray(code, dtype=np.int64)
    if np.any(code == 255):
        raise ValueError("E8M0 NaN code")
    return np.ldexp(1.0, code - 127)
