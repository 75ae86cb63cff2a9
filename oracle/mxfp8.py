"""MXFP8 dispatch quantization (CPU oracle; test only).

P2, description and "Changes": BF16 tokens are quantized to E4M3 data with
E8M0 block scales ("compact scale-inverse") before dispatch; received data and
block scales share one caller-supplied buffer, data region first, then the
scale region.  Only E4M3 data is supported and pre-quantized input is refused
(P2, review comments).
"""

import numpy as np

from . import formats as F

BLOCK = 32


def scale_exponent(amax):
    """R11: E8M0 exponent of a 32-element block with max |x| = amax.

    amax = 0 gives e = 0.  Otherwise e is the least integer with
    amax <= 448 * 2^e (no element clips), clamped to [-127, 127].
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)                      # amax in [2^(E-1), 2^E)
    e = (E - 11).astype(np.int64)              # 448 * 2^(E-11) = 0.875 * 2^(E-2) < amax
    for _ in range(4):
        e = np.where(amax > F.E4M3_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.where(amax == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def pack_rows(x_bits):
    """BF16 rows [N, H] -> (data uint8 [N, H], scales uint8 [N, H/32]).

    data = sign(x) | E4M3(|x| / 2^e) with E4M3 round-to-nearest-even (R3);
    scale byte = e + 127.  |x| / 2^e is exact in float64.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n, h = x_bits.shape
    if h % BLOCK:
        raise ValueError("hidden must be a multiple of 32")
    x = F.bf16_to_f32(x_bits).astype(np.float64)
    ax = np.abs(x)
    amax = ax.reshape(n, h // BLOCK, BLOCK).max(axis=2)
    e = scale_exponent(amax)
    y = ax / np.repeat(np.ldexp(1.0, e), BLOCK, axis=1)
    mag = F.e4m3_encode(y)
    sign = ((x_bits >> np.uint16(15)) & np.uint16(1)).astype(np.uint8)
    data = (sign << np.uint8(7)) | mag
    scales = (e + 127).astype(np.uint8)
    return data, scales


def decode(data, scales):
    """Exact values of MXFP8 rows (float64 [N, H])."""
    n, h = data.shape
    return F.e4m3_decode(data) * np.repeat(F.e8m0_decode(scales), BLOCK, axis=1)


def grouped_receive(data, scales, src_row):
    """R13 analogue for MXFP8: grouped row g copies token src_row[g]; -1 rows are zero bytes."""
    src_row = np.asarray(src_row, dtype=np.int64)
    g_data = np.zeros((src_row.shape[0], data.shape[1]), dtype=np.uint8)
    g_scales = np.zeros((src_row.shape[0], scales.shape[1]), dtype=np.uint8)
    ok = src_row >= 0
    g_data[ok] = data[src_row[ok]]
    g_scales[ok] = scales[src_row[ok]]
    return g_data, g_scales
