"""NVFP4 packed token rows: pack (RNE and stochastic), unpack (CPU oracle; test only).

P1, PR description and first commit message: the sender turns each token into
one NVFP4 row made of E2M1 codes, E4M3 block scales (one per 16 elements) and
a power-of-two FP32 per-token scale; rows that are not consumed directly are
decoded back to BF16; the combine backward quantizes with stochastic rounding.

Row layout (R7): ``[H/2 code bytes | H/16 scale bytes | 4-byte FP32 t]``,
unpadded, stride 9H/16 + 4 bytes, H a multiple of 64.  Decoding multiplies:
x_hat = e2m1 * s_b * t.
"""

import numpy as np

from . import formats as F
from .philox import sr_word

TOKEN_SCALE_BOUND = 6.0 * 448.0     # 2688: largest E2M1 magnitude times largest E4M3 scale


def packed_row_bytes(hidden):
    return 9 * hidden // 16 + 4


def token_scale_exponent(amax):
    """R4: power-of-two token scale t = 2^e for a row with max |x| = amax.

    amax = 0 gives e = 0 (t = 1).  Otherwise e is the least integer with
    amax <= 2688 * 2^e, i.e. the smallest power of two that keeps every block
    scale within E4M3's 448.  Found by walking up from a lower bound with
    exact float64 comparisons.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)                        # amax = m * 2^E, m in [0.5, 1)
    e = (E - 13).astype(np.int64)                # 2688 * 2^(E-13) < 2^(E-1) <= amax
    for _ in range(4):
        e = np.where(amax > TOKEN_SCALE_BOUND * np.ldexp(1.0, e), e + 1, e)
    return np.where(amax == 0, 0, e).astype(np.int64)


def _row_scales(ax32):
    """Token exponents e [N] and block scale codes [N, H/16] for |x| as float32 [N, H].

    R5: s_b = E4M3 round-to-nearest-even of the exact value a_b / (6 * t), with
    a_b = max |x| over the 16-element block.  The float64 quotient is exact when
    3 divides a_b's significand; otherwise the exact quotient is a periodic binary
    fraction (period 2) that is never an E4M3 tie, so the float64 value rounds to
    E4M3 exactly as the exact one does.
    """
    n, h = ax32.shape
    amax = ax32.max(axis=1).astype(np.float64)
    e = token_scale_exponent(amax)
    a_b = ax32.reshape(n, h // 16, 16).max(axis=2).astype(np.float64)
    y = a_b / (6.0 * np.ldexp(1.0, e)[:, None])
    return e, F.e4m3_encode(y)


def pack_rows(x_bits, sr_seed=None, sr_counter_base=0, sr_mode="element", sr_rule="threshold"):
    """R4-R9: BF16 rows [N, H] (uint16 bit patterns) -> packed rows uint8 [N, 9H/16 + 4].

    Block scale (R5): s_b = E4M3(a_b / (6 * t)), a_b = max |x| over the
    16-element block, rounded once from the exact value.

    Codes, round-to-nearest (R6): s_b = 0 gives magnitude index 0.  Otherwise
    the index is the E2M1 rounding (R2) of the exact quotient |x| / (s_b * t).
    The quotient of an 8-bit BF16 significand by a 4-bit E4M3 significand is
    either exactly a tie or at relative distance >= 2^-12 from every tie, so
    the float64 quotient used here decides exactly as the exact one does.

    Codes, stochastic (R8), when ``sr_seed`` is given: v = fl32(|x| / (s_b*t))
    (the float64 quotient rounded once to float32 is exactly fl32 of the exact
    quotient: the quotient's binary expansion is finite or periodic with
    period <= 12 and never lands on a float32 midpoint).  v >= 6 gives index 7.
    Otherwise g_lo <= v < g_hi are neighbouring grid points,
    frac = (v - g_lo) / (g_hi - g_lo) (exact), w = the Philox word for stream
    position n = counter_base + row*H + col, and the code rounds up
    * ``sr_rule="threshold"`` (R8): iff r * 2^-24 < frac, r = the top 24 bits of w;
    * ``sr_rule="carry"`` (R8b): iff floor(frac * 2^32) + w >= 2^32, i.e. the
      32 random bits are added below the kept precision and the sum truncated.

    The code's sign bit is the sign bit of x, always (also for -0 and for
    values that round to zero).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n, h = x_bits.shape
    if h % 64:
        raise ValueError("hidden must be a multiple of 64")
    x = F.bf16_to_f32(x_bits)
    ax = np.abs(x)
    sign = ((x_bits >> np.uint16(15)) & np.uint16(1)).astype(np.uint8)
    e, s_code = _row_scales(ax)
    t = np.ldexp(1.0, e)                                                  # float64, exact
    s_val = F.e4m3_decode(s_code)                                         # [N, H/16]
    denom = np.repeat(s_val, 16, axis=1) * t[:, None]                     # exact in float64
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(denom > 0, ax.astype(np.float64) / np.where(denom > 0, denom, 1.0), 0.0)
    if sr_seed is None:
        idx = F.e2m1_index(q)
    else:
        v = q.astype(np.float32).astype(np.float64)
        rows = np.arange(n, dtype=np.uint64)[:, None]
        cols = np.arange(h, dtype=np.uint64)[None, :]
        pos = np.uint64(sr_counter_base) + rows * np.uint64(h) + cols
        w = sr_word(pos, sr_seed, sr_mode)
        if sr_rule == "threshold":
            idx = stochastic_e2m1_index(v, (w >> np.uint32(8)).astype(np.float64))
        elif sr_rule == "carry":
            idx = stochastic_e2m1_index_carry(v, w)
        else:
            raise ValueError(sr_rule)
    codes = (sign << np.uint8(3)) | idx
    out = np.empty((n, packed_row_bytes(h)), dtype=np.uint8)
    out[:, : h // 2] = F.pack_nibbles(codes)
    out[:, h // 2 : h // 2 + h // 16] = s_code
    out[:, h // 2 + h // 16 :] = t.astype("<f4").view(np.uint8).reshape(n, 4)
    return out


def stochastic_e2m1_index(v, r):
    """R8 rounding step: magnitude v >= 0 (float32 values), r integers in [0, 2^24)."""
    v = np.asarray(v, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    lo = np.clip(np.searchsorted(F.E2M1_GRID, v, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    g_lo, g_hi = F.E2M1_GRID[lo], F.E2M1_GRID[hi]
    with np.errstate(divide="ignore", invalid="ignore"):
        frac = np.where(hi > lo, (v - g_lo) / np.where(hi > lo, g_hi - g_lo, 1.0), 0.0)
    up = (hi > lo) & (r * 2.0 ** -24 < frac)
    return np.where(up, hi, lo).astype(np.uint8)


def stochastic_e2m1_index_carry(v, w):
    """R8b rounding step: magnitude v >= 0 (float32 values), w 32-bit random words.

    v >= 6 gives index 7.  Otherwise frac is v's position between its two
    neighbouring grid points (exact in float64: v has 24 significant bits and
    the grid steps are powers of two), D = floor(frac * 2^32), and the index
    rounds up iff D + w >= 2^32.  So P(up) = D / 2^32 over uniform w, and grid
    points (frac = 0) never move.
    """
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(w, dtype=np.uint64)
    lo = np.clip(np.searchsorted(F.E2M1_GRID, v, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    g_lo, g_hi = F.E2M1_GRID[lo], F.E2M1_GRID[hi]
    with np.errstate(divide="ignore", invalid="ignore"):
        frac = np.where(hi > lo, (v - g_lo) / np.where(hi > lo, g_hi - g_lo, 1.0), 0.0)
    d = np.floor(np.ldexp(frac, 32)).astype(np.uint64)
    up = (hi > lo) & (d + w >= np.uint64(1 << 32))
    return np.where(up, hi, lo).astype(np.uint8)


def split_rows(packed, hidden):
    """Packed rows -> (codes [N, H] uint8, scale codes [N, H/16] uint8, t [N] float64)."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    codes = F.unpack_nibbles(packed[:, : hidden // 2])
    s_code = packed[:, hidden // 2 : hidden // 2 + hidden // 16]
    t = packed[:, hidden // 2 + hidden // 16 :].copy().view("<f4").reshape(n).astype(np.float64)
    return codes, s_code, t


def decode_exact(packed, hidden):
    """Exact decoded values x_hat = e2m1 * s_b * t as float64 [N, H] (R10)."""
    codes, s_code, t = split_rows(packed, hidden)
    s_val = np.repeat(F.e4m3_decode(s_code), 16, axis=1)
    return F.e2m1_value(codes) * s_val * t[:, None]


def unpack_rows(packed, hidden, src_row=None):
    """R10: packed rows -> BF16 bit patterns [M, H].

    x_hat = e2m1 * s_b * t is exact in float64; it is rounded to float32 (exact
    unless below float32's subnormal resolution, where BF16 gives zero anyway)
    and then to BF16 by round-to-nearest-even.  With ``src_row``, output row g
    decodes packed row src_row[g], and src_row[g] = -1 gives a zero row.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    if src_row is not None:
        src_row = np.asarray(src_row, dtype=np.int64)
        gathered = np.zeros((src_row.shape[0], packed.shape[1]), dtype=np.uint8)
        ok = src_row >= 0
        gathered[ok] = packed[src_row[ok]]
        packed = gathered
    vals = decode_exact(packed, hidden)
    return F.f32_to_bf16(vals.astype(np.float32))
