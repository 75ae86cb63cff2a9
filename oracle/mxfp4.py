"""MXFP4 grouped operands at the receiver (CPU oracle; test only).

Not a step the pages take: the direct receive of P1 (PR description and first
commit message) builds grouped NVFP4 operands whose E4M3 block scales cover 16
elements, and gfx950's block-scaled matrix instructions do not read those.  They
read MXFP4 directly: E2M1 elements with one E8M0 scale (a power of two) per 32
consecutive elements along K.  This module defines an MXFP4 variant of the same
receive -- same routing, same decode, same 16-point RHT for the columnwise
operand -- with only the final quantizer replaced.  Its readings (R22, R23) are
ours, not the pages'; every step is exact except the RHT's float32 sums, which are
the ones R15 already fixes.

R22 (block quantizer).  For a block of 32 values with a = max |x|:
    e = the least integer with a <= 6 * 2^e (no element is clipped), clamped to
        [-127, 127]; a = 0 gives e = 0.  For a = m * 2^E, m in [1, 2), that is
        e = E - 2 + [m > 1.5].  The scale byte is e + 127 (E8M0).
    code = sign bit of x (bit 3) | E2M1 index (R2) of |x| / 2^e, which is exact.
    This is the rule the MXFP8 pack uses (R11) with 6, E2M1's largest value, in
    place of 448.
R23 (receive).  Rowwise: grouped row g with source token s >= 0 holds the exact
    decoded values of token s (R10); padding rows hold zeros; R22 applies to
    each 32-element block along H.  Codes [R_cap, H/2] (two per byte, element 2j
    in the low nibble), scales [R_cap, H/32].  Rows off_E .. r_cap are not
    written.  Columnwise: per expert, the RHT of R15 over each 16 consecutive
    grouped rows of a column, then R22 over each 32 consecutive grouped rows
    (two RHT blocks) of the column; P_e must be a multiple of 32, so the
    alignment must be.  Expert e's codes are an [H, P_e/2] byte matrix at byte
    H * off_e / 2 of the columnwise codes, its scales an [H, P_e/32] matrix at
    byte H * off_e / 32.  No per-expert scale: the block scales are powers of
    two, so no amax bound is needed.
"""

import numpy as np

from . import formats as F
from . import nvfp4
from .rht import rht16
from .routing import route_plan

BLOCK = 32


def scale_exponent(amax):
    """R22: least e with amax <= 6 * 2^e, clamped to [-127, 127]; amax = 0 gives 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)                      # amax in [2^(E-1), 2^E)
    e = (E - 5).astype(np.int64)               # 6 * 2^(E-5) = 0.75 * 2^(E-2) < amax
    for _ in range(4):
        e = np.where(amax > F.E2M1_MAX * np.ldexp(1.0, e), e + 1, e)
    e = np.where(amax == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize(x):
    """R22 along the last axis (a multiple of 32): x exact values (float64 or float32).

    Returns (codes uint8 [..., n] one 4-bit code per element, scale bytes uint8 [..., n/32]).
    """
    x = np.asarray(x)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    xb = x.astype(np.float64).reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    e = scale_exponent(np.abs(xb).max(axis=-1))
    y = np.abs(xb) / np.ldexp(1.0, e)[..., None]          # exact: a power-of-two divisor
    idx = F.e2m1_index(y)
    sign = np.signbit(xb).astype(np.uint8)
    codes = (sign << np.uint8(3)) | idx
    return codes.reshape(x.shape), (e + 127).astype(np.uint8)


def decode(codes, scales):
    """Exact values of MXFP4 blocks: codes [..., n] (one per element), scales [..., n/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return F.e2m1_value(codes) * np.repeat(s, BLOCK, axis=-1)


def columnwise_operand(values, count, padded_rows):
    """One expert's MXFP4 columnwise operand (R23): values [count, H] exact, rows
    count .. padded_rows-1 zero padding.  Returns (codes [H, P/2] packed bytes,
    scale bytes [H, P/32])."""
    values = np.asarray(values, dtype=np.float64)
    h = values.shape[1]
    p = int(padded_rows)
    if p % BLOCK:
        raise ValueError("padded rows must be a multiple of 32")
    full = np.zeros((p, h), dtype=np.float64)
    full[:count] = values[:count]
    y = rht16(full.T.reshape(h, p // 16, 16)).reshape(h, p)   # float32, R15
    codes, scales = quantize(y)
    return F.pack_nibbles(codes), scales


def direct_receive(packed, hidden, topk_idx, num_experts, alignment, r_cap=None):
    """R12 + R23: the routing plan plus the MXFP4 rowwise and columnwise operands."""
    if alignment % BLOCK:
        raise ValueError("the MXFP4 receive needs an alignment that is a multiple of 32")
    packed = np.asarray(packed, dtype=np.uint8)
    plan = route_plan(topk_idx, num_experts, alignment, r_cap)
    r_cap = plan["src_row"].shape[0]
    src = plan["src_row"].astype(np.int64)
    off = plan["offsets"].astype(np.int64)
    counts = plan["counts"].astype(np.int64)
    h = hidden
    exact = nvfp4.decode_exact(packed, h)
    rows = np.zeros((r_cap, h), dtype=np.float64)
    ok = src >= 0
    rows[ok] = exact[src[ok]]
    n_out = int(off[-1])
    rc, rs = quantize(rows[:n_out])
    row_codes = np.zeros((r_cap, h // 2), dtype=np.uint8)
    row_scales = np.zeros((r_cap, h // BLOCK), dtype=np.uint8)
    row_codes[:n_out] = F.pack_nibbles(rc)
    row_scales[:n_out] = rs
    col_codes = np.zeros(r_cap * h // 2, dtype=np.uint8)
    col_scales = np.zeros(r_cap * h // BLOCK, dtype=np.uint8)
    for e in range(num_experts):
        p = int(off[e + 1] - off[e])
        if p == 0:
            continue
        c = int(counts[e])
        cc, cs = columnwise_operand(rows[off[e] : off[e] + c], c, p)
        col_codes[h * off[e] // 2 : h * off[e + 1] // 2] = cc.reshape(-1)
        col_scales[h * off[e] // BLOCK : h * off[e + 1] // BLOCK] = cs.reshape(-1)
    return dict(plan, row_codes=row_codes, row_scales=row_scales, col_codes=col_codes, col_scales=col_scales)
