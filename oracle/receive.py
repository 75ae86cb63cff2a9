"""Direct receive: packed NVFP4 rows -> the expert GEMM's grouped operands (CPU oracle; test only).

P1, PR description and first commit message: the receiver builds the grouped
NVFP4 tensor for the expert GEMM straight from the received rows in one pass;
the rowwise operand reuses the sender's codes, and the columnwise operand is
an RHT operand quantized with a per-expert scale derived from a bound, so that
neither a BF16 round trip nor an amax pass is needed.  P3, description and bot
summary: row-scaled (per-token) NVFP4 tensors are GEMM operands, which is the
form the reused rowwise codes take here.

This module defines the direct receive as the unfused pipeline

    route_plan -> gather the packed rows -> decode to exact values ->
    16-point RHT down each column -> quantize with the bound-derived scale.

Decoded NVFP4 values carry at most 6 significant bits, so a BF16 round trip
would be lossless: the one-pass kernel must equal this pipeline exactly.
"""

import numpy as np

from . import formats as F
from . import nvfp4
from .philox import sr_word
from .rht import rht16
from .routing import route_plan


# ------------------------------------------------------------------ shared columnwise quantizer
def block_scale_codes(a, D, mode):
    """E4M3 scale codes of blocks with post-RHT maxima ``a`` (float32, >= 0).

    mode "pow2" (R16; D a power of two, the bound-derived per-expert decode
        scale): s = E4M3 round-to-nearest-even of the exact a / (6 * D).  In
        float64, a / 6 is within 2^-53 (relative) of the exact quotient, which
        is never closer than about 2^-26 to an E4M3 tie (a has 24 bits, a tie
        5), and the division by the power of two D is exact: so the float64
        value rounds to E4M3 exactly as the exact one does.
    mode "fp32" (R19/R20; D any float32): s = E4M3(fl32(fl32(a / 6) / D)),
        fl32 being IEEE binary32 with gradual underflow, as written.
    D = 0 gives code 0.
    """
    a = np.asarray(a, dtype=np.float32)
    D32 = np.float32(D)
    if not D32 > 0:
        return np.zeros(a.shape, dtype=np.uint8)
    if mode == "pow2":
        return F.e4m3_encode(a.astype(np.float64) / 6.0 / float(D32))
    if mode == "fp32":
        with np.errstate(under="ignore", over="ignore"):
            pre = (a / np.float32(6.0)) / D32             # two float32 roundings, as written
        return F.e4m3_encode(pre.astype(np.float64))
    raise ValueError(mode)


def block_codes(y, s_code, D, mode, words=None):
    """E2M1 codes of post-RHT values y [..., 16] (float32) given each block's
    scale code ``s_code`` [...] and the global decode scale D.

    mode "pow2" (R16): index = E2M1 rounding (R2) of v = fl32(|y| / (s * D)),
        the exact quotient rounded once to float32 (s * D is exact in float64).
    mode "fp32" (R19/R20): c = fl32(s * D), v = fl32(|y| / c).
    s = 0 (or D = 0) gives magnitude index 0.  The code's sign is y's sign bit.
    ``words`` (R24): 32-bit random words, one per element (y's shape); the
    index is then the carry-form stochastic rounding of v (R8b) instead of R2.
    """
    y = np.asarray(y, dtype=np.float32)
    D32 = np.float32(D)
    s_val = F.e4m3_decode(s_code)
    ay = np.abs(y)
    ok = (s_val > 0)[..., None] & np.ones(y.shape, dtype=bool)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        if mode == "pow2":
            q = ay.astype(np.float64) / (s_val[..., None] * float(D32))
            v = q.astype(np.float32)
        elif mode == "fp32":
            c = (s_val.astype(np.float32) * D32)[..., None]
            v = ay / c
        else:
            raise ValueError(mode)
    v = np.where(ok, v, np.float32(0.0))
    if words is None:
        idx = F.e2m1_index(v.astype(np.float64))
    else:
        idx = nvfp4.stochastic_e2m1_index_carry(v.astype(np.float64), np.asarray(words).reshape(v.shape))
    sign = (y.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    return (sign << np.uint8(3)) | idx


def quantize_blocks(y, D, mode, words=None):
    """Quantize post-RHT blocks y [..., 16] (float32) with global decode scale D:
    a = max |y_i| over the block, the scale by ``block_scale_codes``, the codes
    by ``block_codes``.  Returns (codes uint8 [..., 16], scale codes uint8 [...]).
    """
    y = np.asarray(y, dtype=np.float32)
    s_code = block_scale_codes(np.abs(y).max(axis=-1), D, mode)
    return block_codes(y, s_code, D, mode, words), s_code


def columnwise_operand(values, count, D, mode, padded_rows=None, sr=None, sr_mode="element"):
    """One expert's columnwise operand from its grouped rows.

    values [count, H]: exact values of the expert's rows (float64), in grouped
    order; rows count..P-1 are zero padding, P = padded_rows (default
    roundup(count, 16)).  Padding rows are transformed and quantized like any
    other rows (their codes carry the sign bits of the signed-zero results).
    ``sr`` = (seed, n0): stochastic codes (R24); the element of column h and
    grouped row r (0-based in the expert) has stream position n0 + h * P + r,
    its index in the expert's [H, P] code matrix plus n0; ``sr_mode`` picks
    the word of a position as the pack does (R8: "element" or "stream").
    Returns (codes uint8 [H, P/2], scale codes uint8 [H, P/16]).
    """
    values = np.asarray(values, dtype=np.float64)
    h = values.shape[1]
    p = (count + 15) // 16 * 16 if padded_rows is None else int(padded_rows)
    full = np.zeros((p, h), dtype=np.float64)
    full[:count] = values[:count]
    blocks = full.T.reshape(h, p // 16, 16)             # [H, P/16, 16] : column h, block m, row i
    y = rht16(blocks)
    words = None
    if sr is not None:
        seed, n0 = sr
        words = sr_word(np.uint64(n0) + np.arange(h * p, dtype=np.uint64).reshape(h, p // 16, 16), seed, sr_mode)
    codes, s_code = quantize_blocks(y, D, mode, words)
    return F.pack_nibbles(codes.reshape(h, p)), s_code


def expert_decode_scale(t_rows):
    """R14: D_e = 4 * max t over the expert's rows (a power of two); 0 if the expert is empty."""
    t_rows = np.asarray(t_rows, dtype=np.float64)
    return 4.0 * float(t_rows.max()) if t_rows.size else 0.0


# ------------------------------------------------------------------ the direct receive
def direct_receive(packed, hidden, topk_idx, num_experts, alignment, r_cap=None, columnwise=True, sr=None,
                   sr_mode="element"):
    """R12-R16 (and R24 with ``sr`` = (seed, counter_base): stochastic columnwise
    codes, expert e's element (h, r) at stream position counter_base +
    H * off_e + h * P_e + r -- the code's index in ``col_codes``, two per byte;
    ``sr_mode`` "element" or "stream" maps a position to its Philox word as R8
    does for the pack).
    Returns the routing plan plus the grouped operands.

    Rowwise (R13): grouped row g with source token s >= 0 holds the sender's
    code bytes, scale bytes and t unchanged; padding rows are zero bytes
    (t = 0).  Rows from off_E to r_cap are left zero here (unspecified).
    Columnwise (R14-R16): per expert, D_e = 4 * max t; the operand is
    ``columnwise_operand`` of the decoded grouped rows in mode "pow2".
    Expert e's codes are an [H, P_e/2] byte matrix at byte H * off_e / 2 of
    ``col_codes``; its scales an [H, P_e/16] matrix at byte H * off_e / 16.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    t_tok, k = np.asarray(topk_idx).shape
    plan = route_plan(topk_idx, num_experts, alignment, r_cap)
    r_cap = plan["src_row"].shape[0]
    src = plan["src_row"].astype(np.int64)
    off = plan["offsets"].astype(np.int64)
    counts = plan["counts"].astype(np.int64)
    h = hidden
    codes, s_code, t = nvfp4.split_rows(packed, h)
    ok = src >= 0
    row_codes = np.zeros((r_cap, h // 2), dtype=np.uint8)
    row_scales = np.zeros((r_cap, h // 16), dtype=np.uint8)
    row_t = np.zeros(r_cap, dtype=np.float32)
    row_codes[ok] = packed[src[ok], : h // 2]
    row_scales[ok] = packed[src[ok], h // 2 : h // 2 + h // 16]
    row_t[ok] = t[src[ok]].astype(np.float32)
    out = dict(plan, row_codes=row_codes, row_scales=row_scales, row_t=row_t)
    if not columnwise:
        return out
    D = np.zeros(num_experts, dtype=np.float32)
    col_codes = np.zeros(r_cap * h // 2, dtype=np.uint8)
    col_scales = np.zeros(r_cap * h // 16, dtype=np.uint8)
    exact = nvfp4.decode_exact(packed, h)
    for e in range(num_experts):
        c = int(counts[e])
        rows = src[off[e] : off[e] + c]
        D[e] = expert_decode_scale(t[rows])
        if c == 0:
            continue
        p = int(off[e + 1] - off[e])                    # P_e: all padded rows of the slot
        cc, cs = columnwise_operand(exact[rows], c, D[e], "pow2", padded_rows=p,
                                    sr=None if sr is None else (sr[0], sr[1] + h * int(off[e])), sr_mode=sr_mode)
        col_codes[h * off[e] // 2 : h * off[e + 1] // 2] = cc.reshape(-1)
        col_scales[h * off[e] // 16 : h * off[e + 1] // 16] = cs.reshape(-1)
    out.update(col_codes=col_codes, col_scales=col_scales, col_scale=D)
    return out


def kblock_layout(col_codes, col_scales, offsets, hidden, block_rows=256, scale_rows=16):
    """The columnwise operand re-laid in K-blocks (a GEMM-ready variant of R16).

    Per expert e (P_e = offsets[e+1] - offsets[e] grouped rows), the grouped
    rows are cut into K-blocks of ``block_rows`` (the last one shorter); block
    kb holds rows [kb*block_rows, kb*block_rows + len) as an [H, len/2] code
    matrix (row h = column h, grouped-row order, low nibble first) at byte
    H*off_e/2 + H*kb*block_rows/2, and an [H, len/S] scale matrix at byte
    H*off_e/S + H*kb*block_rows/S, S = ``scale_rows`` grouped rows per scale
    (16 for NVFP4, 32 for the MXFP4 receive's R23).  The values are those of
    the compact layout; only their places change.
    """
    col_codes = np.asarray(col_codes, dtype=np.uint8)
    col_scales = np.asarray(col_scales, dtype=np.uint8)
    off = np.asarray(offsets, dtype=np.int64)
    h, sr = hidden, scale_rows
    out_c = np.zeros_like(col_codes)
    out_s = np.zeros_like(col_scales)
    for e in range(off.shape[0] - 1):
        o, p = int(off[e]), int(off[e + 1] - off[e])
        if p == 0:
            continue
        cm = col_codes[h * o // 2 : h * (o + p) // 2].reshape(h, p // 2)
        sm = col_scales[h * o // sr : h * (o + p) // sr].reshape(h, p // sr)
        for r0 in range(0, p, block_rows):
            ln = min(block_rows, p - r0)
            c0 = h * (o + r0) // 2
            s0 = h * (o + r0) // sr
            out_c[c0 : c0 + h * ln // 2] = cm[:, r0 // 2 : (r0 + ln) // 2].reshape(-1)
            out_s[s0 : s0 + h * ln // sr] = sm[:, r0 // sr : (r0 + ln) // sr].reshape(-1)
    return out_c, out_s


def columnwise_sample(packed, hidden, plan, expert, col_lo, col_hi, blk_lo, blk_hi, D):
    """Columnwise codes/scales of one expert restricted to columns [col_lo, col_hi)
    and 16-row blocks [blk_lo, blk_hi) -- for sampled checks at full size.

    Returns (codes uint8 [cols, 16*(blk_hi-blk_lo)] unpacked 4-bit codes,
    scale codes uint8 [cols, blk_hi-blk_lo])."""
    src = plan["src_row"].astype(np.int64)
    off = int(plan["offsets"][expert])
    rows = src[off + 16 * blk_lo : off + 16 * blk_hi]
    vals = np.zeros((rows.shape[0], col_hi - col_lo), dtype=np.float64)
    ok = rows >= 0
    if ok.any():
        sub = np.asarray(packed)[rows[ok]]
        ex = nvfp4.decode_exact(sub, hidden)
        vals[ok] = ex[:, col_lo:col_hi]
    blocks = vals.T.reshape(col_hi - col_lo, blk_hi - blk_lo, 16)
    y = rht16(blocks)
    codes, s_code = quantize_blocks(y, D, "pow2")
    return codes.reshape(col_hi - col_lo, -1), s_code
