"""Fused dSwiGLU epilogue with amax, and FC1-gradient NVFP4 quantization (CPU oracle; test only).

P4, description: with the option on, the rowwise amax used to quantize the
FC1 gradient is the exact amax emitted by the dGLU epilogue rounded to BF16,
the columnwise (post-RHT) amax is taken as four times the rowwise amax, and
the separate grouped amax pass is skipped.  P4, bot diagram: FC2 backward and
dGLU produce the BF16 FC1 gradient and the maxima; otherwise the maxima are
computed from the gradient.  P4, test commit: per-expert rowwise amaxes equal
the amaxes of the BF16 FC1 gradient, the rowwise operand is unchanged, and the
FC1 wgrad error stays within 5% of the default path.
"""

import numpy as np

from . import formats as F
from .receive import columnwise_operand, quantize_blocks
from .philox import sr_word
from .rht import rht16
from .nvfp4 import TOKEN_SCALE_BOUND


def f64_to_bf16(x):
    """Round float64 values to BF16 (round-to-nearest-even, subnormals kept), bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                                  # |x| in [2^(e-1), 2^e)
    q_exp = np.maximum(e - 8, -133)                     # BF16 keeps 8 significant bits, lsb >= 2^-133
    q = np.ldexp(1.0, q_exp)
    r = np.rint(x / q) * q                              # np.rint: ties to even; exact scaling
    return F.f32_to_bf16(r.astype(np.float32))          # r is a BF16 value: exact in float32


def dswiglu(preact_bits, dy_bits):
    """R17: dX = d(silu(a) * b) / d[a, b] times dy, in float64, rounded once to BF16.

    preact = [a | b] with a the first F columns (the gate).  s = 1/(1+e^-a);
    da = dy * b * s * (1 + a * (1 - s)); db = dy * a * s.
    Returns BF16 bit patterns [T, 2F].
    """
    p = F.bf16_to_f32(preact_bits).astype(np.float64)
    dy = F.bf16_to_f32(dy_bits).astype(np.float64)
    f = dy.shape[1]
    a, b = p[:, :f], p[:, f:]
    s = 1.0 / (1.0 + np.exp(-a))
    da = dy * b * s * (1.0 + a * (1.0 - s))
    db = dy * a * s
    return f64_to_bf16(np.concatenate([da, db], axis=1))


def expert_offsets(counts, alignment=1):
    counts = np.asarray(counts, dtype=np.int64)
    p = (counts + alignment - 1) // alignment * alignment
    off = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    off[1:] = np.cumsum(p)
    return off


def expert_amax(dx_bits, counts):
    """R18: per-expert max |dX| over the expert's rows (BF16 values, held in float32); 0 if empty."""
    x = np.abs(F.bf16_to_f32(dx_bits))
    off = expert_offsets(counts)
    out = np.zeros(len(counts), dtype=np.float32)
    for e in range(len(counts)):
        if counts[e]:
            out[e] = x[off[e] : off[e + 1]].max()
    return out


def rowwise_quant(dx_bits, counts, amax, sr=None, sr_mode="element"):
    """R19: per-expert rowwise NVFP4 operand of the FC1 gradient.

    D_row,e = fl32(amax_e / 2688).  Per 16-element block of a row of expert e:
    s_b = E4M3(fl32(fl32(a_b / 6) / D_row,e)); c = fl32(s_b * D_row,e);
    v = fl32(|x| / c); index = E2M1 rounding (R2).  D = 0 or s_b = 0 gives
    index 0.  With ``sr`` = (seed, counter_base) the index is the carry-form
    stochastic rounding of v (R24): element (row, col) at stream position
    counter_base + row * 2F + col, its index in the [T, 2F] code array, its
    word taken as R8's ``sr_mode`` ("element" or "stream") says.
    Returns (codes uint8 [T, F] packed, scale codes [T, 2F/16], D_row float32 [E]).
    """
    x = F.bf16_to_f32(dx_bits)
    t, h = x.shape
    off = expert_offsets(counts)
    D = (np.asarray(amax, dtype=np.float32) / np.float32(TOKEN_SCALE_BOUND)).astype(np.float32)
    codes = np.zeros((t, h), dtype=np.uint8)
    scales = np.zeros((t, h // 16), dtype=np.uint8)
    for e in range(len(counts)):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        blk = x[r0:r1].reshape(r1 - r0, h // 16, 16)
        words = None
        if sr is not None:
            pos = np.uint64(sr[1]) + (np.arange(r0, r1, dtype=np.uint64)[:, None] * np.uint64(h)
                                      + np.arange(h, dtype=np.uint64)[None, :])
            words = sr_word(pos.reshape(r1 - r0, h // 16, 16), sr[0], sr_mode)
        c, s = quantize_blocks(blk, D[e], "fp32", words)
        codes[r0:r1] = c.reshape(r1 - r0, h)
        scales[r0:r1] = s
    return F.pack_nibbles(codes), scales, D


def columnwise_quant(dx_bits, counts, amax, exact_amax=False, sr=None, sr_mode="element"):
    """R20 (and R21 with ``exact_amax``): per-expert RHT columnwise operand.

    D_col,e = fl32(4 * amax_e / 2688) -- the bound from P4 -- or, for the
    default-path reference, fl32(amax_post,e / 2688) with amax_post the exact
    max |y| over the expert's post-RHT values.  Rows are zero-padded to
    P_e = roundup(count_e, 16).  Expert e's codes form an [2F, P_e/2] matrix
    at byte 2F * off_e / 2 and its scales an [2F, P_e/16] matrix at byte
    2F * off_e / 16, with off_e the padded offsets.  With ``sr`` = (seed,
    counter_base), stochastic codes (R24): expert e's element (h, r) at stream
    position counter_base + 2F * off_e + h * P_e + r, its index in the codes.
    """
    x = F.bf16_to_f32(dx_bits).astype(np.float64)
    t, h = x.shape
    off = expert_offsets(counts)
    poff = expert_offsets(counts, 16)
    codes = np.zeros(h * poff[-1] // 2, dtype=np.uint8)
    scales = np.zeros(h * poff[-1] // 16, dtype=np.uint8)
    D = np.zeros(len(counts), dtype=np.float32)
    for e in range(len(counts)):
        c = int(counts[e])
        if c == 0:
            continue
        if exact_amax:
            p = (c + 15) // 16 * 16
            full = np.zeros((p, h)); full[:c] = x[off[e] : off[e + 1]]
            amax_post = np.abs(rht16(full.T.reshape(h, p // 16, 16))).max()
            D[e] = np.float32(amax_post) / np.float32(TOKEN_SCALE_BOUND)
        else:
            D[e] = (np.float32(4.0) * np.float32(amax[e])) / np.float32(TOKEN_SCALE_BOUND)
        cc, cs = columnwise_operand(x[off[e] : off[e + 1]], c, D[e], "fp32",
                                    sr=None if sr is None else (sr[0], sr[1] + h * int(poff[e])), sr_mode=sr_mode)
        codes[h * poff[e] // 2 : h * poff[e + 1] // 2] = cc.reshape(-1)
        scales[h * poff[e] // 16 : h * poff[e + 1] // 16] = cs.reshape(-1)
    return codes, scales, D


def fc1_grad_quant(dx_bits, counts, amax, sr=None, sr_mode="element"):
    """The fused path after the epilogue: rowwise (R19) and columnwise (R20) operands;
    ``sr`` = (seed, counter_base) makes both stochastic (R24), the columnwise
    operand's positions following the rowwise operand's T * 2F; ``sr_mode`` picks
    each position's Philox word as R8 does ("element" or "stream")."""
    t, h = np.asarray(dx_bits).shape
    rc, rs, drow = rowwise_quant(dx_bits, counts, amax, sr, sr_mode)
    cc, cs, dcol = columnwise_quant(dx_bits, counts, amax,
                                    sr=None if sr is None else (sr[0], sr[1] + t * h), sr_mode=sr_mode)
    return dict(row_codes=rc, row_scales=rs, row_scale=drow, col_codes=cc, col_scales=cs, col_scale=dcol)
