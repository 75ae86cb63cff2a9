"""Pins of R24: carry-form stochastic rounding of the gradient operands (the receive's
columnwise operand, the FC1-grad rowwise and columnwise operands), with each code's
stream position its index in the operand's code array.

* The FC1-grad rowwise operand on inputs whose quotients are exact E2M1 midpoints:
  frac = 1/2 there, so an element rounds up iff the top bit of the Philox word at its
  position is set -- the positions are then read off the codes and compared with the
  code-array index, enumerated here byte by byte.
* The columnwise operands: every code is one of the two grid neighbours of its
  quotient, and the choice follows the carry rule with the word at the code's index
  in the code array (enumerated here from the byte layout).
* Scales never change, and the words' all-zero / all-ones limits give the floor /
  ceiling indices.
"""

import numpy as np
import pytest

import workloads
from oracle import dswiglu as D
from oracle import formats as F
from oracle import nvfp4, receive, rht
from oracle.philox import sr_word

MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _grid_floor_ceil(v):
    g = F.E2M1_GRID
    lo = np.clip(np.searchsorted(g, v, side="right") - 1, 0, 7)
    hi = np.where(g[lo] == v, lo, np.minimum(lo + 1, 7))
    return lo, hi


def test_words_at_the_limits_give_floor_and_ceiling():
    rng = np.random.default_rng(1)
    y = np.clip(rng.standard_normal((50, 16)) * 3, -5.9, 5.9).astype(np.float32)
    y[:, 0] = 6.0                                                    # D = 1, s = 1: v = |y|
    down, s0 = receive.quantize_blocks(y, 1.0, "pow2", np.zeros(y.shape, np.uint32))
    up, s1 = receive.quantize_blocks(y, 1.0, "pow2", np.full(y.shape, 0xFFFFFFFF, np.uint32))
    _, s_rne = receive.quantize_blocks(y, 1.0, "pow2")
    assert np.array_equal(s0, s_rne) and np.array_equal(s1, s_rne)
    lo, hi = _grid_floor_ceil(np.abs(y).astype(np.float64))
    assert np.array_equal(down & 7, lo) and np.array_equal(up & 7, hi)


@pytest.mark.parametrize("words, base", [("element", 12345), ("stream", 12345), ("stream", 12346)])
def test_fc1_rowwise_positions_from_midpoint_inputs(words, base):
    # amax 2688 -> D_row = 1 exactly; each 16-block holds 2688 (s = 448, c = 448) and
    # values 448 * m with m an E2M1 midpoint, so v = m exactly and frac = 1/2
    rng = np.random.default_rng(2)
    t, h = 24, 64
    vals = 448.0 * rng.choice(MIDS, size=(t, h)) * rng.choice([-1.0, 1.0], size=(t, h))
    vals[:, ::16] = 2688.0
    bits = F.f32_to_bf16(vals.astype(np.float32))
    counts = np.array([10, 0, 14])
    seed = 77
    amax = D.expert_amax(bits, counts)
    assert np.all(amax[counts > 0] == 2688.0)
    rc, rs, drow = D.rowwise_quant(bits, counts, amax, sr=(seed, base), sr_mode=words)
    codes = F.unpack_nibbles(rc)                                     # [t, h]
    lo, hi = _grid_floor_ceil(np.abs(vals) / 448.0)
    for j in range(rc.size * 2):                                     # flat code index = byte * 2 + nibble
        r, c = divmod(j, h)
        if c % 16 == 0:
            assert codes[r, c] & 7 == 7
            continue
        w = int(sr_word(np.uint64(base + j), seed, words))
        want = hi[r, c] if w >= (1 << 31) else lo[r, c]
        assert codes[r, c] & 7 == want, (r, c)


def _check_columnwise(codes_bytes, scale_bytes, y_blocks, Dv, mode, seed, base, h, p, words="element"):
    """Columnwise [h, p] operand of one expert: each code against the carry rule with
    the word at its index in the code bytes (base = the position of byte 0, nibble 0)."""
    codes = F.unpack_nibbles(codes_bytes.reshape(h, p // 2))       # [h, p]
    s_val = F.e4m3_decode(scale_bytes.reshape(h, p // 16))
    for j in range(h * p):
        col, r = divmod(j, p)
        y = np.float32(y_blocks[col, r // 16, r % 16])
        if mode == "pow2":
            v = np.float32(abs(float(y)) / (float(s_val[col, r // 16]) * float(Dv)))
        else:
            c = np.float32(np.float32(s_val[col, r // 16]) * np.float32(Dv))
            v = np.float32(abs(y) / c) if c > 0 else np.float32(0)
        if s_val[col, r // 16] == 0:
            v = np.float32(0)
        want = nvfp4.stochastic_e2m1_index_carry(np.float64(v), sr_word(np.uint64(base + j), seed, words))
        assert codes[col, r] & 7 == want, (col, r)


@pytest.mark.parametrize("words, base", [("element", 1 << 33), ("stream", 1 << 33), ("stream", (1 << 33) + 3)])
def test_receive_columnwise_positions(words, base):
    """Both word mappings (R8) at the receive's positions (R24); the stream mapping also
    with a counter base that is not a multiple of 4, so blocks of four words straddle
    the 16-row blocks."""
    w = workloads.small_dispatch(3, 40, 64, 3, 2, alignment=16, empty=[1])
    packed = nvfp4.pack_rows(w.x_bits)
    seed = 99
    out = receive.direct_receive(packed, 64, w.topk_idx, 3, 16, sr=(seed, base), sr_mode=words)
    rne = receive.direct_receive(packed, 64, w.topk_idx, 3, 16)
    assert np.array_equal(out["col_scales"], rne["col_scales"])
    off, src = out["offsets"].astype(np.int64), out["src_row"].astype(np.int64)
    exact = nvfp4.decode_exact(packed, 64)
    for e in range(3):
        p = int(off[e + 1] - off[e])
        if p == 0:
            continue
        rows = np.zeros((p, 64))
        ok = src[off[e] : off[e + 1]] >= 0
        rows[ok] = exact[src[off[e] : off[e + 1]][ok]]
        y = rht.rht16(rows.T.reshape(64, p // 16, 16))
        _check_columnwise(out["col_codes"][64 * off[e] // 2 : 64 * off[e + 1] // 2],
                          out["col_scales"][64 * off[e] // 16 : 64 * off[e + 1] // 16], y, out["col_scale"][e],
                          "pow2", seed, base + 64 * int(off[e]), 64, p, words)
    if words == "stream":   # the mappings give different codes: the parameter is not ignored
        other = receive.direct_receive(packed, 64, w.topk_idx, 3, 16, sr=(seed, base))
        assert not np.array_equal(out["col_codes"], other["col_codes"])


@pytest.mark.parametrize("words, base", [("element", 1000), ("stream", 1000), ("stream", 1001)])
def test_fc1_columnwise_positions_follow_the_rowwise_operand(words, base):
    w = workloads.small_dswiglu(4, [7, 0, 20], 32)
    dx = D.dswiglu(w.preact_bits, w.dy_bits)
    t, h = dx.shape
    amax = D.expert_amax(dx, w.counts)
    seed = 5
    q = D.fc1_grad_quant(dx, w.counts, amax, sr=(seed, base), sr_mode=words)
    q_rne = D.fc1_grad_quant(dx, w.counts, amax)
    assert np.array_equal(q["row_scales"], q_rne["row_scales"]) and np.array_equal(q["col_scales"], q_rne["col_scales"])
    x = F.bf16_to_f32(dx).astype(np.float64)
    off = D.expert_offsets(w.counts)
    poff = D.expert_offsets(w.counts, 16)
    for e in range(3):
        c = int(w.counts[e])
        if c == 0:
            continue
        p = (c + 15) // 16 * 16
        full = np.zeros((p, h))
        full[:c] = x[off[e] : off[e + 1]]
        y = rht.rht16(full.T.reshape(h, p // 16, 16))
        _check_columnwise(q["col_codes"][h * poff[e] // 2 : h * poff[e + 1] // 2],
                          q["col_scales"][h * poff[e] // 16 : h * poff[e + 1] // 16], y, q["col_scale"][e],
                          "fp32", seed, base + t * h + h * int(poff[e]), h, p, words)


def test_stochastic_codes_are_unbiased():
    """Mean of the decoded stochastic values over many seeds equals v (D = 1, s = 1)."""
    y = np.array([[6.0, 0.3, 1.1, 2.2, 3.3, 4.4, 5.5, 0.1, 0.6, 1.6, 2.6, 3.6, 4.6, 5.6, 0.05, 1.9]], np.float32)
    acc = np.zeros(16)
    n = 4000
    for s in range(n):
        words = sr_word(np.arange(16, dtype=np.uint64) + np.uint64(16 * s), 31)
        codes, _ = receive.quantize_blocks(y, 1.0, "pow2", words.reshape(1, 16))
        acc += F.e2m1_value(codes[0])
    mean = acc / n
    assert np.all(np.abs(mean - y[0].astype(np.float64)) < 0.05)
