"""Pins of the MXFP4 oracle (R22, R23) against definitions written out independently here:
brute-force exponent and nearest-grid searches, a hand-worked block, the Hadamard
matrix, and the NVFP4 values each MXFP4 element approximates."""

from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import mxfp4 as M
from oracle import nvfp4, rht
from oracle.routing import route_plan

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def brute_exponent(a):
    """Least e in [-127, 127] with a <= 6 * 2^e, by scanning; 0 for a = 0."""
    if a == 0:
        return 0
    for e in range(-127, 128):
        if Fraction(a) <= 6 * Fraction(2) ** e:
            return e
    return 127


def brute_index(v):
    """Nearest E2M1 magnitude to v >= 0 (exact rationals), ties to the even index."""
    v = Fraction(v)
    best = min(range(8), key=lambda i: (abs(GRID[i] - v), i % 2))
    return best


def test_scale_exponent_matches_the_scan_and_the_closed_form():
    rng = np.random.default_rng(1)
    a = np.concatenate([
        np.ldexp(rng.uniform(1, 2, 2000), rng.integers(-150, 120, 2000)),
        6.0 * np.ldexp(1.0, np.arange(-127, 120)),                        # exactly 6 * 2^e: no step up
        np.nextafter(6.0 * np.ldexp(1.0, np.arange(-120, 120)), np.inf),  # just above: one step up
        1.5 * np.ldexp(1.0, np.arange(-120, 120)),                        # m = 1.5 exactly
        [0.0, 5e-324, 1e-45, 3.4e38],
    ])
    got = M.scale_exponent(a)
    want = np.array([brute_exponent(float(x)) for x in a])
    assert np.array_equal(got, want)
    # closed form e = E - 2 + [m > 1.5] away from the clamp
    m, E = np.frexp(a[a > 0])
    m, E = 2 * m, E - 1
    closed = E - 2 + (m > 1.5)
    inside = (closed >= -127) & (closed <= 127)
    assert np.array_equal(got[a > 0][inside], closed[inside])


def test_no_element_clips_and_the_exponent_is_minimal():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((400, 64)) * np.ldexp(1.0, rng.integers(-30, 30, (400, 1)))
    codes, scales = M.quantize(x)
    e = scales.astype(np.int64) - 127
    a = np.abs(x).reshape(400, 2, 32).max(axis=2)
    assert np.all(a <= 6.0 * np.ldexp(1.0, e))
    assert np.all(a > 6.0 * np.ldexp(1.0, e - 1))


def test_codes_are_the_nearest_grid_point_ties_to_even():
    rng = np.random.default_rng(3)
    # a block whose scale is 2^0 (max 6) holding every midpoint, their negatives and random values
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = np.concatenate([[6.0], mids, [-m for m in mids], rng.uniform(-6, 6, 17)])
    codes, scales = M.quantize(vals.reshape(1, 32))
    assert scales[0, 0] == 127
    for v, c in zip(vals, codes[0]):
        assert (c & 7) == brute_index(abs(v)), v
        assert (c >> 3) == (1 if np.signbit(v) else 0)
    # the tie rule at each midpoint: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    assert [int(c & 7) for c in codes[0, 1:8]] == [0, 2, 2, 4, 4, 6, 6]
    assert [int(c) for c in codes[0, 8:15]] == [8, 10, 10, 12, 12, 14, 14]


def test_hand_worked_block():
    """Block max 5.5 -> e = 0 (5.5 <= 6); values 5.5, -2.6, 0.3, 0, -0.0, 1.75, then 26 x 0.1."""
    x = np.array([5.5, -2.6, 0.3, 0.0, -0.0, 1.75] + [0.1] * 26)
    codes, scales = M.quantize(x.reshape(1, 32))
    assert scales[0, 0] == 127                                  # 2^0
    # 5.5 -> 6 (index 7); -2.6 -> 3 (index 5) negative; 0.3 -> 0.5 (index 1);
    # 0 -> 0; -0 -> negative zero (code 8); 1.75 -> tie -> 2 (index 4); 0.1 -> 0
    assert codes[0, :6].tolist() == [7, 8 | 5, 1, 0, 8, 4]
    assert np.all(codes[0, 6:] == 0)
    # block max 7 -> e = 1 (7 > 6, 7 <= 12): 7/2 = 3.5 -> tie -> 4 (index 6)
    codes, scales = M.quantize(np.array([7.0] + [0.0] * 31).reshape(1, 32))
    assert scales[0, 0] == 128 and codes[0, 0] == 6


def test_decode_error_is_at_most_half_a_step():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((200, 96)) * 10.0 ** rng.uniform(-3, 3, (200, 1))
    codes, scales = M.quantize(x)
    back = M.decode(codes, scales)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    # the E2M1 step around |x|/2^e is at most 2 (between 4 and 6), 0.5 below 2
    step = np.where(np.abs(x) / np.ldexp(1.0, e) >= 4, 2.0, np.where(np.abs(x) / np.ldexp(1.0, e) >= 2, 1.0, 0.5))
    assert np.all(np.abs(back - x) <= 0.5 * step * np.ldexp(1.0, e))


def test_columnwise_equals_the_hadamard_matrix_on_exact_inputs():
    """On inputs whose transform is exact in float32 (small integers times 2^-3),
    the RHT is the Sylvester Hadamard matrix times the signs over 4."""
    rng = np.random.default_rng(5)
    vals = rng.integers(-8, 9, (40, 64)).astype(np.float64) / 8.0
    codes, scales = M.columnwise_operand(vals, 40, 64)
    H16 = np.array([[1.0]])
    for _ in range(4):
        H16 = np.block([[H16, H16], [H16, -H16]])
    d = rht.signs()
    full = np.zeros((64, 64))
    full[:40] = vals
    y = np.zeros((64, 64))                                       # [column, row]
    for c in range(64):
        for b in range(4):
            y[c, 16 * b : 16 * b + 16] = H16 @ (d * full[16 * b : 16 * b + 16, c]) / 4.0
    want_c, want_s = M.quantize(y)
    got_c = F.unpack_nibbles(codes)
    # the butterfly gives -0 where the matrix product gives +0 (sign flips of zero
    # rows): compare magnitudes everywhere and signs of the nonzero codes
    assert np.array_equal(got_c & 7, want_c & 7)
    nz = (want_c & 7) != 0
    assert np.array_equal(got_c[nz], want_c[nz])
    assert np.array_equal(scales, want_s)


def test_receive_rowwise_approximates_the_nvfp4_values():
    w = workloads.small_dispatch(6, 120, 128, 5, 2, alignment=32, unused_frac=0.1, empty=[2])
    packed = nvfp4.pack_rows(w.x_bits)
    out = M.direct_receive(packed, 128, w.topk_idx, 5, 32)
    plan = route_plan(w.topk_idx, 5, 32)
    off = plan["offsets"].astype(np.int64)
    src = plan["src_row"].astype(np.int64)
    exact = nvfp4.decode_exact(packed, 128)
    rows = np.where(src[: off[-1], None] >= 0, exact[np.maximum(src[: off[-1]], 0)], 0.0)
    got = M.decode(F.unpack_nibbles(out["row_codes"][: off[-1]]), out["row_scales"][: off[-1]])
    e = np.repeat(out["row_scales"][: off[-1]].astype(np.int64) - 127, 32, axis=1)
    assert np.all(np.abs(got - rows) <= np.ldexp(1.0, e))       # within one step of 2^e (steps <= 2)
    # padding rows: zero codes, scale byte 127
    pad = src[: off[-1]] < 0
    assert np.all(out["row_codes"][: off[-1]][pad] == 0) and np.all(out["row_scales"][: off[-1]][pad] == 127)
    # each expert's columnwise block count
    for e_ in range(5):
        assert (off[e_ + 1] - off[e_]) % 32 == 0


def test_receive_needs_a_32_alignment():
    w = workloads.small_dispatch(7, 10, 64, 3, 1)
    with pytest.raises(ValueError):
        M.direct_receive(nvfp4.pack_rows(w.x_bits), 64, w.topk_idx, 3, 16)


def test_receive_columnwise_inverts_to_the_grouped_rows():
    """Each expert's columnwise operand, decoded and inverse-transformed ((1/4) D H16 is
    the inverse of (1/4) H16 D), gives back the expert's grouped rows to within the
    quantization error: the layout (offsets, [H, P_e] order, 32-row scale blocks) and
    the transform are the ones R23 states."""
    w = workloads.small_dispatch(8, 90, 64, 4, 2, alignment=32, empty=[1])
    packed = nvfp4.pack_rows(w.x_bits)
    out = M.direct_receive(packed, 64, w.topk_idx, 4, 32)
    off = out["offsets"].astype(np.int64)
    src = out["src_row"].astype(np.int64)
    exact = nvfp4.decode_exact(packed, 64)
    H16 = np.array([[1.0]])
    for _ in range(4):
        H16 = np.block([[H16, H16], [H16, -H16]])
    d = rht.signs()
    for e in range(4):
        p = int(off[e + 1] - off[e])
        if p == 0:
            continue
        codes = F.unpack_nibbles(out["col_codes"][64 * off[e] // 2 : 64 * off[e + 1] // 2].reshape(64, p // 2))
        scales = out["col_scales"][64 * off[e] // 32 : 64 * off[e + 1] // 32].reshape(64, p // 32)
        y = M.decode(codes, scales)                                  # [H, P_e]
        back = np.zeros((p, 64))
        for b in range(p // 16):
            back[16 * b : 16 * b + 16] = ((d[:, None] * (H16 @ y[:, 16 * b : 16 * b + 16].T)) / 4.0)
        rows = np.where(src[off[e] : off[e + 1], None] >= 0, exact[np.maximum(src[off[e] : off[e + 1]], 0)], 0.0)
        # the inverse is orthonormal (rows of (1/4) D H16 have unit norm): the error of each
        # 16-row block is at most the norm of its quantization errors, 1 step of 2^e each
        err = np.linalg.norm((back - rows).reshape(p // 16, 16, 64), axis=1)
        bound = np.linalg.norm(np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1).T
                               .reshape(p // 16, 16, 64), axis=1)
        assert np.all(err <= bound + 1e-12)
        assert np.max(np.abs(back - rows)) < 0.5 * np.max(np.abs(rows)) + 1e-12
