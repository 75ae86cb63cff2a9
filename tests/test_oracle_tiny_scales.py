"""Pins for the columnwise block quantizers where FP32 runs out of range (CPU).

The block scales and codes of the direct receive's columnwise operand (R16, a
power-of-two decode scale D_e) and of the FC1-gradient operands (R19/R20, any
float32 D) are checked here against integer arithmetic that has no rounding of
its own (``exact_rounding``), exhaustively over every float32 subnormal block
maximum and on samples of the tiny normal range, for decode scales from 2^-140
up.  That is the corner where fl32(a / 6) itself is subnormal, so the two rules
differ there by construction:

* R16: s = E4M3 of the exact a / (6 * D_e) -- one rounding, the same rule the
  pack uses for its block scales (R5);
* R19/R20: s = E4M3(fl32(fl32(a / 6) / D)) with IEEE binary32 gradual
  underflow -- the two roundings as written.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import receive as orecv

import exact_rounding as X


def _all_subnormals():
    return np.arange(1, 1 << 23, dtype=np.uint32).view(np.float32)


def _tiny_normals(n, seed, top=-118):
    """n random float32 values in [2^-126, 2^top)."""
    rng = np.random.default_rng(seed)
    lo = np.float32(2.0 ** -126).view(np.uint32)
    hi = np.float32(2.0 ** top).view(np.uint32)
    return rng.integers(lo, hi, size=n, dtype=np.uint32).view(np.float32)


def _f32(x):
    return np.float32(x)


@pytest.mark.parametrize("d,stride", [(-140, 1), (-131, 1), (-137, 7), (-134, 7), (-127, 7), (-122, 7), (-119, 7)])
def test_pow2_scale_exact_quotient_subnormal_maxima(d, stride):
    """R16 over every float32 subnormal block max a (every 5th for some D_e) and
    D_e = 2^d: the oracle's scale code equals E4M3 round-to-nearest-even of the
    exact a / (6 * 2^d).  (From d = -116 on, no subnormal a gets a nonzero scale.)"""
    a = _all_subnormals()[::stride]
    ours = orecv.block_scale_codes(a, _f32(2.0 ** d), "pow2")
    N, q = X.f32_parts(a)
    want = X.e4m3_rne(N, q - d, 6)
    np.testing.assert_array_equal(ours, want)
    assert (want > 0).any()


@pytest.mark.parametrize("d", [-135, -128, -121, -113, -100, 0, 20])
def test_pow2_scale_exact_quotient_normal_maxima(d):
    a = np.concatenate([_tiny_normals(1 << 21, 300 + d), _tiny_normals(1 << 18, 500 + d, top=100)])
    ours = orecv.block_scale_codes(a, _f32(2.0 ** d), "pow2")
    N, q = X.f32_parts(a)
    np.testing.assert_array_equal(ours, X.e4m3_rne(N, q - d, 6))


def _fp32_scale_exact(a, D):
    """E4M3(fl32(fl32(a / 6) / D)) with every fl32 an exact IEEE binary32 rounding."""
    N, q = X.f32_parts(a)
    Q1, k1 = X.round_rne(N, q, 6, 24, -126)                 # fl32(a / 6), gradual underflow
    Dn, dq = X.f32_parts(np.full(a.shape, D, dtype=np.float32))
    Q2, k2 = X.round_rne(Q1, k1 - dq, Dn, 24, -126)         # fl32(that / D)
    return X.e4m3_rne(Q2, k2, 1)


@pytest.mark.parametrize("D,stride", [(2.0 ** -131 * 1.7, 1), (2.0 ** -140 * 3, 7), (2.0 ** -127 * 1.9921875, 7),
                                      (2.0 ** -124 * 1.3, 7), (2.0 ** -119 * 1.0000001, 7)])
def test_fp32_scale_two_ieee_roundings_subnormal_maxima(D, stride):
    """R19/R20 over every float32 subnormal block max (every 5th for some D): the
    oracle's scale code is E4M3 of fl32(fl32(a / 6) / D), each fl32 an IEEE
    binary32 rounding with gradual underflow (subnormal D included)."""
    a = _all_subnormals()[::stride]
    D = _f32(D)
    np.testing.assert_array_equal(orecv.block_scale_codes(a, D, "fp32"), _fp32_scale_exact(a, D))


def test_fp32_scale_two_ieee_roundings_normal_maxima():
    rng = np.random.default_rng(7)
    for D in (2.0 ** -130 * 1.25, 2.0 ** -120 * 1.7, 2.0 ** -100 * 1.1, 1.0 / 2688.0, 3.3):
        D = _f32(D * (1 + rng.random() * 1e-3))
        a = np.concatenate([_tiny_normals(1 << 19, int(rng.integers(1 << 30))),
                            _tiny_normals(1 << 17, int(rng.integers(1 << 30)), top=20)])
        np.testing.assert_array_equal(orecv.block_scale_codes(a, D, "fp32"), _fp32_scale_exact(a, D))


def test_the_two_rules_differ_only_where_a_over_6_is_subnormal():
    """The corner that tells the readings apart exists, and only there: with D a
    power of two, the single- and double-rounding rules agree whenever
    fl32(a / 6) is a normal float."""
    a = _all_subnormals()[::2]
    D = _f32(2.0 ** -135)
    one = orecv.block_scale_codes(a, D, "pow2")
    two = orecv.block_scale_codes(a, D, "fp32")
    assert (one != two).sum() > 100
    b = _tiny_normals(1 << 20, 3, top=-100)
    b = b[b.astype(np.float64) / 6.0 >= 2.0 ** -126]
    np.testing.assert_array_equal(orecv.block_scale_codes(b, D, "pow2"), orecv.block_scale_codes(b, D, "fp32"))


def _blocks_of(y):
    """Each value as a block of its own (the code rule broadcasts a block's scale
    over its last axis, whatever its length)."""
    return np.asarray(y, dtype=np.float32)[:, None]


@pytest.mark.parametrize("sc,d", [(0x01, -140), (0x07, -138), (0x08, -135), (0x3B, -131), (0x55, -135),
                                  (0x7E, -140), (0x2F, -142)])
def test_pow2_codes_exact_quotient_subnormal_values(sc, d):
    """R16 codes for every float32 subnormal value (both signs) with a tiny s * D_e:
    the E2M1 index of the exact |y| / (s * 2^d), the sign bit kept."""
    y = _all_subnormals()[::3]
    y = np.concatenate([y, -y])
    codes = orecv.block_codes(_blocks_of(y), np.full(y.shape[0], sc, np.uint8), _f32(2.0 ** d), "pow2")[:, 0]
    N, q = X.f32_parts(np.abs(y))
    s_num, s_q = X.f32_parts(np.float32(F.e4m3_decode(np.uint8(sc))))
    idx = X.e2m1_rne_index(N, q - s_q - d, s_num)
    np.testing.assert_array_equal(codes & 7, idx)
    np.testing.assert_array_equal(codes >> 3, (y.view(np.uint32) >> 31).astype(np.uint8))
    assert len(np.unique(idx)) > 2


@pytest.mark.parametrize("sc,D", [(0x01, 2.0 ** -140 * 3), (0x30, 2.0 ** -133 * 1.7), (0x3B, 2.0 ** -129 * 1.3),
                                  (0x55, 2.0 ** -137 * 1.9921875), (0x7E, 2.0 ** -136 * 1.1), (0x20, 2.0 ** -139 * 1.5)])
def test_fp32_codes_two_ieee_roundings_subnormal_values(sc, D):
    """R19/R20 codes for every float32 subnormal value: c = fl32(s * D) (IEEE,
    possibly subnormal), v = fl32(|y| / c), the E2M1 index of v."""
    y = _all_subnormals()[::3]
    D = _f32(D)
    codes = orecv.block_codes(_blocks_of(y), np.full(y.shape[0], sc, np.uint8), D, "fp32")[:, 0]
    s_num, s_q = X.f32_parts(np.float32(F.e4m3_decode(np.uint8(sc))))
    Dn, dq = X.f32_parts(D)
    Qc, kc = X.round_rne(np.int64(s_num) * Dn, s_q + dq, 1, 24, -126)     # fl32(s * D)
    if Qc == 0:
        np.testing.assert_array_equal(codes & 7, 0)
        return
    N, q = X.f32_parts(y)
    Qv, kv = X.round_rne(N, q - kc, Qc, 24, -126)                         # fl32(|y| / c)
    idx = X.e2m1_rne_index(Qv, kv, 1)
    np.testing.assert_array_equal(codes & 7, idx)
    assert len(np.unique(idx)) > 2


def test_exact_rounding_helper_against_fractions():
    """The integer helper itself, against Python's exact rationals on random cases."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    N = rng.integers(1, 1 << 40, size=400)
    M = rng.integers(1, 1 << 30, size=400)
    q = rng.integers(-180, 40, size=400)
    for P, emin in ((24, -126), (4, -6), (2, 0)):
        Q, k = X.round_rne(N, q, M, P, emin)
        for i in range(0, 400, 7):
            r = Fraction(int(N[i]) * 2 ** int(max(q[i], 0)), int(M[i]) * 2 ** int(max(-q[i], 0)))
            kk = int(k[i])
            unit = Fraction(2) ** kk
            lo = (r / unit).numerator // (r / unit).denominator
            rem = r / unit - lo
            want = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else 0)
            if int(Q[i]) == 0:
                assert r < Fraction(2) ** (emin - P + 1) / 2 * 2 or want == 0
            else:
                assert int(Q[i]) == want, (P, i)
                assert Fraction(2) ** (P - 1) <= Q[i] or kk == emin - P + 1
