"""Exact round-to-nearest-even of rationals onto binary floating-point grids,
in integer arithmetic only (numpy int64, vectorized).  Test infrastructure: it
pins the oracle's float64/float32 shortcuts against arithmetic that has no
rounding of its own.

A value is handled as r = N * 2^q / M with integers N >= 0, M >= 1 and q.  A
grid with P significant bits and minimum normal exponent emin holds the
numbers Q * 2^k, Q < 2^P, with k >= emin - P + 1 (gradual underflow below
2^emin).  ``round_rne`` returns (Q, k) with r rounded to the nearest grid
point and an exact tie sent to the even Q.  Q may come out as 2^P after a
carry; the value Q * 2^k is still right.
"""

import numpy as np


def _bitlen(n):
    """Bit length of non-negative integers below 2^53 (exact through float64)."""
    n = np.asarray(n, dtype=np.int64)
    _, e = np.frexp(n.astype(np.float64))
    return np.where(n > 0, e, 0).astype(np.int64)


def floor_log2_ratio(N, M):
    """floor(log2(N / M)) for N, M >= 1 (below 2^53)."""
    N = np.asarray(N, dtype=np.int64)
    M = np.asarray(M, dtype=np.int64)
    b = _bitlen(N) - _bitlen(M)
    sh_l = np.clip(b, 0, 62)
    sh_r = np.clip(-b, 0, 62)
    ge = np.where(b >= 0, N >= (M << sh_l), (N << sh_r) >= M)
    return np.where(ge, b, b - 1)


def round_rne(N, q, M, P, emin):
    """(Q, k): N * 2^q / M rounded to nearest-even on the (P, emin) grid."""
    N, q, M = np.broadcast_arrays(np.asarray(N, dtype=np.int64), np.asarray(q, dtype=np.int64),
                                  np.asarray(M, dtype=np.int64))
    if np.any(N < 0) or np.any(M < 1):
        raise ValueError("N >= 0 and M >= 1 expected")
    if np.any(N >= 2 ** 52) or np.any(M >= 2 ** 36):
        raise ValueError("operands too wide for the int64 arithmetic here")
    kmin = emin - P + 1
    pos = N > 0
    E = q + floor_log2_ratio(np.maximum(N, 1), M)          # floor(log2 r) where r > 0
    k = np.maximum(E, emin) - (P - 1)
    tiny = ~pos | (E < kmin - 2)                            # r < 2^(kmin-2): rounds to 0
    k = np.where(tiny, kmin, k)
    s = np.where(tiny, 0, q - k)
    num = np.where(s >= 0, N << np.clip(s, 0, 62), N)
    den = np.where(s >= 0, M, M << np.clip(-s, 0, 62))
    if np.any((s >= 0) & ~tiny & ((N << np.clip(s, 0, 62)) >> np.clip(s, 0, 62) != N)):
        raise OverflowError("numerator shift overflowed")
    Q = num // den
    R = num - Q * den
    up = (2 * R > den) | ((2 * R == den) & ((Q & 1) == 1))
    Q = np.where(tiny, 0, Q + up)
    return Q.astype(np.int64), k.astype(np.int64)


def value(Q, k):
    """Q * 2^k as float64 (exact for the grids used here)."""
    return np.ldexp(np.asarray(Q, dtype=np.float64), np.asarray(k, dtype=np.int64))


def f32_parts(x):
    """Positive float32 values (or +0) -> (N, q) with x = N * 2^q, N < 2^24."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    ef = (b >> 23) & 0xFF
    man = b & 0x7FFFFF
    N = np.where(ef > 0, man | 0x800000, man)
    q = np.where(ef > 0, ef - 150, -149)
    return N, q


def e4m3_code_of(Q, k):
    """E4M3FN code of the grid value Q * 2^k produced by round_rne(P=4, emin=-6),
    saturated at 448 (code 0x7E)."""
    Q = np.asarray(Q, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    carry = Q >= 16
    Q = np.where(carry, Q >> 1, Q)
    k = np.where(carry, k + 1, k)
    normal = Q >= 8
    code = np.where(normal, ((k + 10) << 3) | (Q - 8), Q)   # k = -9 below 2^-6: code = Q
    sat = value(Q, k) >= 448.0
    return np.where(sat, 0x7E, code).astype(np.uint8)


def e4m3_rne(N, q, M):
    """E4M3 code of min(N * 2^q / M, 448), round-to-nearest-even."""
    Q, k = round_rne(N, q, M, 4, -6)
    return e4m3_code_of(Q, k)


def e2m1_rne_index(N, q, M):
    """E2M1 magnitude index of N * 2^q / M (ties to the even index, > 6 saturates)."""
    Q, k = round_rne(N, q, M, 2, 0)                          # grid 0, .5, 1, 1.5, 2, 3, 4, 6, 8, ...
    v = value(Q, k)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    idx = np.searchsorted(grid, np.minimum(v, 6.0))
    return idx.astype(np.uint8)
