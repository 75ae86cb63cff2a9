"""Pins for the oracle's NVFP4 row pack / unpack / stochastic rounding (CPU)."""

import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import nvfp4
from oracle.philox import sr_word


def _all_bf16_pos():
    b = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)     # positive finite, non-zero
    return F.bf16_to_f32(b).astype(np.float64)


def test_token_scale_exhaustive():
    """R4 over every positive finite BF16 amax: bound, minimality, and the closed form
    e = E - 11 + [m > 1.3125] with amax = m * 2^E, m in [1, 2)."""
    a = _all_bf16_pos()
    e = nvfp4.token_scale_exponent(a)
    t = np.ldexp(1.0, e)
    assert np.all(a <= 2688.0 * t)
    assert np.all(a > 1344.0 * t)
    m, E = np.frexp(a)
    m, E = m * 2, E - 1
    np.testing.assert_array_equal(e, E - 11 + (m > 1.3125))
    assert np.all(np.isfinite(t.astype(np.float32))) and np.all(t.astype(np.float32) > 0)
    assert nvfp4.token_scale_exponent(np.array([0.0]))[0] == 0


def _check_block_bound(x_bits, packed, h):
    """Decode-error bound per element: |x - x_hat| <= s*t * step(v)/2 for v <= 6,
    and = (v - 6) * s * t when saturated, with v = |x| / (s*t)."""
    x = F.bf16_to_f32(x_bits).astype(np.float64)
    codes, s_code, t = nvfp4.split_rows(packed, h)
    st = np.repeat(F.e4m3_decode(s_code), 16, axis=1) * t[:, None]
    xh = nvfp4.decode_exact(packed, h)
    err = np.abs(x - xh)
    pos = st > 0
    v = np.where(pos, np.abs(x) / np.where(pos, st, 1), 0)
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    bound = np.where(v <= 6, st * step / 2, (v - 6) * st)
    assert np.all(err[pos] <= bound[pos] * (1 + 1e-12))
    # blocks whose scale flushes to zero are exactly those with a_b / (6 t) <= 2^-10
    # (the tie at 2^-10 rounds to the even code 0); compared without division
    a_b = np.abs(F.bf16_to_f32(x_bits)).reshape(x.shape[0], h // 16, 16).max(axis=2).astype(np.float64)
    np.testing.assert_array_equal(s_code == 0, a_b <= 6.0 * t[:, None] * 2.0 ** -10)
    # flushed blocks decode to (signed) zero
    assert np.all(xh[~pos] == 0)
    # the largest block scale of each non-zero row lies in (224, 448]
    s_val = F.e4m3_decode(s_code)
    nz = np.abs(x).max(axis=1) > 0
    smax = s_val.max(axis=1)[nz]
    assert np.all((smax > 224 * (1 - 1 / 16)) & (smax <= 448))


def test_pack_bounds_config1():
    w = workloads.config1()
    packed = nvfp4.pack_rows(w.x_bits)
    assert packed.shape == (256, 512 + 64 + 4)           # 512 B codes, 64 scales, one FP32 scale
    _check_block_bound(w.x_bits, packed, 1024)


def test_pack_bounds_wide_range():
    w = workloads.small_dispatch(5, 300, 320, 4, 1)
    x = F.bf16_to_f32(w.x_bits).astype(np.float64)
    rng = np.random.default_rng(9)
    x *= 10.0 ** rng.uniform(-30, 30, size=(x.shape[0], 1))
    x[0] = 0.0
    x[1, :16] = 0.0
    x[2] *= 1e-10
    bits = F.f32_to_bf16(x.astype(np.float32))
    _check_block_bound(bits, nvfp4.pack_rows(bits), 320)


def test_tiny_rows_brute_force():
    """H = 64: given the scales, every code is the nearest of the 16 candidates
    (ties to the even magnitude index) -- brute force over all candidates."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((500, 64)) * 10.0 ** rng.uniform(-3, 3, size=(500, 1))
    bits = F.f32_to_bf16(x.astype(np.float32))
    packed = nvfp4.pack_rows(bits)
    codes, s_code, t = nvfp4.split_rows(packed, 64)
    st = np.repeat(F.e4m3_decode(s_code), 16, axis=1) * t[:, None]
    xv = F.bf16_to_f32(bits).astype(np.float64)
    for r in range(500):
        for c in range(64):
            cand = [(abs(abs(xv[r, c]) - g * st[r, c]), i) for i, g in enumerate(F.E2M1_GRID)]
            best = min(d for d, _ in cand)
            allowed = [i for d, i in cand if d == best]
            pick = [i for i in allowed if i % 2 == 0] if len(allowed) > 1 else allowed
            if st[r, c] == 0:
                pick = [0]
            assert (codes[r, c] & 7) == pick[0], (r, c)
            assert (codes[r, c] >> 3) == (bits[r, c] >> 15)


def test_unpack_identity_on_grid_values():
    """R10: rows already on the NVFP4 grid (x = g * s * t) survive pack -> unpack exactly."""
    rng = np.random.default_rng(6)
    h = 128
    rows = []
    for r in range(64):
        e = int(rng.integers(-20, 20))
        t = 2.0 ** e
        s = F.E4M3_VALUES[rng.integers(8, 127, size=h // 16)]
        s[0] = 448.0                                   # pins t: the row max is 6 * 448 * t
        g = F.E2M1_GRID[rng.integers(0, 8, size=h)] * np.where(rng.random(h) < 0.5, -1, 1)
        g[0] = 6.0
        g.reshape(-1, 16)[:, 1] = 6.0                  # each block's max is 6 * s: pins s
        rows.append(g * np.repeat(s, 16) * t)
    x = np.array(rows)
    bits = F.f32_to_bf16(x.astype(np.float32))
    assert np.array_equal(F.bf16_to_f32(bits).astype(np.float64), x)
    out = nvfp4.unpack_rows(nvfp4.pack_rows(bits), h)
    np.testing.assert_array_equal(out, bits)


def test_signed_zero_and_zero_rows():
    bits = np.zeros((3, 64), dtype=np.uint16)
    bits[1, 0] = 0x8000                                # -0
    bits[2, 0] = F.f32_to_bf16(np.float32(-1e-3))      # rounds to zero in a block with a large max
    bits[2, 1] = F.f32_to_bf16(np.float32(100.0))
    packed = nvfp4.pack_rows(bits)
    codes, s_code, t = nvfp4.split_rows(packed, 64)
    assert t[0] == 1.0 and np.all(s_code[0] == 0) and np.all(codes[0] == 0)
    assert codes[1, 0] == 8
    assert codes[2, 0] == 8


def test_unpack_src_row_gather():
    w = workloads.small_dispatch(7, 40, 128, 4, 2)
    packed = nvfp4.pack_rows(w.x_bits)
    src = np.array([3, -1, 0, 39, 3], dtype=np.int32)
    out = nvfp4.unpack_rows(packed, 128, src)
    full = nvfp4.unpack_rows(packed, 128)
    np.testing.assert_array_equal(out[0], full[3])
    assert np.all(out[1] == 0)
    np.testing.assert_array_equal(out[3], full[39])


# ------------------------------------------------------------------ stochastic rounding
def test_sr_on_grid_values_never_move():
    rng = np.random.default_rng(8)
    h = 64
    g = F.E2M1_GRID[rng.integers(0, 8, size=(32, h))]
    g[:, 0] = 6.0
    g.reshape(32, -1, 16)[:, :, 1] = 6.0
    x = g * 448.0 * 2.0 ** -3
    bits = F.f32_to_bf16(x.astype(np.float32))
    a = nvfp4.pack_rows(bits)
    b = nvfp4.pack_rows(bits, sr_seed=99)
    np.testing.assert_array_equal(a, b)


def test_sr_matches_rne_scales_and_layout():
    w = workloads.small_dispatch(11, 64, 256, 4, 1)
    a = nvfp4.pack_rows(w.x_bits)
    b = nvfp4.pack_rows(w.x_bits, sr_seed=1234)
    np.testing.assert_array_equal(a[:, 128:], b[:, 128:])          # scales and t are deterministic


def test_sr_unbiased_1e6_draws():
    """Each value v inside every grid interval, 10^6 distinct counters: the mean of the
    stochastically rounded value is v within 5 standard errors."""
    vals = []
    for lo, hi in zip(F.E2M1_GRID[:-1], F.E2M1_GRID[1:]):
        vals += [lo + (hi - lo) * f for f in (0.125, 0.5, 0.8125)]
    vals = np.array(vals, dtype=np.float32)
    n = 1_000_000
    for j, v in enumerate(vals):
        pos = np.arange(n, dtype=np.uint64) + np.uint64(j * n)
        r = (sr_word(pos, 1234, "element") >> np.uint32(8)).astype(np.float64)
        idx = nvfp4.stochastic_e2m1_index(np.full(n, v), r)
        q = F.E2M1_GRID[idx]
        lo = F.E2M1_GRID[np.searchsorted(F.E2M1_GRID, v, side="right") - 1]
        hi = F.E2M1_GRID[np.searchsorted(F.E2M1_GRID, v, side="right")]
        p = (v - lo) / (hi - lo)
        se = (hi - lo) * np.sqrt(p * (1 - p) / n)
        assert abs(q.mean() - v) < 5 * se, (v, q.mean())
        assert set(np.unique(q)) <= {lo, hi}


def test_sr_random_bits_uniform():
    """Chi-square over the top 8 bits of r for 10^6 consecutive counters."""
    n = 1_000_000
    r = sr_word(np.arange(n, dtype=np.uint64), 1234, "element") >> np.uint32(24)
    counts = np.bincount(r.astype(np.int64), minlength=256)
    chi2 = ((counts - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 400                                   # dof 255: p < 1e-7 beyond this


def test_sr_probability_rule():
    """R8: with r uniform over [0, 2^24), P(up) = ceil(frac * 2^24) / 2^24 -- checked on
    all 2^24 values of r for a few fractions."""
    r = np.arange(2 ** 24, dtype=np.float64)
    for v in (0.1, 0.5 + 2.0 ** -25, 1.75, 2.0 + 3 * 2.0 ** -22, 5.999999):
        v32 = np.float32(v)
        idx = nvfp4.stochastic_e2m1_index(np.full(r.shape, v32), r)
        lo = np.searchsorted(F.E2M1_GRID, float(v32), side="right") - 1
        frac = (float(v32) - F.E2M1_GRID[lo]) / (F.E2M1_GRID[lo + 1] - F.E2M1_GRID[lo])
        assert (idx == lo + 1).sum() == np.ceil(frac * 2 ** 24)


def test_sr_word_positions():
    """The counter of element (row, col) is counter_base + row * H + col."""
    w = workloads.small_dispatch(12, 8, 64, 2, 1)
    base = 1000
    a = nvfp4.pack_rows(w.x_bits, sr_seed=5, sr_counter_base=base)
    b = nvfp4.pack_rows(w.x_bits[1:], sr_seed=5, sr_counter_base=base + 64)
    np.testing.assert_array_equal(a[1:], b)


# ------------------------------------------------------------------ stochastic rounding, carry rule (R8b)
def test_sr_carry_on_grid_values_never_move():
    rng = np.random.default_rng(18)
    g = F.E2M1_GRID[rng.integers(0, 8, size=(16, 64))]
    g.reshape(16, -1, 16)[:, :, 3] = 6.0         # every block holds a 6: its values sit on the grid
    bits = F.f32_to_bf16((g * 448.0 * 2.0 ** -5).astype(np.float32))
    np.testing.assert_array_equal(nvfp4.pack_rows(bits), nvfp4.pack_rows(bits, sr_seed=7, sr_rule="carry"))


def test_sr_carry_matches_exact_rationals():
    """R8b against exact rational arithmetic: up iff frac + w / 2^32 >= 1, frac the exact
    position of v between its grid neighbours (Python fractions, no floating point)."""
    from fractions import Fraction
    rng = np.random.default_rng(19)
    v = rng.uniform(0, 6.5, 4000).astype(np.float32)
    v[:50] = np.float32(2.0) ** -rng.integers(10, 140, 50).astype(np.float32)   # tiny values
    w = rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32)
    idx = nvfp4.stochastic_e2m1_index_carry(v.astype(np.float64), w)
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for vi, wi, got in zip(v, w, idx):
        fv = Fraction(float(vi))
        if fv >= 6:
            assert got == 7
            continue
        lo = max(i for i in range(7) if grid[i] <= fv)
        frac = (fv - grid[lo]) / (grid[lo + 1] - grid[lo])
        want = lo + 1 if frac + Fraction(int(wi), 2 ** 32) >= 1 else lo
        assert got == want, (float(vi), int(wi))


def test_sr_carry_boundary_words():
    """For each v the words that round up are exactly [2^32 - D, 2^32), D = floor(frac 2^32):
    P(up) = D / 2^32, so the bias is below 2^-32 of a grid step."""
    from fractions import Fraction
    rng = np.random.default_rng(20)
    v = rng.uniform(0, 6, 500).astype(np.float32)
    grid = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for vi in v:
        fv = Fraction(float(vi))
        lo = max(i for i in range(7) if grid[i] <= fv)
        d = int((fv - grid[lo]) / (grid[lo + 1] - grid[lo]) * 2 ** 32)
        if d == 0:
            continue
        ws = np.array([2 ** 32 - d - 1, 2 ** 32 - d, 2 ** 32 - 1, 0], dtype=np.uint32)
        got = nvfp4.stochastic_e2m1_index_carry(np.full(4, float(vi)), ws)
        np.testing.assert_array_equal(got, [lo, lo + 1, lo + 1, lo if d < 2 ** 32 else lo + 1])


def test_sr_carry_unbiased_1e6_draws():
    vals = []
    for lo, hi in zip(F.E2M1_GRID[:-1], F.E2M1_GRID[1:]):
        vals += [lo + (hi - lo) * f for f in (0.0625, 0.5, 0.9375)]
    n = 1_000_000
    for j, v in enumerate(np.array(vals, dtype=np.float32)):
        w = sr_word(np.arange(n, dtype=np.uint64) + np.uint64(j * n), 1234, "element")
        q = F.E2M1_GRID[nvfp4.stochastic_e2m1_index_carry(np.full(n, v, dtype=np.float64), w)]
        lo = F.E2M1_GRID[np.searchsorted(F.E2M1_GRID, v, side="right") - 1]
        hi = F.E2M1_GRID[np.searchsorted(F.E2M1_GRID, v, side="right")]
        p = (v - lo) / (hi - lo)
        assert abs(q.mean() - v) < 5 * (hi - lo) * np.sqrt(p * (1 - p) / n), (v, q.mean())
        assert set(np.unique(q)) <= {lo, hi}


def test_sr_carry_scales_and_positions():
    """Scales and t are the deterministic ones; the counter of (row, col) is base + row*H + col."""
    w = workloads.small_dispatch(13, 8, 128, 2, 1)
    a = nvfp4.pack_rows(w.x_bits, sr_seed=5, sr_counter_base=300, sr_rule="carry")
    b = nvfp4.pack_rows(w.x_bits[2:], sr_seed=5, sr_counter_base=300 + 2 * 128, sr_rule="carry")
    np.testing.assert_array_equal(a[2:], b)
    np.testing.assert_array_equal(a[:, 64:], nvfp4.pack_rows(w.x_bits)[:, 64:])


def test_block_scale_exact_rounding_exhaustive():
    """R5: the E4M3 block scale of a_b / (6 * 2^e) for every positive finite BF16 a_b
    and e in [-24, 24] equals torch's E4M3 cast of the float32-rounded quotient (the
    quotient by 6 never lands on an E4M3 tie unless exact, so one rounding or two
    agree) -- an independent library route to the same codes."""
    import torch
    a = _all_bf16_pos()
    for e in range(-24, 25):
        y = a / (6.0 * 2.0 ** e)
        keep = y <= 448.0
        ours = F.e4m3_encode(y[keep])
        ref = torch.from_numpy(y[keep].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(ours, ref)
