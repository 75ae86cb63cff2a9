"""Pins for the oracle's number formats (CPU).  Each check compares against a
library cast, a published table or an exhaustive exact computation."""

import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_bf16_finite():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


def test_golden_points():
    """OCP table points (tests/golden/ocp_fp8_fp4_points.txt)."""
    for line in open(os.path.join(GOLDEN, "ocp_fp8_fp4_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        fmt, code, val = line.split()
        code, val = int(code, 16), float(val)
        if fmt == "e2m1":
            got = F.e2m1_value(code)
        elif fmt == "e4m3":
            got = F.e4m3_decode(code)
        else:
            got = F.e8m0_decode(code)
        assert float(got) == val and np.signbit(got) == np.signbit(val), (fmt, code)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000),
        rng.random(100000).astype(np.float32) * np.float32(1e-38),            # subnormal territory
        (np.arange(1, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32),  # exact ties
    ]).astype(np.float32)
    ours = F.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    b = _all_bf16_finite()
    np.testing.assert_array_equal(F.f32_to_bf16(F.bf16_to_f32(b)), b)


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(codes)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(np.signbit(ours), np.signbit(ref))


def test_e4m3_encode_matches_torch():
    """Library pin: torch's float8_e4m3fn cast (round-to-nearest-even) of min(y, 448)."""
    rng = np.random.default_rng(2)
    b = _all_bf16_finite()
    y_bf = np.abs(F.bf16_to_f32(b))
    mids = (F.E4M3_VALUES[:-1] + F.E4M3_VALUES[1:]) / 2.0            # every tie point
    y = np.concatenate([
        y_bf,
        rng.random(1_000_000).astype(np.float32) * np.float32(500.0),
        rng.random(200_000).astype(np.float32) * np.float32(0.02),
        mids.astype(np.float32),
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(0)),
    ]).astype(np.float32)
    ours = F.e4m3_encode(y.astype(np.float64))
    clamped = np.minimum(y, np.float32(448.0))
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def _e2m1_threshold_count(v):
    """Independent closed form of R2: count the tie thresholds crossed; a tie
    counts as crossed exactly when the upper neighbour has the even index."""
    v = np.asarray(v, dtype=np.float64)
    return ((v > 0.25).astype(int) + (v >= 0.75) + (v > 1.25) + (v >= 1.75)
            + (v > 2.5) + (v >= 3.5) + (v > 5.0)).astype(np.uint8)


def test_e2m1_index_matches_threshold_form():
    rng = np.random.default_rng(3)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    near = np.concatenate([np.nextafter(ties, np.float32(0)), ties, np.nextafter(ties, np.float32(9))])
    grid = F.E2M1_GRID.astype(np.float32)
    v = np.concatenate([
        near, grid, np.abs(F.bf16_to_f32(_all_bf16_finite())),
        rng.random(1_000_000).astype(np.float32) * np.float32(8.0),
        np.array([6.5, 1e30, 0.0, 1e-45], dtype=np.float32),
    ]).astype(np.float32)
    np.testing.assert_array_equal(F.e2m1_index(v), _e2m1_threshold_count(v))
    # the tie directions spelled out in R2
    np.testing.assert_array_equal(F.e2m1_index(ties), [0, 2, 2, 4, 4, 6, 6])


def test_e2m1_quotient_exhaustive_bf16_by_e4m3():
    """R6: for every positive finite BF16 x and every positive finite E4M3 scale s,
    the oracle's float64 quotient route (and the float32 quotient) decides the
    E2M1 index exactly as the exact comparison |x| vs tie * s does."""
    b = _all_bf16_finite()
    x = np.abs(F.bf16_to_f32(b)).astype(np.float64)
    x = np.unique(x)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for s in F.E4M3_VALUES[1:]:                      # 126 positive finite scales
        q = x / s
        ours = F.e2m1_index(q)
        with np.errstate(over="ignore"):
            q32 = (x.astype(np.float32) / np.float32(s)).astype(np.float64)
        fin = np.isfinite(q32)                        # float32 overflow only where the index saturates
        ours32 = np.where(fin, F.e2m1_index(np.where(fin, q32, 0.0)), 7).astype(np.uint8)
        # exact: tie*s is exact in float64 and x is exact, so comparisons are exact
        thr = ties * s
        exact = ((x > thr[0]).astype(int) + (x >= thr[1]) + (x > thr[2]) + (x >= thr[3])
                 + (x > thr[4]) + (x >= thr[5]) + (x > thr[6])).astype(np.uint8)
        np.testing.assert_array_equal(ours, exact)
        np.testing.assert_array_equal(ours32, exact)


def test_nibble_order():
    codes = np.array([[1, 2, 3, 4, 0xF, 0x8]], dtype=np.uint8)
    packed = F.pack_nibbles(codes)
    np.testing.assert_array_equal(packed, [[0x21, 0x43, 0x8F]])
    np.testing.assert_array_equal(F.unpack_nibbles(packed), codes)
