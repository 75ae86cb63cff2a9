"""Pins for the oracle's MXFP8 pack, routing plan and 16-point RHT (CPU)."""

import numpy as np
import pytest
import scipy.linalg
import torch

import workloads
from oracle import formats as F
from oracle import mxfp8, rht
from oracle.routing import route_plan, capacity


# ------------------------------------------------------------------ MXFP8
def test_mxfp8_scale_exponent_exhaustive():
    """R11 over every positive finite BF16 amax: bound, minimality, closed form
    e = E - 8 + [m > 1.75] (amax = m * 2^E, m in [1, 2)), clamp to [-127, 127]."""
    b = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)
    a = F.bf16_to_f32(b).astype(np.float64)
    e = mxfp8.scale_exponent(a)
    m, E = np.frexp(a)
    m, E = m * 2, E - 1
    closed = np.clip(E - 8 + (m > 1.75), -127, 127)
    np.testing.assert_array_equal(e, closed)
    un = closed > -127
    assert np.all(a <= 448.0 * np.ldexp(1.0, e))
    assert np.all(a[un] > 224.0 * np.ldexp(1.0, e[un]))


def test_mxfp8_data_matches_torch_cast():
    """Library pin: data = torch float8_e4m3fn cast of x / 2^e (exact scaling)."""
    w = workloads.small_dispatch(21, 256, 512, 4, 1)
    x = F.bf16_to_f32(w.x_bits).astype(np.float64)
    x[3, :32] = 0.0
    x[4, :32] *= 1e-36
    bits = F.f32_to_bf16(x.astype(np.float32))
    data, scales = mxfp8.pack_rows(bits)
    xv = F.bf16_to_f32(bits).astype(np.float64)
    scale = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    ref = torch.from_numpy((xv / scale).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(data, ref)
    assert np.all(scales[3, 0] == 127)
    # no element saturates and every block's max lies in (224, 448] (unless clamped / zero)
    blk = np.abs(mxfp8.decode(data, scales)).reshape(256, -1, 32).max(axis=2) / np.ldexp(1.0, scales.astype(np.int64) - 127)
    nz = np.abs(xv).reshape(256, -1, 32).max(axis=2) > 0
    assert np.all(blk[nz] <= 448)


# ------------------------------------------------------------------ routing
def _brute_plan(topk, E, A, r_cap):
    T, k = topk.shape
    lists = {e: [] for e in range(E)}
    err = False
    for t in range(T):
        for j in range(k):
            v = int(topk[t, j])
            if v == -1:
                continue
            if not 0 <= v < E:
                err = True
                continue
            lists[v].append((t, j))
    counts = [len(lists[e]) for e in range(E)]
    off = [0]
    for e in range(E):
        off.append(off[-1] + -(-counts[e] // A) * A)
    dst = -np.ones((T, k), dtype=np.int64)
    src = -np.ones(r_cap, dtype=np.int64)
    for e in range(E):
        for r, (t, j) in enumerate(lists[e]):
            dst[t, j] = off[e] + r
            src[off[e] + r] = t
    return counts, off, dst, src, err


@pytest.mark.parametrize("A", [16, 128, 256])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_plan_brute_force(A, seed):
    rng = np.random.default_rng(seed)
    T, k, E = 97, 3, 6
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    topk[rng.random((T, k)) < 0.1] = -1
    topk[topk == 4] = -1                                   # expert 4 empty
    if seed == 2:
        topk[5, 0] = 9                                     # invalid id -> error, dropped
        topk[6, 1] = -7
    r_cap = capacity(T, k, E, A)
    plan = route_plan(topk, E, A)
    counts, off, dst, src, err = _brute_plan(topk, E, A, r_cap)
    np.testing.assert_array_equal(plan["counts"], counts)
    np.testing.assert_array_equal(plan["offsets"], off)
    np.testing.assert_array_equal(plan["dst_row"], dst)
    np.testing.assert_array_equal(plan["src_row"], src)
    assert plan["error"] == err
    assert np.all(np.asarray(off) % A == 0) and off[-1] <= r_cap


@pytest.mark.parametrize("A", [32, 128])
def test_mxfp8_grouped_receive_brute_force(A):
    """P2, description and "Changes": the per-expert grouped receive holds each
    expert's rows back to back in data-then-scale regions, slots padded to the
    alignment.  Walked row by row from a brute-force plan: grouped row g holds
    the data and scale bytes of its token, padding rows and every row from off_E
    to r_cap are zero bytes, and the expert's rows appear in token order."""
    rng = np.random.default_rng(A)
    T, k, E, H = 61, 2, 5, 96
    x = rng.standard_normal((T, H)) * 10.0 ** rng.uniform(-3, 3, (T, 1))
    data, scales = mxfp8.pack_rows(F.f32_to_bf16(x.astype(np.float32)))
    topk = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    topk[topk == 3] = -1                                   # expert 3 empty
    r_cap = capacity(T, k, E, A)
    counts, off, dst, src, _ = _brute_plan(topk, E, A, r_cap)
    gd, gs = mxfp8.grouped_receive(data, scales, src)
    assert gd.shape == (r_cap, H) and gs.shape == (r_cap, H // 32)
    for g in range(r_cap):
        e = next((e for e in range(E) if off[e] <= g < off[e + 1]), None)
        if e is not None and g - off[e] < counts[e]:
            toks = sorted({t for t in range(T) for j in range(k) if topk[t, j] == e})
            t = toks[g - off[e]]
            assert bytes(gd[g]) == bytes(data[t]) and bytes(gs[g]) == bytes(scales[t]), g
        else:
            assert not gd[g].any() and not gs[g].any(), g
    for t in range(T):
        for j in range(k):
            if topk[t, j] >= 0:
                assert bytes(gd[dst[t, j]]) == bytes(data[t])


def test_route_plan_config2_shape():
    w = workloads.config2()
    plan = route_plan(w.topk_idx, 8, 16)
    assert plan["counts"][7] == 0 and plan["counts"].sum() == 8192
    assert plan["src_row"].shape[0] == 8192 + 8 * 15


# ------------------------------------------------------------------ RHT
def test_sign_vector_is_not_a_walsh_row():
    d = rht.signs()
    H = scipy.linalg.hadamard(16)
    for row in H:
        assert not np.array_equal(d, row) and not np.array_equal(d, -row)
    assert rht.sign_mask() == 0xE8D5


def test_rht_equals_dense_sylvester_on_exact_inputs():
    """Inputs that are small dyadic integers: no rounding anywhere, so the butterfly
    must equal (1/4) * H16 @ (d * z) exactly, H16 = scipy.linalg.hadamard(16)."""
    rng = np.random.default_rng(1)
    z = rng.integers(-64, 64, size=(1000, 16)).astype(np.float64) * 2.0 ** rng.integers(-10, 10, size=(1000, 1))
    y = rht.rht16(z).astype(np.float64)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    ref = (z * rht.signs()) @ H.T / 4.0
    np.testing.assert_array_equal(y, ref)
    # inverse: z = (1/4) * D * H16 @ y
    back = (y @ H.T / 4.0) * rht.signs()
    np.testing.assert_array_equal(back, z)


def test_rht_bound_and_norm():
    """|y| <= 4 max|z| (the bound the pages use) holds in float32, and the transform
    preserves Euclidean norms up to float32 rounding."""
    rng = np.random.default_rng(2)
    z = (rng.standard_normal((20000, 16)) * 10.0 ** rng.uniform(-5, 5, size=(20000, 1))).astype(np.float32)
    z[0] = 1.0
    z[1] = rht.signs()                               # adversarial: every term adds up
    z[2] = -rht.signs() * 3.0
    y = rht.rht16(z)
    amax = np.abs(z).max(axis=1)
    assert np.all(np.abs(y).max(axis=1) <= 4 * amax)
    assert np.abs(y[1]).max() == 4.0
    nz = np.linalg.norm(z.astype(np.float64), axis=1)
    ny = np.linalg.norm(y.astype(np.float64), axis=1)
    np.testing.assert_allclose(ny, nz, rtol=1e-6)


def test_rht_rounding_order_is_stride_1_2_4_8():
    """A case where float32 rounding depends on the order of the butterfly stages:
    the oracle must reproduce the documented order (stride 1 first)."""
    z = np.zeros(16, dtype=np.float64)
    z[0], z[1], z[2] = 2.0 ** 26, 1.0, 1.0
    y = rht.rht16(z[None])[0]
    d = rht.signs()
    a = np.float32(0.25 * d[0] * z[0]); b = np.float32(0.25 * d[1] * z[1]); c = np.float32(0.25 * d[2] * z[2])
    # stage 1 pairs (0,1): a+b rounds; stage 2 pairs (0,2): (a+b)+c rounds again
    expect0 = np.float32(np.float32(a + b) + c)
    assert y[0] == expect0
