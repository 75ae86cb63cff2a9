"""Pins for the oracle's direct receive and the dSwiGLU / FC1-gradient path (CPU)."""

import numpy as np
import pytest
import scipy.linalg
import torch

import workloads
from oracle import formats as F
from oracle import nvfp4, receive, rht, dswiglu
from oracle.routing import route_plan

H16 = scipy.linalg.hadamard(16).astype(np.float64)


def _dense_rht_exact(vals):
    """(1/4) H16 D applied down 16-row blocks of each column, float64 (no butterfly)."""
    p, h = vals.shape
    blocks = vals.T.reshape(h, p // 16, 16) * rht.signs()
    return blocks @ H16.T / 4.0


def _decode_col(codes_packed, scales, D):
    """Decode one expert's columnwise operand: [H, P/2] codes, [H, P/16] scales -> [H, P/16, 16]."""
    c = F.unpack_nibbles(codes_packed)
    h, p = c.shape
    return (F.e2m1_value(c).reshape(h, p // 16, 16)
            * F.e4m3_decode(scales)[..., None] * float(D))


def _check_columnwise(vals, codes, scales, D, bound_is_pow2):
    """Decoded columnwise operand vs the dense exact transform: every element within
    half a grid step at its block scale (plus float32 rounding of the butterfly), no
    block scale above 448, and every block's scale consistent with its amax."""
    y = _dense_rht_exact(vals)
    yq = _decode_col(codes, scales, D)
    s = F.e4m3_decode(scales)[..., None] * float(D)
    v = np.abs(y) / np.where(s > 0, s, 1)
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    tol = np.where(v <= 6, step / 2, v - 6) * s + 2.0 ** -21 * np.abs(y).max(axis=-1, keepdims=True)
    flushed = s[..., 0] == 0
    assert np.all(np.abs(yq - y)[~flushed] <= tol[~flushed])
    assert np.all(F.e4m3_decode(scales) <= 448)
    if bound_is_pow2:
        assert np.all(np.abs(y) <= 2688 * float(D) * (1 + 2 ** -20))


@pytest.mark.parametrize("alignment", [16, 128, 256])
def test_direct_receive_small(alignment):
    w = workloads.small_dispatch(3, 150, 256, 5, 2, alignment=alignment, unused_frac=0.05, empty=[3])
    packed = nvfp4.pack_rows(w.x_bits)
    out = receive.direct_receive(packed, 256, w.topk_idx, 5, alignment)
    off, counts, src = out["offsets"], out["counts"], out["src_row"]
    assert counts[3] == 0 and out["col_scale"][3] == 0
    # P1 test analogue: decoding the grouped rowwise operand equals decoding the
    # sender's rows and then permuting them into grouped order.
    grouped = np.concatenate([out["row_codes"], out["row_scales"],
                              out["row_t"].astype("<f4").view(np.uint8).reshape(-1, 4)], axis=1)
    np.testing.assert_array_equal(nvfp4.unpack_rows(grouped[: off[-1]], 256),
                                  nvfp4.unpack_rows(packed, 256, src[: off[-1]]))
    exact = nvfp4.decode_exact(packed, 256)
    _, _, t = nvfp4.split_rows(packed, 256)
    for e in range(5):
        c = int(counts[e])
        if c == 0:
            continue
        rows = src[off[e] : off[e] + c]
        assert out["col_scale"][e] == 4 * t[rows].max()
        p = int(off[e + 1] - off[e])
        vals = np.zeros((p, 256)); vals[:c] = exact[rows]
        cc = out["col_codes"][256 * off[e] // 2 : 256 * off[e + 1] // 2].reshape(256, p // 2)
        cs = out["col_scales"][256 * off[e] // 16 : 256 * off[e + 1] // 16].reshape(256, p // 16)
        _check_columnwise(vals, cc, cs, out["col_scale"][e], True)
        # padding-only 16-row blocks decode to zero (signed-zero codes) with zero scales
        pc = (c + 15) // 16
        assert np.all((F.unpack_nibbles(cc[:, pc * 8 :]) & 7) == 0) and np.all(cs[:, pc:] == 0)


def test_expert_slice_equals_standalone():
    """P3 analogue: the grouped operand of expert e equals the operand built from
    expert e's tokens alone, routed as a single-expert dispatch."""
    w = workloads.small_dispatch(4, 120, 128, 4, 2)
    packed = nvfp4.pack_rows(w.x_bits)
    out = receive.direct_receive(packed, 128, w.topk_idx, 4, 16)
    off = out["offsets"]
    for e in range(4):
        toks = np.nonzero((w.topk_idx == e).any(axis=1))[0]
        solo = receive.direct_receive(packed[toks], 128, np.zeros((len(toks), 1), np.int32), 1, 16)
        p = int(off[e + 1] - off[e])
        np.testing.assert_array_equal(out["row_codes"][off[e] : off[e + 1]], solo["row_codes"][:p])
        np.testing.assert_array_equal(out["col_codes"][128 * off[e] // 2 : 128 * off[e + 1] // 2],
                                      solo["col_codes"][: 128 * p // 2])
        np.testing.assert_array_equal(out["col_scales"][128 * off[e] // 16 : 128 * off[e + 1] // 16],
                                      solo["col_scales"][: 128 * p // 16])
        assert out["col_scale"][e] == solo["col_scale"][0]


def test_columnwise_sample_matches_full():
    w = workloads.small_dispatch(8, 200, 192, 3, 2)
    packed = nvfp4.pack_rows(w.x_bits)
    out = receive.direct_receive(packed, 192, w.topk_idx, 3, 16)
    plan = route_plan(w.topk_idx, 3, 16)
    e = 1
    off = out["offsets"]
    p = int(off[e + 1] - off[e])
    full = F.unpack_nibbles(out["col_codes"][192 * off[e] // 2 : 192 * off[e + 1] // 2].reshape(192, p // 2))
    codes, sc = receive.columnwise_sample(packed, 192, plan, e, 32, 80, 1, 3, out["col_scale"][e])
    np.testing.assert_array_equal(codes, full[32:80, 16:48])


# ------------------------------------------------------------------ dSwiGLU
def test_dswiglu_matches_autograd_float64():
    """Library pin: torch.autograd in float64 of silu(a) * b, rounded to BF16."""
    w = workloads.small_dswiglu(1, [3, 40, 0, 21], 96)
    ours = dswiglu.dswiglu(w.preact_bits, w.dy_bits)
    p = torch.from_numpy(F.bf16_to_f32(w.preact_bits).astype(np.float64)).requires_grad_(True)
    dy = torch.from_numpy(F.bf16_to_f32(w.dy_bits).astype(np.float64))
    a, b = p[:, :96], p[:, 96:]
    (torch.nn.functional.silu(a) * b).backward(dy)
    ref = dswiglu.f64_to_bf16(p.grad.numpy())
    diff = np.abs(ours.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 1e-3


def test_f64_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-40, 30, 100000)).astype(np.float32)
    np.testing.assert_array_equal(dswiglu.f64_to_bf16(x.astype(np.float64)),
                                  torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_amax_and_fused_rowwise_equal_default():
    """P4 test: per-expert rowwise amaxes equal the amaxes of the BF16 gradient (empty
    experts give 0), and the rowwise operand from the epilogue amax is identical to
    the one from a separate amax pass over the gradient."""
    w = workloads.small_dswiglu(2, [0, 17, 64, 1, 0, 33], 64)
    dx = dswiglu.dswiglu(w.preact_bits, w.dy_bits)
    am = dswiglu.expert_amax(dx, w.counts)
    x = np.abs(F.bf16_to_f32(dx))
    off = np.concatenate([[0], np.cumsum(w.counts)])
    for e in range(6):
        want = x[off[e] : off[e + 1]].max() if w.counts[e] else 0.0
        assert am[e] == want
    sep = np.array([x[off[e] : off[e + 1]].max() if w.counts[e] else 0 for e in range(6)], np.float32)
    a = dswiglu.rowwise_quant(dx, w.counts, am)
    b = dswiglu.rowwise_quant(dx, w.counts, sep)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_fc1_columnwise_bound_and_decode():
    w = workloads.small_dswiglu(3, [5, 40, 0, 16, 1], 64)
    dx = dswiglu.dswiglu(w.preact_bits, w.dy_bits)
    am = dswiglu.expert_amax(dx, w.counts)
    q = dswiglu.fc1_grad_quant(dx, w.counts, am)
    np.testing.assert_array_equal(q["col_scale"], 4 * q["row_scale"])
    x = F.bf16_to_f32(dx).astype(np.float64)
    off = dswiglu.expert_offsets(w.counts)
    poff = dswiglu.expert_offsets(w.counts, 16)
    h = 128
    for e in range(5):
        c = int(w.counts[e])
        if not c:
            continue
        p = int(poff[e + 1] - poff[e])
        vals = np.zeros((p, h)); vals[:c] = x[off[e] : off[e + 1]]
        cc = q["col_codes"][h * poff[e] // 2 : h * poff[e + 1] // 2].reshape(h, p // 2)
        cs = q["col_scales"][h * poff[e] // 16 : h * poff[e + 1] // 16].reshape(h, p // 16)
        _check_columnwise(vals, cc, cs, q["col_scale"][e], False)
    # rowwise decode within the per-element bound
    codes = F.unpack_nibbles(q["row_codes"])
    s = np.repeat(F.e4m3_decode(q["row_scales"]), 16, axis=1)
    De = np.repeat(q["row_scale"], w.counts)[:, None]
    xh = F.e2m1_value(codes) * s * De
    st = s * De
    v = np.abs(x) / np.where(st > 0, st, 1)
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    tol = np.where(v <= 6, step / 2, v - 6) * st * (1 + 1e-6)
    assert np.all((np.abs(x - xh) <= tol)[st > 0])


def test_fc1_wgrad_error_within_5_percent_of_default():
    """P4 test: FC1 wgrad error with the bound-derived columnwise scale stays within 5%
    of the default path (exact post-RHT amax).  wgrad_e = dX_e^T X_e contracts over the
    expert's tokens; both operands use the same RHT, so the transform cancels."""
    counts = [0, 256, 48, 512, 16]
    w = workloads.small_dswiglu(5, counts, 64)
    dx = dswiglu.dswiglu(w.preact_bits, w.dy_bits)
    am = dswiglu.expert_amax(dx, np.array(counts))
    rng = np.random.default_rng(7)
    T, hin = sum(counts), 96
    X = F.bf16_to_f32(F.f32_to_bf16(rng.standard_normal((T, hin)).astype(np.float32))).astype(np.float64)
    xam = np.array([np.abs(X[a:b]).max() if b > a else 0 for a, b in
                    zip(np.cumsum([0] + counts)[:-1], np.cumsum(counts))], np.float32)
    xbits = F.f32_to_bf16(X.astype(np.float32))
    xc, xs, xd = dswiglu.columnwise_quant(xbits, np.array(counts), xam, exact_amax=True)
    fused = dswiglu.columnwise_quant(dx, np.array(counts), am)
    default = dswiglu.columnwise_quant(dx, np.array(counts), am, exact_amax=True)
    g = F.bf16_to_f32(dx).astype(np.float64)
    off = dswiglu.expert_offsets(counts)
    poff = dswiglu.expert_offsets(counts, 16)
    errs = {"fused": 0.0, "default": 0.0}
    ref_norm = 0.0
    for e, c in enumerate(counts):
        if not c:
            continue
        p = int(poff[e + 1] - poff[e])
        wx = _decode_col(xc[hin * poff[e] // 2 : hin * poff[e + 1] // 2].reshape(hin, p // 2),
                         xs[hin * poff[e] // 16 : hin * poff[e + 1] // 16].reshape(hin, p // 16), xd[e]).reshape(hin, p)
        ref = g[off[e] : off[e + 1]].T @ X[off[e] : off[e + 1]]
        ref_norm += (ref ** 2).sum()
        for name, (cc, cs, D) in (("fused", fused), ("default", default)):
            wg = _decode_col(cc[128 * poff[e] // 2 : 128 * poff[e + 1] // 2].reshape(128, p // 2),
                             cs[128 * poff[e] // 16 : 128 * poff[e + 1] // 16].reshape(128, p // 16), D[e]).reshape(128, p)
            errs[name] += ((wg @ wx.T - ref) ** 2).sum()
    assert np.sqrt(errs["fused"]) <= 1.05 * np.sqrt(errs["default"]), errs
    assert np.sqrt(errs["default"]) / np.sqrt(ref_norm) < 0.2


@pytest.mark.parametrize("scale_rows, sizes", [
    (16, [272, 0, 256, 16, 528, 32]),     # NVFP4: experts of 256 + 16 rows, exactly 256, 16 and empty
    (32, [288, 0, 256, 32, 544, 64]),     # MXFP4: one scale per 32 rows
])
def test_kblock_layout_is_a_permutation_read_back_by_a_blocked_consumer(scale_rows, sizes):
    """The K-blocked columnwise layout holds the compact operand's bytes: a consumer that
    walks experts, then K-blocks, then columns recovers every (column, grouped row) code
    and scale of the compact layout -- including a last K-block shorter than 256 rows,
    an expert of exactly 256 rows, one of a single scale block and an empty one."""
    from oracle.receive import kblock_layout
    rng = np.random.default_rng(41 + scale_rows)
    h = 64
    sr = scale_rows
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(off[-1])
    comp_c = rng.integers(0, 256, h * n // 2, dtype=np.uint8)
    comp_s = rng.integers(0, 127, h * n // sr, dtype=np.uint8)
    kc, ks = kblock_layout(comp_c, comp_s, off, h, scale_rows=sr)
    assert sorted(kc.tolist()) == sorted(comp_c.tolist())          # a permutation of the bytes
    assert sorted(ks.tolist()) == sorted(comp_s.tolist())
    for e, p in enumerate(sizes):
        o = int(off[e])
        cpos = h * o // 2
        spos = h * o // sr
        for r0 in range(0, p, 256):
            ln = min(256, p - r0)
            for col in range(h):
                for j in range(0, ln, 2):              # grouped rows r0 + j, r0 + j + 1 share a byte
                    want = comp_c[h * o // 2 + col * (p // 2) + (r0 + j) // 2]
                    assert kc[cpos] == want, (e, r0, col, j)
                    cpos += 1
            for col in range(h):
                for b in range(ln // sr):
                    assert ks[spos] == comp_s[h * o // sr + col * (p // sr) + r0 // sr + b]
                    spos += 1
        assert cpos == h * (o + p) // 2 and spos == h * (o + p) // sr
