"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact for codes, block scales, token scales, MXFP8 data/scales,
routing (counts, offsets, dst_row, src_row), the rowwise grouped operand, the
expert scales D_e, unpacked BF16 and stochastic rounding; for values derived
from FP32 amaxes or post-RHT values, the tolerance in ``gpu_util.tolerant_codes``
(the bar: a differing E2M1 code is off by one grid step, in at most 1e-4 of
elements).  Inputs come from ``workloads`` (seeded, synthetic).
"""

import types

import numpy as np
import pytest
import torch

import moe_token_block_amd as mtb
import workloads
from oracle import formats as F
from oracle import mxfp8 as omx
from oracle import mxfp4 as omx4
from oracle import nvfp4 as onv
from oracle import dswiglu as odsw
from oracle import receive as orecv
from oracle.routing import route_plan as o_route

from gpu_util import require_gpu, bf16_dev, host, i32_dev, assert_bytes_equal, tolerant_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _edge_rows(h, rng):
    """Rows that exercise the corner cases of the token / block scale rules."""
    rows = []
    rows.append(np.zeros(h))                                   # all-zero row
    r = rng.standard_normal(h); r[:16] = 0.0; rows.append(r)   # a zero block
    rows.append(rng.standard_normal(h) * 1e-38)                # BF16 subnormal territory
    rows.append(rng.standard_normal(h) * 1e-30)                # tiny t
    rows.append(rng.standard_normal(h) * 1e36)                 # huge t
    r = rng.standard_normal(h) * 1e-3; r[5] = 1e3; rows.append(r)  # one outlier
    r = np.full(h, -0.0); rows.append(r)                      # all -0
    r = rng.standard_normal(h); r[::7] = -0.0; rows.append(r)
    # values on exact E2M1 ties relative to the block scale
    r = np.tile([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.25, 0.5, 3.0, 4.0, 1.5, 1.0, 2.0], h // 16)
    rows.append(r * 3.0)
    r = rng.standard_normal(h) * np.exp(rng.uniform(-20, 20, h)); rows.append(r)  # wide in-row range
    return np.array(rows)


def _bits(x):
    return F.f32_to_bf16(np.asarray(x, dtype=np.float32))


# ------------------------------------------------------------------ NVFP4 pack / unpack
@pytest.mark.parametrize("h", [64, 128, 192, 1024, 2112, 7168, 16384])
def test_pack_unpack_bit_exact(dev, h):
    rng = np.random.default_rng(h)
    n = 37
    x = rng.standard_normal((n, h)) * 10.0 ** rng.uniform(-4, 4, size=(n, 1))
    x = np.concatenate([x, _edge_rows(h, rng)])
    bits = _bits(x)
    print(f"pack/unpack h={h} rows={bits.shape[0]}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    want = onv.pack_rows(bits)
    assert_bytes_equal(host(packed), want, f"pack h={h}")
    un = mtb.ep_nvfp4_unpack(packed, h)
    assert_bytes_equal(host(un), onv.unpack_rows(want, h), f"unpack h={h}")
    src = rng.integers(-1, bits.shape[0], size=2 * bits.shape[0]).astype(np.int32)
    un2 = mtb.ep_nvfp4_unpack(packed, h, src_row=i32_dev(src, dev))
    assert_bytes_equal(host(un2), onv.unpack_rows(want, h, src), f"unpack gather h={h}")


def test_pack_empty_and_config1(dev):
    out = mtb.ep_nvfp4_pack(torch.empty((0, 128), dtype=torch.bfloat16, device=dev))
    assert out.shape == (0, 76)
    w = workloads.config1()
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    want = onv.pack_rows(w.x_bits)
    assert_bytes_equal(host(packed), want, "pack config1")
    assert_bytes_equal(host(mtb.ep_nvfp4_unpack(packed, 1024)), onv.unpack_rows(want, 1024), "unpack config1")


@pytest.mark.parametrize("mode,seed,base", [(1, 1234, 0), (1, 2 ** 40 + 3, 12345), (2, 1234, 0), (2, 77, 6),
                                           (3, 1234, 0), (3, 2 ** 40 + 3, 12345), (4, 1234, 0), (4, 77, 6)])
def test_stochastic_rounding_bit_exact(dev, mode, seed, base):
    rng = np.random.default_rng(seed % 1000 + mode)
    h = 256
    x = rng.standard_t(3, size=(48, h)) * 1e-3
    x = np.concatenate([x, _edge_rows(h, rng)])
    bits = _bits(x)
    st = torch.tensor([seed, base], dtype=torch.int64, device=dev)
    print(f"sr mode={mode} seed={seed} base={base}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev), round_mode=mode, sr_state=st)
    want = onv.pack_rows(bits, sr_seed=seed, sr_counter_base=base, sr_mode="element" if mode in (1, 3) else "stream",
                         sr_rule="carry" if mode >= 3 else "threshold")
    assert_bytes_equal(host(packed), want, f"SR mode {mode}")


@pytest.mark.parametrize("h,rows,mode", [(64, 13001, 3), (1088, 70, 3), (2048, 33, 1), (4096, 41, 3), (4096, 9, 2),
                                         (8192, 9, 3)])
def test_stochastic_rounding_shapes(dev, h, rows, mode):
    """Row counts and widths that exercise the row-pipelined SR kernel (one, two and
    four blocks per lane, lanes past the row's end, many rows per wave, a ragged
    last pair of rows) and the two-pass kernel beyond 4096 columns."""
    rng = np.random.default_rng(h + rows)
    x = rng.standard_t(3, size=(rows, h)) * 10.0 ** rng.uniform(-4, 1, size=(rows, 1))
    bits = _bits(x)
    seed, base = 1234 + h, 99 * rows
    st = torch.tensor([seed, base], dtype=torch.int64, device=dev)
    print(f"sr shapes h={h} rows={rows} mode={mode}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev), round_mode=mode, sr_state=st)
    want = onv.pack_rows(bits, sr_seed=seed, sr_counter_base=base, sr_mode="element" if mode in (1, 3) else "stream",
                         sr_rule="carry" if mode >= 3 else "threshold")
    assert_bytes_equal(host(packed), want, f"SR h={h} rows={rows} mode={mode}")


# ------------------------------------------------------------------ MXFP8
@pytest.mark.parametrize("h", [32, 96, 1024, 4096])
def test_mxfp8_pack_bit_exact(dev, h):
    rng = np.random.default_rng(100 + h)
    x = rng.standard_normal((41, h)) * 10.0 ** rng.uniform(-5, 5, size=(41, 1))
    if h >= 64:
        x = np.concatenate([x, _edge_rows(h, rng)])
    x[0, :32] = 1e-39
    bits = _bits(x)
    data, scales, _ = mtb.ep_mxfp8_pack(bf16_dev(bits, dev))
    wd, ws = omx.pack_rows(bits)
    assert_bytes_equal(host(scales), ws, f"mxfp8 scales h={h}")
    assert_bytes_equal(host(data), wd, f"mxfp8 data h={h}")


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("tokens,k,E,A,idx64,unused", [
    (1, 1, 1, 16, False, 0.0), (97, 3, 6, 16, False, 0.1), (300, 2, 8, 128, True, 0.0),
    (513, 4, 33, 256, False, 0.05), (2048, 8, 32, 16, True, 0.0), (1000, 1, 1024, 16, False, 0.0),
    (0, 2, 4, 16, False, 0.0),
    (600, 2, 40, 1024, False, 0.0),      # one workgroup, capacity beyond the LDS-staged src_row
    (4100, 8, 16, 16, False, 0.02),      # > 16384 entries: the three-kernel path, a ragged last wave
    (2049, 8, 64, 16, True, 0.0)])       # 16392 entries: just past the one-workgroup limit
def test_route_plan_bit_exact(dev, tokens, k, E, A, idx64, unused):
    rng = np.random.default_rng(tokens * 7 + E)
    topk = np.array([rng.permutation(E)[:k] for _ in range(tokens)], dtype=np.int32).reshape(tokens, k)
    if unused:
        topk[rng.random(topk.shape) < unused] = -1
    if E > 2 and tokens > 0:
        topk[topk == E - 2] = -1                       # one empty expert
    t_dev = torch.from_numpy(topk.astype(np.int64 if idx64 else np.int32)).to(dev)
    plan = mtb.ep_route_plan(t_dev, E, A)
    want = o_route(topk, E, A)
    for key in ("counts", "offsets", "dst_row", "src_row"):
        assert_bytes_equal(host(plan[key]), want[key], f"route {key}")
    assert int(host(plan["d_error"])[0]) == 0


def test_route_plan_flags_bad_ids(dev):
    topk = np.array([[0, 1], [5, -1], [2, -3], [1, 0]], dtype=np.int32)
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), 4, 16)
    want = o_route(topk, 4, 16)
    assert int(host(plan["d_error"])[0]) == mtb.EP_DEVERR_EXPERT_ID
    for key in ("counts", "offsets", "dst_row", "src_row"):
        assert_bytes_equal(host(plan[key]), want[key], f"route {key}")


# ------------------------------------------------------------------ direct receive
def _check_receive(dev, w, packed_np, got, plan_np, hidden, exact=True):
    off = plan_np["offsets"].astype(np.int64)
    rc = host(got["row_codes"])[: off[-1]]
    want = orecv.direct_receive(packed_np, hidden, w.topk_idx, w.num_experts, w.alignment)
    assert_bytes_equal(rc, want["row_codes"][: off[-1]], "rowwise codes")
    assert_bytes_equal(host(got["row_scales"])[: off[-1]], want["row_scales"][: off[-1]], "rowwise scales")
    assert_bytes_equal(host(got["row_t"])[: off[-1]].view(np.uint32), want["row_t"][: off[-1]].view(np.uint32), "row t")
    assert_bytes_equal(host(got["col_scale"]).view(np.uint32), want["col_scale"].view(np.uint32), "D_e")
    n = hidden * off[-1]
    gc = host(got["col_codes"])[: n // 2]
    gs = host(got["col_scales"])[: n // 16]
    if exact:
        assert_bytes_equal(gs, want["col_scales"][: n // 16], "columnwise scales")
        assert_bytes_equal(gc, want["col_codes"][: n // 2], "columnwise codes")
    else:
        tolerant_codes(F.unpack_nibbles(gc), F.unpack_nibbles(want["col_codes"][: n // 2]), gs,
                       want["col_scales"][: n // 16], "columnwise")


@pytest.mark.parametrize("case", [
    dict(seed=1, tokens=150, hidden=256, E=5, k=2, A=16, unused=0.05, empty=[3]),
    dict(seed=2, tokens=600, hidden=128, E=8, k=2, A=128, unused=0.0, empty=[]),
    dict(seed=3, tokens=333, hidden=192, E=3, k=1, A=256, unused=0.2, empty=[]),
    dict(seed=4, tokens=1024, hidden=512, E=16, k=4, A=16, unused=0.0, empty=[0, 15]),
    dict(seed=5, tokens=7, hidden=64, E=4, k=2, A=16, unused=0.0, empty=[]),
    dict(seed=6, tokens=1000, hidden=128, E=1024, k=1, A=16, unused=0.0, empty=[]),   # the maximum expert count
    dict(seed=7, tokens=500, hidden=64, E=300, k=3, A=32, unused=0.1, empty=list(range(0, 300, 3))),
    dict(seed=8, tokens=300, hidden=448, E=6, k=2, A=16, unused=0.1, empty=[2]),      # a 192-column last tile
    dict(seed=9, tokens=64, hidden=16384, E=4, k=2, A=16, unused=0.0, empty=[]),      # the widest packed row
])
def test_direct_receive_bit_exact(dev, case):
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"], unused_frac=case["unused"], empty=case["empty"])
    print(f"receive case {case}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    packed_np = onv.pack_rows(w.x_bits)
    assert_bytes_equal(host(packed), packed_np, "pack")
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), w.num_experts, w.alignment)
    got = mtb.ep_nvfp4_direct_receive(packed, w.x_bits.shape[1], plan)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    _check_receive(dev, w, packed_np, got, plan_np, w.x_bits.shape[1])


def test_direct_receive_edge_rows(dev):
    """Zero, -0, subnormal, tiny-t (t < 2^-100: the two-step decode), huge-t and
    outlier rows routed among ordinary rows, so 16-row blocks mix them."""
    rng = np.random.default_rng(21)
    h = 256
    edge = _edge_rows(h, rng)
    x = np.concatenate([rng.standard_normal((70, h)) * 10.0 ** rng.uniform(-1, 1, (70, 1)), edge, edge, edge])
    x = x[rng.permutation(len(x))]
    bits = _bits(x)
    topk = np.argsort(-rng.standard_normal((len(x), 4)), axis=1)[:, :2].astype(np.int32)
    print("receive edge rows", bits.shape, flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    packed_np = onv.pack_rows(bits)
    assert_bytes_equal(host(packed), packed_np, "pack")
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), 4, 16)
    got = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    w = types.SimpleNamespace(topk_idx=topk, num_experts=4, alignment=16)
    _check_receive(dev, w, packed_np, got, plan_np, h)


def _tiny_max_rows(seed, h=256):
    """Experts whose rows all have amax below 2^-110 (so D_e is 2^-122 .. 2^-135),
    with 16-row blocks whose post-RHT max a has a / 6 below FP32's normal range:
    the corner where the block-scale rule's rounding of a / 6 is on FP32's
    subnormal grid.  Each expert's first row sets its D_e."""
    rng = np.random.default_rng(seed)
    rows, ex = [], []
    for e, (lead, n, lo, hi) in enumerate([(-116, 64, -134, -121), (-113, 48, -134, -121), (-120, 80, -134, -121),
                                           (-127.5, 512, -133, -127.5), (-126.7, 512, -133, -127)]):
        r = rng.standard_normal((n, h)) * 2.0 ** rng.uniform(lo, hi, (n, 1))
        r[0] = rng.standard_normal(h)
        r[0] *= 2.0 ** lead / np.abs(r[0]).max()
        rows.append(r)
        ex += [e] * n
    return _bits(np.concatenate(rows)), np.array(ex, np.int32)[:, None]


def test_direct_receive_tiny_max_corner(dev):
    """Columnwise blocks with a / 6 below FP32's normal range (R16: the scale is
    E4M3 of the exact a / (6 D_e)), compared byte for byte; the oracle confirms
    that thousands of such blocks have a nonzero scale."""
    from oracle.rht import rht16
    bits, topk = _tiny_max_rows(5)
    h, E = bits.shape[1], 5
    packed_np = onv.pack_rows(bits)
    want = orecv.direct_receive(packed_np, h, topk, E, 16)
    ex = onv.decode_exact(packed_np, h)
    off, src = want["offsets"], want["src_row"]
    n_corner = 0
    for e in range(E):
        y = rht16(ex[src[off[e]:off[e + 1]]].T.reshape(h, -1, 16))
        a = np.abs(y).max(axis=-1)
        s = orecv.block_scale_codes(a, want["col_scale"][e], "pow2")
        n_corner += int(((a.astype(np.float64) / 6 < 2.0 ** -126) & (s > 0)).sum())
    assert n_corner > 10000
    assert want["col_scale"].max() < 2.0 ** -120
    print("receive tiny-max corner", bits.shape, n_corner, flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    assert_bytes_equal(host(packed), packed_np, "pack")
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), E, 16)
    got = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    w = types.SimpleNamespace(topk_idx=topk, num_experts=E, alignment=16)
    _check_receive(dev, w, packed_np, got, plan_np, h)
    # the operand built from the grouped rows takes the same rule
    n = h * int(off[-1])
    grp = mtb.ep_nvfp4_columnwise_grouped(got, h, plan)
    assert_bytes_equal(host(grp["col_scales"])[: n // 16], want["col_scales"][: n // 16], "grouped columnwise scales")
    assert_bytes_equal(host(grp["col_codes"])[: n // 2], want["col_codes"][: n // 2], "grouped columnwise codes")


def test_direct_receive_tiny_expert(dev):
    """An expert whose rows all have tiny token scales (t near 2^-110, so its
    D_e < 2^-95 and every block of it, padding included, takes the general
    decode and quantizer) beside an expert of ordinary rows: byte for byte."""
    rng = np.random.default_rng(71)
    h = 256
    tiny = rng.standard_normal((37, h)) * 2.0 ** -100   # amax near 2^-98: t near 2^-110
    mid = rng.standard_normal((5, h)) * 2.0 ** -80      # t near 2^-91: slow by t, ordinary D_e
    big = rng.standard_normal((45, h))
    bits = _bits(np.concatenate([tiny, mid, big]))
    topk = np.concatenate([np.zeros(37), np.ones(5), np.ones(45)]).astype(np.int32)[:, None]
    print("receive tiny expert", bits.shape, flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    packed_np = onv.pack_rows(bits)
    assert_bytes_equal(host(packed), packed_np, "pack")
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), 2, 16)
    got = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    assert host(got["col_scale"])[0] < 2.0 ** -95
    w = types.SimpleNamespace(topk_idx=topk, num_experts=2, alignment=16)
    _check_receive(dev, w, packed_np, got, plan_np, h)
    # the K-blocked layout and the operand built from the grouped rows share the column code
    want = orecv.direct_receive(packed_np, h, topk, 2, 16)
    off = plan_np["offsets"].astype(np.int64)
    n = h * int(off[-1])
    kb = {k: torch.empty_like(v) for k, v in got.items()}
    kb["col_scale"] = got["col_scale"].clone()
    mtb.ep_nvfp4_direct_receive_kblock(packed, h, plan, kb)
    wc, ws = orecv.kblock_layout(want["col_codes"][: n // 2], want["col_scales"][: n // 16], off, h)
    assert_bytes_equal(host(kb["col_codes"])[: n // 2], wc, "K-block columnwise codes")
    assert_bytes_equal(host(kb["col_scales"])[: n // 16], ws, "K-block columnwise scales")
    grp = mtb.ep_nvfp4_columnwise_grouped(got, h, plan)
    assert_bytes_equal(host(grp["col_codes"])[: n // 2], want["col_codes"][: n // 2], "grouped columnwise codes")
    assert_bytes_equal(host(grp["col_scales"])[: n // 16], want["col_scales"][: n // 16], "grouped columnwise scales")
    # and with stochastic columnwise codes
    sr = torch.tensor([77, 3], dtype=torch.int64, device=dev)
    srg = {k: torch.empty_like(v) for k, v in got.items()}
    srg["col_scale"] = got["col_scale"].clone()
    mtb.ep_nvfp4_direct_receive_sr(packed, h, plan, srg, sr)
    want_sr = orecv.direct_receive(packed_np, h, topk, 2, 16, sr=(77, 3))
    assert_bytes_equal(host(srg["col_codes"])[: n // 2], want_sr["col_codes"][: n // 2], "SR columnwise codes")
    assert_bytes_equal(host(srg["col_scales"])[: n // 16], want["col_scales"][: n // 16], "SR columnwise scales")


@pytest.mark.parametrize("idx64", [False, True])
def test_direct_receive_topk_one_call(dev, idx64):
    """The receive from top-k indices in one C call (route plan + D_e + operands)
    equals the oracle byte for byte, plan included; a bad expert id sets the
    device error word and the entry is dropped, as for the route plan alone."""
    w = workloads.small_dispatch(81, 333, 192, 6, 2, alignment=32, unused_frac=0.05, empty=[4])
    topk = w.topk_idx.copy()
    topk[7, 1] = 9                                  # out of range: flagged and dropped
    print(f"one-call receive idx64={idx64}", flush=True)
    packed_np = onv.pack_rows(w.x_bits)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    t_dev = torch.from_numpy(topk.astype(np.int64 if idx64 else np.int32)).to(dev)
    plan, got = mtb.ep_nvfp4_direct_receive_topk(packed, 192, t_dev, 6, 32)
    want_plan = o_route(topk, 6, 32)
    for key in ("counts", "offsets", "dst_row", "src_row"):
        assert_bytes_equal(host(plan[key]), want_plan[key], f"one-call {key}")
    assert int(host(plan["d_error"])[0]) == mtb.EP_DEVERR_EXPERT_ID
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    wv = types.SimpleNamespace(topk_idx=topk, num_experts=6, alignment=32)
    _check_receive(dev, wv, packed_np, got, plan_np, 192)
    # rowwise only
    plan2, rows = mtb.ep_nvfp4_direct_receive_topk(packed, 192, t_dev, 6, 32, columnwise=False)
    off = int(want_plan["offsets"][-1])
    assert "col_codes" not in rows
    assert_bytes_equal(host(rows["row_codes"])[:off], host(got["row_codes"])[:off], "one-call rowwise only")


def test_binding_refuses_missized_buffers(dev):
    """Buffers too small for the sizes passed with them, a packed width that does
    not match hidden, and preact/dy shapes that disagree are refused before
    anything is launched (the outputs keep their sentinel bytes)."""
    w = workloads.small_dispatch(82, 64, 128, 4, 2)
    x = bf16_dev(w.x_bits, dev)
    packed = mtb.ep_nvfp4_pack(x)
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), 4, 16)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        mtb.ep_nvfp4_pack(x, out=torch.full((64, 70), 0xAB, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        mtb.ep_nvfp4_unpack(packed, 192)                                   # 76-byte rows are hidden 128
    small = torch.full((10, 128), 7, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        mtb.ep_nvfp4_unpack(packed, 128, out=small)
    ref = mtb.ep_nvfp4_direct_receive(packed, 128, plan)
    for key in ("row_codes", "row_scales", "row_t", "col_codes", "col_scales", "col_scale"):
        bad = {k: v.clone() for k, v in ref.items()}
        bad[key] = torch.full((bad[key].numel() - 1,), 3, dtype=bad[key].dtype, device=dev)
        with pytest.raises(ValueError):
            mtb.ep_nvfp4_direct_receive(packed, 128, plan, out=bad)
        torch.cuda.synchronize()
        assert (bad[key] == 3).all(), key
    short_plan = dict(plan, src_row=plan["src_row"][:-1].clone())
    with pytest.raises(ValueError):
        mtb.ep_nvfp4_direct_receive(packed, 128, short_plan)
    sw = workloads.small_dswiglu(83, [5, 9], 64)
    pre, dy = bf16_dev(sw.preact_bits, dev), bf16_dev(sw.dy_bits, dev)
    cnt = i32_dev(sw.counts, dev)
    with pytest.raises(ValueError):
        mtb.dswiglu_nvfp4_quant(pre[:, :96].contiguous(), dy, cnt)         # preact must be [T, 2F]
    good = mtb.dswiglu_nvfp4_quant(pre, dy, cnt)
    for key in ("amax", "row_codes", "col_scales"):
        bad = dict(good)
        bad[key] = torch.zeros(good[key].numel() - 1, dtype=good[key].dtype, device=dev)
        with pytest.raises(ValueError):
            mtb.dswiglu_nvfp4_quant(pre, dy, cnt, out=bad)
    with pytest.raises(ValueError):
        mtb.dswiglu_nvfp4_quant(pre, dy, cnt, workspace=torch.zeros(8, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()


def test_direct_receive_config1(dev):
    w = workloads.config1()
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), 4, 16)
    got = mtb.ep_nvfp4_direct_receive(packed, 1024, plan)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    _check_receive(dev, w, onv.pack_rows(w.x_bits), got, plan_np, 1024)
    # P1 test analogue: decoding the grouped rowwise rows equals decoding the sender rows in grouped order
    off = int(plan_np["offsets"][-1])
    dec = mtb.ep_nvfp4_unpack(packed, 1024, src_row=plan["src_row"][:off].contiguous())
    assert_bytes_equal(host(dec), onv.unpack_rows(onv.pack_rows(w.x_bits), 1024, plan_np["src_row"][:off]),
                       "grouped decode")


def test_direct_receive_rowwise_only(dev):
    w = workloads.small_dispatch(9, 200, 192, 4, 2)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), 4, 16)
    got = mtb.ep_nvfp4_direct_receive(packed, 192, plan, columnwise=False)
    want = orecv.direct_receive(onv.pack_rows(w.x_bits), 192, w.topk_idx, 4, 16, columnwise=False)
    off = int(host(plan["offsets"])[-1])
    assert_bytes_equal(host(got["row_codes"])[:off], want["row_codes"][:off], "rowwise-only codes")


@pytest.mark.parametrize("tokens", [0, 50])
def test_receives_without_routed_rows(dev, tokens):
    """No routed row at all -- no tokens, or every slot unused (-1): the plans
    hold only zero counts, and every receive returns cleanly with D_e = 0 and
    the oracle's (empty) operands."""
    h, E, A = 192, 4, 32
    rng = np.random.default_rng(61 + tokens)
    bits = _bits(rng.standard_normal((tokens, h)))
    topk = np.full((tokens, 2), -1, np.int32)
    print(f"receives without routed rows tokens={tokens}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    packed_np = onv.pack_rows(bits)
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), E, A)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    assert not plan_np["offsets"].any() and not plan_np["counts"].any()
    assert (plan_np["src_row"] == -1).all()
    w = types.SimpleNamespace(topk_idx=topk, num_experts=E, alignment=A)
    _check_receive(dev, w, packed_np, mtb.ep_nvfp4_direct_receive(packed, h, plan), plan_np, h)
    got4 = mtb.ep_mxfp4_direct_receive(packed, h, plan)
    _check_mxfp4(got4, omx4.direct_receive(packed_np, h, topk, E, A), 0, h)
    data, scales, _ = mtb.ep_mxfp8_pack(bf16_dev(bits, dev))
    gd, gs = mtb.ep_mxfp8_direct_receive(data, scales, plan)
    assert not host(gd).any() and not host(gs).any()  # every grouped row is padding
    torch.cuda.synchronize(dev)


@pytest.mark.parametrize("case", [
    dict(seed=31, tokens=150, hidden=256, E=5, k=2, A=16, unused=0.05, empty=[3]),
    dict(seed=32, tokens=600, hidden=4096, E=8, k=2, A=128, unused=0.0, empty=[]),
    dict(seed=33, tokens=333, hidden=192, E=3, k=1, A=256, unused=0.2, empty=[]),
    dict(seed=34, tokens=257, hidden=512, E=16, k=8, A=16, unused=0.0, empty=[0, 15]),
    dict(seed=35, tokens=1000, hidden=128, E=1024, k=1, A=16, unused=0.0, empty=[]),
])
def test_pack_scatter_and_grouped_columnwise(dev, case):
    """Fused dispatch: the pack writing grouped rows directly, then the columnwise operand
    from those rows, equal the oracle's direct receive byte for byte (and the unfused GPU path)."""
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"], unused_frac=case["unused"], empty=case["empty"])
    h = case["hidden"]
    print(f"pack-scatter case {case}", flush=True)
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), w.num_experts, w.alignment)
    rows = mtb.ep_nvfp4_pack_scatter(bf16_dev(w.x_bits, dev), plan)
    got = dict(rows)
    got.update(mtb.ep_nvfp4_columnwise_grouped(rows, h, plan))
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    _check_receive(dev, w, onv.pack_rows(w.x_bits), got, plan_np, h)
    # and the unfused GPU receive of the same rows
    ref = mtb.ep_nvfp4_direct_receive(mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev)), h, plan)
    off = int(plan_np["offsets"][-1])
    for key in ("row_codes", "row_scales", "row_t"):
        assert_bytes_equal(host(got[key])[:off], host(ref[key])[:off], f"fused vs unfused {key}")
    n = h * off
    assert_bytes_equal(host(got["col_codes"])[: n // 2], host(ref["col_codes"])[: n // 2], "fused vs unfused col codes")


@pytest.mark.parametrize("case", [
    dict(seed=41, tokens=300, hidden=256, E=5, k=2, A=16, unused=0.05, empty=[3]),
    dict(seed=42, tokens=700, hidden=4096, E=3, k=1, A=16, unused=0.0, empty=[]),    # experts of > 256 rows
    dict(seed=43, tokens=257, hidden=512, E=16, k=8, A=128, unused=0.0, empty=[0, 15]),
    dict(seed=44, tokens=1000, hidden=128, E=1024, k=1, A=16, unused=0.0, empty=[]),
    dict(seed=45, tokens=400, hidden=448, E=6, k=2, A=16, unused=0.1, empty=[2]),     # a 192-column last tile
    dict(seed=46, tokens=90, hidden=64, E=3, k=2, A=16, unused=0.0, empty=[]),        # one 64-column tile
    dict(seed=47, tokens=64, hidden=16384, E=4, k=2, A=16, unused=0.0, empty=[]),     # the widest packed row
])
def test_direct_receive_kblock_layout(dev, case):
    """The K-blocked columnwise layout: the oracle's operand re-laid by oracle.kblock_layout,
    byte for byte; the rowwise operand and D_e as in the compact receive."""
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"], unused_frac=case["unused"], empty=case["empty"])
    h = case["hidden"]
    print(f"kblock receive case {case}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), w.num_experts, w.alignment)
    got = mtb.ep_nvfp4_direct_receive(packed, h, plan)           # compact, with D_e
    kb = {k: torch.empty_like(v) for k, v in got.items()}
    kb["col_scale"] = got["col_scale"].clone()
    mtb.ep_nvfp4_direct_receive_kblock(packed, h, plan, kb)
    want = orecv.direct_receive(onv.pack_rows(w.x_bits), h, w.topk_idx, w.num_experts, w.alignment)
    off = host(plan["offsets"]).astype(np.int64)
    n = h * int(off[-1])
    wc, ws = orecv.kblock_layout(want["col_codes"][: n // 2], want["col_scales"][: n // 16], off, h)
    assert_bytes_equal(host(kb["col_codes"])[: n // 2], wc, "K-block columnwise codes")
    assert_bytes_equal(host(kb["col_scales"])[: n // 16], ws, "K-block columnwise scales")
    for key in ("row_codes", "row_scales", "row_t"):
        assert_bytes_equal(host(kb[key])[: off[-1]], host(got[key])[: off[-1]], f"K-block receive {key}")


def _check_mxfp4_kblock(packed, h, plan, want, off):
    """The K-blocked MXFP4 receive: the rowwise operand as the compact one's, the
    columnwise operand the oracle's re-laid by K-blocks of 32-row scale blocks."""
    got = mtb.ep_mxfp4_direct_receive(packed, h, plan, kblock=True)
    assert_bytes_equal(host(got["row_codes"])[:off], want["row_codes"][:off], "mxfp4 K-blocked: rowwise codes")
    assert_bytes_equal(host(got["row_scales"])[:off], want["row_scales"][:off], "mxfp4 K-blocked: rowwise scales")
    n = h * off
    offs = host(plan["offsets"]).astype(np.int64)
    wc, ws = orecv.kblock_layout(want["col_codes"][: n // 2], want["col_scales"][: n // 32], offs, h, scale_rows=32)
    assert_bytes_equal(host(got["col_codes"])[: n // 2], wc, "mxfp4 K-blocked columnwise codes")
    assert_bytes_equal(host(got["col_scales"])[: n // 32], ws, "mxfp4 K-blocked columnwise scales")


def _check_mxfp4(got, want, off, h, exact=True):
    assert_bytes_equal(host(got["row_codes"])[:off], want["row_codes"][:off], "mxfp4 rowwise codes")
    assert_bytes_equal(host(got["row_scales"])[:off], want["row_scales"][:off], "mxfp4 rowwise scales")
    n = h * off
    gc, gs = host(got["col_codes"])[: n // 2], host(got["col_scales"])[: n // 32]
    if exact:
        assert_bytes_equal(gs, want["col_scales"][: n // 32], "mxfp4 columnwise scales")
        assert_bytes_equal(gc, want["col_codes"][: n // 2], "mxfp4 columnwise codes")
    else:
        tolerant_codes(F.unpack_nibbles(gc), F.unpack_nibbles(want["col_codes"][: n // 2]), gs,
                       want["col_scales"][: n // 32], "mxfp4 columnwise", block=32)


@pytest.mark.parametrize("h", [256, 512])
def test_receive_slow_blocks_with_padding(dev, h):
    """16-row blocks that take the two-step decode (a row with a tiny t) and
    also hold padding rows, with columns that are zero in every row of the
    block: the transform of an all-zero column is a pattern of signed zeros set
    by the sign vector, and its codes carry those signs.  Expert 0 holds one
    tiny row (zero in its first half) and padding; expert 1 ordinary rows;
    expert 2 a tiny row among ordinary ones.  The NVFP4 and MXFP4 receives in
    both layouts, byte for byte."""
    rng = np.random.default_rng(58 + h)
    tiny = rng.standard_normal((2, h)) * 1e-30
    tiny[0, : h // 2] = 0.0
    x = np.concatenate([tiny[:1], rng.standard_normal((20, h)), tiny[1:], rng.standard_normal((16, h))])
    topk = np.array([0] + [1] * 20 + [2] * 17, dtype=np.int32)[:, None]
    bits = _bits(x)
    print(f"slow blocks with padding h={h}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    packed_np = onv.pack_rows(bits)
    assert_bytes_equal(host(packed), packed_np, "pack")
    assert packed_np[0, h // 2 + h // 16:].view(np.float32)[0] < 2.0 ** -100   # the two-step decode's rows
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), 3, 32)
    plan_np = {k: host(v) for k, v in plan.items() if torch.is_tensor(v)}
    got = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    w = types.SimpleNamespace(topk_idx=topk, num_experts=3, alignment=32)
    _check_receive(dev, w, packed_np, got, plan_np, h)
    kb = {key: torch.empty_like(v) for key, v in got.items()}
    kb["col_scale"] = got["col_scale"].clone()
    mtb.ep_nvfp4_direct_receive_kblock(packed, h, plan, kb)
    want = orecv.direct_receive(packed_np, h, topk, 3, 32)
    off = plan_np["offsets"].astype(np.int64)
    n = h * int(off[-1])
    wc, ws = orecv.kblock_layout(want["col_codes"][: n // 2], want["col_scales"][: n // 16], off, h)
    assert_bytes_equal(host(kb["col_codes"])[: n // 2], wc, "K-blocked columnwise codes")
    assert_bytes_equal(host(kb["col_scales"])[: n // 16], ws, "K-blocked columnwise scales")
    g4 = mtb.ep_mxfp4_direct_receive(packed, h, plan)
    w4 = omx4.direct_receive(packed_np, h, topk, 3, 32)
    _check_mxfp4(g4, w4, int(off[-1]), h)
    _check_mxfp4_kblock(packed, h, plan, w4, int(off[-1]))

def test_mxfp4_kblock_operand_feeds_the_scaled_matrix_instruction(dev):
    """The K-blocked MXFP4 operand read as stored by gfx950's block-scaled matrix
    instruction (ep_mxfp4_kblock_tile: each lane 16 contiguous code bytes and one
    scale byte, no reshuffle) gives the product of the oracle's operand: 16 x 16
    tiles of A A^T over a full K-block (256 rows: two 128-value K steps) and over
    a short last block (a K step with K groups past its end), within the worst
    case of FP32 accumulation.  A tile that read a wrong byte, nibble or scale would be
    off by far more than that."""
    h = 512
    w = workloads.small_dispatch(59, 900, h, 3, 1, alignment=32)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), 3, 32)
    got = mtb.ep_mxfp4_direct_receive(packed, h, plan, kblock=True)
    want = omx4.direct_receive(onv.pack_rows(w.x_bits), h, w.topk_idx, 3, 32)
    off = want["offsets"].astype(np.int64)
    tried = 0
    for e in range(3):
        o, p = int(off[e]), int(off[e + 1] - off[e])
        if p == 0:
            continue
        codes = F.unpack_nibbles(want["col_codes"][h * o // 2 : h * (o + p) // 2].reshape(h, p // 2))
        vals = omx4.decode(codes, want["col_scales"][h * o // 32 : h * (o + p) // 32].reshape(h, p // 32))
        for kb in range((p + 255) // 256):
            r0, ln = 256 * kb, min(256, p - 256 * kb)
            blk = vals[:, r0 : r0 + ln]
            for ha, hb in ((0, 16), (128, 496), (240, 240)):
                print(f"mfma tile expert {e} K-block {kb} (len {ln}) rows {ha}, {hb}", flush=True)
                tile = host(mtb.ep_mxfp4_kblock_tile(got["col_codes"], got["col_scales"], h, o + r0, ln, ha, hb))
                ref = blk[ha : ha + 16] @ blk[hb : hb + 16].T
                bound = np.abs(blk[ha : ha + 16]) @ np.abs(blk[hb : hb + 16]).T
                # any summation order of 256 exact products in FP32: at most 255 roundings of 2^-24
                assert np.all(np.abs(tile.astype(np.float64) - ref) <= 2e-5 * bound + 1e-30), (e, kb, ha, hb)
                assert np.count_nonzero(ref) > 200
                # the check is sharp: pairing A's K groups with B's from the next group of
                # the step (a lane mapping off by one group) misses the bound everywhere
                perm = np.concatenate([np.roll(np.arange(min(128, ln - c)).reshape(-1, 32), 1, axis=0).ravel() + c
                                       for c in range(0, ln, 128)])
                off_by = blk[ha : ha + 16] @ blk[hb : hb + 16][:, perm].T
                if ln > 32:
                    assert np.mean(np.abs(off_by - ref) > 2e-5 * bound + 1e-30) > 0.9
                tried += 1
    assert tried >= 12

@pytest.mark.parametrize("case", [
    dict(seed=51, tokens=150, hidden=256, E=5, k=2, A=32, unused=0.05, empty=[3]),
    dict(seed=52, tokens=600, hidden=192, E=8, k=2, A=128, unused=0.0, empty=[]),     # a 64-column last tile
    dict(seed=53, tokens=333, hidden=64, E=3, k=1, A=64, unused=0.2, empty=[]),
    dict(seed=54, tokens=257, hidden=512, E=16, k=8, A=32, unused=0.0, empty=[0, 15]),
    dict(seed=55, tokens=700, hidden=4096, E=3, k=1, A=32, unused=0.0, empty=[]),     # experts of > 256 rows
    dict(seed=56, tokens=1000, hidden=128, E=1024, k=1, A=32, unused=0.0, empty=[]),  # the maximum expert count
])
def test_mxfp4_receive_bit_exact(dev, case):
    """The MXFP4 receive (rowwise re-quantization and RHT columnwise operand) equals
    the oracle byte for byte."""
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"], unused_frac=case["unused"], empty=case["empty"])
    h = case["hidden"]
    print(f"mxfp4 receive case {case}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), w.num_experts, w.alignment)
    got = mtb.ep_mxfp4_direct_receive(packed, h, plan)
    want = omx4.direct_receive(onv.pack_rows(w.x_bits), h, w.topk_idx, w.num_experts, w.alignment)
    _check_mxfp4(got, want, int(host(plan["offsets"])[-1]), h)
    _check_mxfp4_kblock(packed, h, plan, want, int(host(plan["offsets"])[-1]))


def test_mxfp4_receive_edge_rows(dev):
    """Zero, -0, subnormal, tiny-t (the two-step decode), huge-t, outlier and
    exact-tie rows routed among ordinary rows: byte for byte as well."""
    rng = np.random.default_rng(57)
    h = 256
    edge = _edge_rows(h, rng)
    x = np.concatenate([rng.standard_normal((70, h)) * 10.0 ** rng.uniform(-1, 1, (70, 1)), edge, edge, edge])
    x = x[rng.permutation(len(x))]
    bits = _bits(x)
    topk = np.argsort(-rng.standard_normal((len(x), 4)), axis=1)[:, :2].astype(np.int32)
    print("mxfp4 receive edge rows", bits.shape, flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(topk).to(dev), 4, 32)
    got = mtb.ep_mxfp4_direct_receive(packed, h, plan)
    want = omx4.direct_receive(onv.pack_rows(bits), h, topk, 4, 32)
    _check_mxfp4(got, want, int(host(plan["offsets"])[-1]), h)
    _check_mxfp4_kblock(packed, h, plan, want, int(host(plan["offsets"])[-1]))


@pytest.mark.parametrize("case", [
    dict(seed=61, tokens=150, hidden=256, E=5, k=2, A=16, unused=0.05, empty=[3]),
    dict(seed=62, tokens=600, hidden=192, E=8, k=2, A=128, unused=0.0, empty=[]),
    dict(seed=63, tokens=1000, hidden=128, E=1024, k=1, A=16, unused=0.0, empty=[]),
])
@pytest.mark.parametrize("words", ["element", "stream"])
def test_direct_receive_sr_bit_exact(dev, case, words):
    """Stochastic columnwise codes (R24, with either word mapping of R8) equal the
    oracle's byte for byte; the scales and the rowwise operand equal the deterministic
    receive's."""
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"], unused_frac=case["unused"], empty=case["empty"])
    h = case["hidden"]
    seed, base = 1234 + case["seed"], (1 << 33) + 5
    print(f"receive SR case {case} words={words}", flush=True)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), w.num_experts, w.alignment)
    ref = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    got = {k: torch.empty_like(v) for k, v in ref.items()}
    got["col_scale"] = ref["col_scale"].clone()
    sr = torch.tensor([seed, base], dtype=torch.int64, device=dev)
    mtb.ep_nvfp4_direct_receive_sr(packed, h, plan, got, sr, stream_words=words == "stream")
    want = orecv.direct_receive(onv.pack_rows(w.x_bits), h, w.topk_idx, w.num_experts, w.alignment, sr=(seed, base),
                                sr_mode=words)
    off = int(host(plan["offsets"])[-1])
    n = h * off
    assert_bytes_equal(host(got["col_codes"])[: n // 2], want["col_codes"][: n // 2], "SR columnwise codes")
    assert_bytes_equal(host(got["col_scales"])[: n // 16], host(ref["col_scales"])[: n // 16], "SR columnwise scales")
    for key in ("row_codes", "row_scales"):
        assert_bytes_equal(host(got[key])[:off], host(ref[key])[:off], f"SR receive {key}")


@pytest.mark.parametrize("h", [32, 96, 256, 4096, 7168])  # one to several 4 KiB load groups per row
def test_mxfp8_receive_bit_exact(dev, h):
    w = workloads.small_dispatch(11, 300, h, 6, 2, alignment=128, unused_frac=0.1)
    data, scales, _ = mtb.ep_mxfp8_pack(bf16_dev(w.x_bits, dev))
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), 6, 128)
    gd, gs = mtb.ep_mxfp8_direct_receive(data, scales, plan)
    wd, ws = omx.pack_rows(w.x_bits)
    src = host(plan["src_row"])
    ed, es = omx.grouped_receive(wd, ws, src)
    assert_bytes_equal(host(gd), ed, f"mxfp8 grouped data h={h}")
    assert_bytes_equal(host(gs), es, f"mxfp8 grouped scales h={h}")


# ------------------------------------------------------------------ dSwiGLU
@pytest.mark.parametrize("counts,ffn,dy_scales", [([0, 17, 64, 1, 0, 33], 64, None), ([5, 40, 0, 16, 1], 128, None),
                                                  ([300, 0, 129], 256, None), ([1], 64, None),
                                                  # tiny D (c = s*D below 2^-104: the general block path),
                                                  # huge values, and an all-zero expert
                                                  ([40, 24, 19, 8], 64, [1e-33, 1e32, 0.0, 1.0]),
                                                  # many experts, mostly empty (the offsets scan spans waves)
                                                  ([3] + [0] * 200 + [17] + [0] * 97 + [5], 64, None),
                                                  # the maximum expert count, one row each
                                                  ([1] * 1024, 64, None)])
def test_dswiglu_two_stage(dev, counts, ffn, dy_scales):
    w = workloads.small_dswiglu(sum(counts) + ffn, counts, ffn, dy_scales)
    print(f"dswiglu counts={counts} ffn={ffn} dy_scales={dy_scales}", flush=True)
    out = mtb.dswiglu_nvfp4_quant(bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev), i32_dev(w.counts, dev))
    dx = host(out["dx"])
    # stage 1: dX within one BF16 ulp of the float64 oracle; amax == max |dX_gpu| exactly
    want_dx = odsw.dswiglu(w.preact_bits, w.dy_bits)
    ulp = np.abs(dx.view(np.int16).astype(np.int64) - want_dx.view(np.int16).astype(np.int64))
    assert ulp.max(initial=0) <= 1, f"dX differs by {ulp.max()} ulp"
    am = host(out["amax"])
    assert_bytes_equal(am.view(np.uint32), odsw.expert_amax(dx, w.counts).view(np.uint32), "amax")
    # stage 2: the oracle quantizer on the GPU's own dX and amax
    q = odsw.fc1_grad_quant(dx, w.counts, am)
    assert_bytes_equal(host(out["row_scale"]).view(np.uint32), q["row_scale"].view(np.uint32), "D_row")
    assert_bytes_equal(host(out["col_scale"]).view(np.uint32), q["col_scale"].view(np.uint32), "D_col")
    # the quantizer follows R19/R20 to the last bit: byte for byte on the GPU's own dX
    n = q["col_codes"].size
    assert_bytes_equal(host(out["row_scales"]), q["row_scales"], "fc1 rowwise scales")
    assert_bytes_equal(host(out["row_codes"]), q["row_codes"], "fc1 rowwise codes")
    assert_bytes_equal(host(out["col_scales"])[: q["col_scales"].size], q["col_scales"], "fc1 columnwise scales")
    assert_bytes_equal(host(out["col_codes"])[:n], q["col_codes"], "fc1 columnwise codes")


def test_dswiglu_tiny_corner(dev):
    """Experts whose dX is FP32-subnormal-sized (dy scaled to ~1e-38 .. 1e-41): block
    maxima a with a / 6 below FP32's normal range and a subnormal D_row -- the
    corner where R19/R20 round fl32(a / 6) on the subnormal grid.  Stage 2 byte
    for byte; the oracle confirms the corner is reached."""
    counts = [40, 24, 19, 64, 8]
    w = workloads.small_dswiglu(91, counts, 64, [1e-36, 3e-37, 5e-38, 1e-34, 1.0])
    print(f"dswiglu tiny corner counts={counts}", flush=True)
    out = mtb.dswiglu_nvfp4_quant(bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev), i32_dev(w.counts, dev))
    dx, am = host(out["dx"]), host(out["amax"])
    want_dx = odsw.dswiglu(w.preact_bits, w.dy_bits)
    ulp = np.abs(dx.view(np.int16).astype(np.int64) - want_dx.view(np.int16).astype(np.int64))
    assert ulp.max(initial=0) <= 1
    assert_bytes_equal(am.view(np.uint32), odsw.expert_amax(dx, w.counts).view(np.uint32), "amax")
    q = odsw.fc1_grad_quant(dx, w.counts, am)
    D = (am / np.float32(2688.0)).astype(np.float32)
    assert (D[:3] < 2.0 ** -126).all() and (D[:3] > 0).all()          # subnormal D_row
    a_b = np.abs(F.bf16_to_f32(dx[:83])).reshape(83, -1, 16).max(axis=-1)
    assert ((a_b / np.float32(6) < 2.0 ** -126) & (a_b > 0)).sum() > 100
    n = q["col_codes"].size
    assert_bytes_equal(host(out["row_scale"]).view(np.uint32), q["row_scale"].view(np.uint32), "D_row")
    # R20: D_col = fl32(4 amax / 2688), which is not 4 D_row once D_row is subnormal
    assert_bytes_equal(host(out["col_scale"]).view(np.uint32), q["col_scale"].view(np.uint32), "D_col")
    assert (q["col_scale"][:3] != np.float32(4) * q["row_scale"][:3]).any()
    assert_bytes_equal(host(out["row_scales"]), q["row_scales"], "tiny rowwise scales")
    assert_bytes_equal(host(out["row_codes"]), q["row_codes"], "tiny rowwise codes")
    assert_bytes_equal(host(out["col_scales"])[: q["col_scales"].size], q["col_scales"], "tiny columnwise scales")
    assert_bytes_equal(host(out["col_codes"])[:n], q["col_codes"], "tiny columnwise codes")


@pytest.mark.parametrize("dev_counts,rows", [([30, 40], 50), ([-5, 50, 7], 50), ([0, 0], 9)])
def test_dswiglu_counts_cut_at_tokens(dev, dev_counts, rows):
    """Counts are device data: a negative count is 0 and the running total is cut
    at the token count, so the call reads and writes only the tokens' rows; the
    result is the oracle's for the counts so cut."""
    cut, run = [], 0
    for c in dev_counts:
        c = min(max(c, 0), rows - run)
        cut.append(c)
        run += c
    w = workloads.small_dswiglu(rows + 11, [rows], 64)
    print(f"dswiglu device counts={dev_counts} rows={rows} -> {cut}", flush=True)
    out = mtb.dswiglu_nvfp4_quant(bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev),
                                  i32_dev(np.array(dev_counts, dtype=np.int32), dev))
    dx, am = host(out["dx"]), host(out["amax"])
    cut = np.array(cut, dtype=np.int32)
    assert_bytes_equal(am.view(np.uint32), odsw.expert_amax(dx[: cut.sum()], cut).view(np.uint32), "amax")
    if cut.sum() == 0:
        return
    q = odsw.fc1_grad_quant(dx[: cut.sum()], cut, am)
    n = int(cut.sum())
    tolerant_codes(F.unpack_nibbles(host(out["row_codes"])[:n]), F.unpack_nibbles(q["row_codes"]),
                   host(out["row_scales"])[:n], q["row_scales"], "cut rowwise")
    m = q["col_codes"].size
    tolerant_codes(F.unpack_nibbles(host(out["col_codes"])[:m]), F.unpack_nibbles(q["col_codes"]),
                   host(out["col_scales"])[: q["col_scales"].size], q["col_scales"], "cut columnwise")


@pytest.mark.parametrize("words", ["element", "stream"])
@pytest.mark.parametrize("counts,ffn", [([0, 17, 64, 1, 0, 33], 64), ([300, 0, 129], 256), ([40, 24, 19, 8], 128)])
def test_dswiglu_sr_bit_exact(dev, counts, ffn, words):
    """Stochastic FC1-gradient codes (R24, with either word mapping of R8) equal the
    oracle's on the GPU's own dX and amax byte for byte, with and without a
    materialized dX; scales as the RNE call's."""
    w = workloads.small_dswiglu(sum(counts) + 3 * ffn, counts, ffn)
    print(f"dswiglu SR counts={counts} ffn={ffn} words={words}", flush=True)
    args = (bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev), i32_dev(w.counts, dev))
    seed, base = 777, (1 << 32) + 3
    sr = torch.tensor([seed, base], dtype=torch.int64, device=dev)
    sw = words == "stream"
    got = mtb.dswiglu_nvfp4_quant(*args, sr_state=sr, stream_words=sw)
    got_nodx = mtb.dswiglu_nvfp4_quant(*args, materialize_dx=False, sr_state=sr, stream_words=sw)
    ref = mtb.dswiglu_nvfp4_quant(*args)
    q = odsw.fc1_grad_quant(host(got["dx"]), w.counts, host(got["amax"]), sr=(seed, base), sr_mode=words)
    t = sum(counts)
    n = 2 * ffn * sum((c + 15) // 16 * 16 for c in counts)
    assert_bytes_equal(host(got["row_codes"]), q["row_codes"], "SR rowwise codes")
    assert_bytes_equal(host(got["col_codes"])[: n // 2], q["col_codes"], "SR columnwise codes")
    for key in ("row_scales", "col_scales"):
        m = n // 16 if key == "col_scales" else None
        assert_bytes_equal(host(got[key])[:m], host(ref[key])[:m], f"SR {key}")
    for key in ("row_codes", "row_scales", "col_codes", "col_scales"):
        m = (n // 2 if key == "col_codes" else n // 16) if key.startswith("col") else None
        assert_bytes_equal(host(got_nodx[key])[:m], host(got[key])[:m], f"SR recompute {key}")


@pytest.mark.parametrize("counts,ffn", [([0, 17, 64, 1, 0, 33], 64), ([300, 0, 129], 256), ([40, 24, 19, 8], 128)])
def test_dswiglu_without_dx(dev, counts, ffn):
    """dX not materialized: the quantizer recomputes it; every output equals the
    materializing call's byte for byte (and that call is checked against the oracle above)."""
    w = workloads.small_dswiglu(sum(counts) + 7 * ffn, counts, ffn)
    print(f"dswiglu recompute counts={counts} ffn={ffn}", flush=True)
    args = (bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev), i32_dev(w.counts, dev))
    ref = mtb.dswiglu_nvfp4_quant(*args)
    got = mtb.dswiglu_nvfp4_quant(*args, materialize_dx=False)
    assert got["dx"] is None
    t = sum(counts)
    for key in ("amax", "row_scale", "col_scale", "row_codes", "row_scales", "col_codes", "col_scales"):
        g, r = host(got[key]), host(ref[key])
        if key in ("col_codes", "col_scales"):
            n = 2 * ffn * sum((c + 15) // 16 * 16 for c in counts) // (2 if key == "col_codes" else 16)
            g, r = g[:n], r[:n]
        assert_bytes_equal(g, r, f"recompute {key}")
    # and against the oracle quantizer on the materialized dX
    q = odsw.fc1_grad_quant(host(ref["dx"]), w.counts, host(ref["amax"]))
    tolerant_codes(F.unpack_nibbles(host(got["row_codes"])), F.unpack_nibbles(q["row_codes"]),
                   host(got["row_scales"]), q["row_scales"], "recompute rowwise")


# ------------------------------------------------------------------ determinism and graph capture
def test_deterministic_and_graph_capturable(dev):
    w = workloads.small_dispatch(21, 700, 512, 8, 2, unused_frac=0.02)
    x = bf16_dev(w.x_bits, dev)
    topk = torch.from_numpy(w.topk_idx).to(dev)
    plan = mtb.ep_route_plan(topk, 8, 16)
    packed = mtb.ep_nvfp4_pack(x)
    ref = mtb.ep_nvfp4_direct_receive(packed, 512, plan)
    again = mtb.ep_nvfp4_direct_receive(packed, 512, mtb.ep_route_plan(topk, 8, 16))
    off = int(plan["offsets"][-1])          # rows from off_E on are not written by the receive
    for k in ("row_codes", "row_scales", "row_t"):
        assert torch.equal(ref[k][:off], again[k][:off]), k
    assert torch.equal(ref["col_codes"][: 256 * off], again["col_codes"][: 256 * off])
    assert torch.equal(ref["col_scales"][: 32 * off], again["col_scales"][: 32 * off])
    assert torch.equal(ref["col_scale"], again["col_scale"])
    # capture pack -> route -> receive in one HIP graph; replay several times with
    # eager work in between and check every replay against the eager result
    out_p = torch.empty_like(packed)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    derr = torch.zeros(1, dtype=torch.int32, device=dev)
    outs = {k: torch.empty_like(v) for k, v in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                       # warm-up on a side stream before capture
        mtb.ep_nvfp4_pack(x, out=out_p)
        wplan = mtb.ep_route_plan(topk, 8, 16, d_error=derr, workspace=ws)
        mtb.ep_nvfp4_direct_receive(out_p, 512, wplan, out=outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mtb.ep_nvfp4_pack(x, out=out_p)
        gplan = mtb.ep_route_plan(topk, 8, 16, d_error=derr, workspace=ws)
        mtb.ep_nvfp4_direct_receive(out_p, 512, gplan, out=outs)
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        out_p.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_p, packed), rep
        assert torch.equal(gplan["src_row"], plan["src_row"]), rep
        assert torch.equal(gplan["dst_row"], plan["dst_row"]), rep
        off = int(plan["offsets"][-1])
        for k in ("row_codes", "row_scales", "row_t"):
            assert torch.equal(outs[k][:off], ref[k][:off]), (rep, k)
        n = 512 * off
        assert torch.equal(outs["col_codes"][: n // 2], ref["col_codes"][: n // 2]), rep
        assert torch.equal(outs["col_scales"][: n // 16], ref["col_scales"][: n // 16]), rep
        assert torch.equal(outs["col_scale"], ref["col_scale"]), rep
