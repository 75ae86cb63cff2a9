"""Seeded sweeps of random small shapes, every output compared with the oracle
byte for byte.  Dispatch: the pack, the routing plan, the direct receive in
both columnwise layouts, the unpack of the routed rows and (for 32-row
alignments) the MXFP4 receive in both layouts; dSwiGLU: the epilogue and the FC1-gradient
operands, with and without a materialized dX; stochastic rounding: the pack in
each word mapping and rule, and the receive's stochastic columnwise codes.  The shapes are drawn once from
fixed seeds: ragged token counts, widths from one to many 256-column tiles with
partial last tiles, expert counts up to 80 with empty experts, every alignment
the plan accepts up to 256, unused (-1) slots, and grouped row counts that are
not multiples of 16 with an occasional large expert."""

import numpy as np
import pytest
import torch

import moe_token_block_amd as mtb
import workloads
from oracle import dswiglu as odsw
from oracle import mxfp4 as omx4
from oracle import nvfp4 as onv
from oracle import receive as orecv
from oracle.routing import route_plan as o_route

from gpu_util import require_gpu, bf16_dev, host, i32_dev, assert_bytes_equal

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 81))
        n_empty = int(rng.integers(0, E // 2 + 1)) if E > 1 else 0
        empty = sorted(int(e) for e in rng.choice(E, size=n_empty, replace=False)) if n_empty else []
        k = int(rng.integers(1, min(8, E - len(empty)) + 1))
        out.append(dict(seed=1000 + i, tokens=int(rng.integers(1, 501)), hidden=64 * int(rng.integers(1, 25)),
                        E=E, k=k, A=int(rng.choice([16, 32, 48, 64, 128, 256])),
                        unused=float(rng.choice([0.0, 0.1, 0.3])), empty=empty))
    return out


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"s{c['seed']}-t{c['tokens']}-h{c['hidden']}-e{c['E']}-k{c['k']}-a{c['A']}")
def test_dispatch_sweep(dev, case):
    print(f"sweep case {case}", flush=True)
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"], unused_frac=case["unused"], empty=case["empty"])
    h, E, A = case["hidden"], case["E"], case["A"]
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev))
    packed_np = onv.pack_rows(w.x_bits)
    assert_bytes_equal(host(packed), packed_np, "pack")
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), E, A)
    want_plan = o_route(w.topk_idx, E, A)
    for key in ("counts", "offsets", "dst_row", "src_row"):
        assert_bytes_equal(host(plan[key]), want_plan[key], f"route {key}")
    off = int(want_plan["offsets"][-1])
    want = orecv.direct_receive(packed_np, h, w.topk_idx, E, A)
    got = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    for key in ("row_codes", "row_scales"):
        assert_bytes_equal(host(got[key])[:off], want[key][:off], key)
    assert_bytes_equal(host(got["row_t"])[:off].view(np.uint32), want["row_t"][:off].view(np.uint32), "row t")
    assert_bytes_equal(host(got["col_scale"]).view(np.uint32), want["col_scale"].view(np.uint32), "D_e")
    n = h * off
    assert_bytes_equal(host(got["col_scales"])[: n // 16], want["col_scales"][: n // 16], "columnwise scales")
    assert_bytes_equal(host(got["col_codes"])[: n // 2], want["col_codes"][: n // 2], "columnwise codes")
    kb = {key: torch.empty_like(v) for key, v in got.items()}
    kb["col_scale"] = got["col_scale"].clone()
    mtb.ep_nvfp4_direct_receive_kblock(packed, h, plan, kb)
    wc, ws = orecv.kblock_layout(want["col_codes"][: n // 2], want["col_scales"][: n // 16],
                                 want_plan["offsets"].astype(np.int64), h)
    assert_bytes_equal(host(kb["col_codes"])[: n // 2], wc, "K-blocked columnwise codes")
    assert_bytes_equal(host(kb["col_scales"])[: n // 16], ws, "K-blocked columnwise scales")
    src = want_plan["src_row"][:off]
    routed = src[src >= 0]
    if routed.size:
        un = mtb.ep_nvfp4_unpack(packed, h, src_row=i32_dev(routed, dev))
        assert_bytes_equal(host(un), onv.unpack_rows(packed_np, h, routed), "unpack of the routed rows")
    if A % 32 == 0:
        g4 = mtb.ep_mxfp4_direct_receive(packed, h, plan)
        w4 = omx4.direct_receive(packed_np, h, w.topk_idx, E, A)
        for key in ("row_codes", "row_scales"):
            assert_bytes_equal(host(g4[key])[:off], w4[key][:off], f"MXFP4 {key}")
        assert_bytes_equal(host(g4["col_codes"])[: n // 2], w4["col_codes"][: n // 2], "MXFP4 columnwise codes")
        assert_bytes_equal(host(g4["col_scales"])[: n // 32], w4["col_scales"][: n // 32], "MXFP4 columnwise scales")
        k4 = mtb.ep_mxfp4_direct_receive(packed, h, plan, kblock=True)
        for key in ("row_codes", "row_scales"):
            assert_bytes_equal(host(k4[key])[:off], w4[key][:off], f"MXFP4 K-blocked {key}")
        wc4, ws4 = orecv.kblock_layout(w4["col_codes"][: n // 2], w4["col_scales"][: n // 32],
                                       want_plan["offsets"].astype(np.int64), h, scale_rows=32)
        assert_bytes_equal(host(k4["col_codes"])[: n // 2], wc4, "MXFP4 K-blocked columnwise codes")
        assert_bytes_equal(host(k4["col_scales"])[: n // 32], ws4, "MXFP4 K-blocked columnwise scales")


def _dswiglu_cases(n=12, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 41))
        counts = rng.integers(0, 300, size=E)
        counts[rng.random(E) < 0.2] = 0                       # empty experts
        if rng.random() < 0.3:
            counts[int(rng.integers(0, E))] = int(rng.integers(700, 1500))   # one large expert
        if counts.sum() == 0:
            counts[0] = 1
        out.append(dict(seed=2000 + i, counts=[int(c) for c in counts], ffn=64 * int(rng.integers(1, 25))))
    return out


@pytest.mark.parametrize("case", _dswiglu_cases(), ids=lambda c: f"s{c['seed']}-e{len(c['counts'])}-f{c['ffn']}")
def test_dswiglu_sweep(dev, case):
    """dSwiGLU + FC1-grad quantization on random grouped shapes: dX within one BF16
    ulp of float64 and the amax exact (stage 1); the oracle quantizer on the GPU's
    own dX and amax byte for byte (stage 2); the recompute form (no dX) equal to
    the materializing call in every operand byte."""
    counts, ffn = case["counts"], case["ffn"]
    print(f"dswiglu sweep case seed={case['seed']} E={len(counts)} rows={sum(counts)} ffn={ffn}", flush=True)
    w = workloads.small_dswiglu(case["seed"], counts, ffn)
    args = (bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev), i32_dev(w.counts, dev))
    out = mtb.dswiglu_nvfp4_quant(*args)
    dx = host(out["dx"])
    want_dx = odsw.dswiglu(w.preact_bits, w.dy_bits)
    ulp = np.abs(dx.view(np.int16).astype(np.int64) - want_dx.view(np.int16).astype(np.int64))
    assert ulp.max(initial=0) <= 1, f"dX differs by {ulp.max()} ulp"
    am = host(out["amax"])
    assert_bytes_equal(am.view(np.uint32), odsw.expert_amax(dx, w.counts).view(np.uint32), "amax")
    q = odsw.fc1_grad_quant(dx, w.counts, am)
    for key in ("row_scale", "col_scale"):
        assert_bytes_equal(host(out[key]).view(np.uint32), q[key].view(np.uint32), key)
    assert_bytes_equal(host(out["row_scales"]), q["row_scales"], "rowwise scales")
    assert_bytes_equal(host(out["row_codes"]), q["row_codes"], "rowwise codes")
    assert_bytes_equal(host(out["col_scales"])[: q["col_scales"].size], q["col_scales"], "columnwise scales")
    assert_bytes_equal(host(out["col_codes"])[: q["col_codes"].size], q["col_codes"], "columnwise codes")
    rec = mtb.dswiglu_nvfp4_quant(*args, materialize_dx=False)
    for key in ("amax", "row_scale", "col_scale", "row_codes", "row_scales"):
        assert_bytes_equal(host(rec[key]), host(out[key]), f"recompute {key}")
    assert_bytes_equal(host(rec["col_codes"])[: q["col_codes"].size], q["col_codes"], "recompute columnwise codes")
    assert_bytes_equal(host(rec["col_scales"])[: q["col_scales"].size], q["col_scales"], "recompute columnwise scales")


def _sr_cases(n=8, seed=20261204):
    rng = np.random.default_rng(seed)
    return [dict(seed=3000 + i, tokens=int(rng.integers(1, 400)), hidden=64 * int(rng.integers(1, 25)),
                 E=int(rng.integers(2, 33)), k=int(rng.integers(1, 3)), A=int(rng.choice([16, 32, 64, 128])),
                 mode=int(rng.integers(1, 5)), sr_seed=int(rng.integers(0, 1 << 62)),
                 base=int(rng.integers(0, 1 << 40))) for i in range(n)]


@pytest.mark.parametrize("case", _sr_cases(), ids=lambda c: f"s{c['seed']}-t{c['tokens']}-h{c['hidden']}-m{c['mode']}")
def test_stochastic_sweep(dev, case):
    """The stochastic-rounding pack in a random word mapping and rule, and the
    receive's stochastic columnwise codes (element words in even cases, stream words in
    odd ones), on random shapes, seeds and counter bases."""
    print(f"SR sweep case {case}", flush=True)
    w = workloads.small_dispatch(case["seed"], case["tokens"], case["hidden"], case["E"], case["k"],
                                 alignment=case["A"])
    h, mode = case["hidden"], case["mode"]
    st = torch.tensor([case["sr_seed"], case["base"]], dtype=torch.int64, device=dev)
    packed = mtb.ep_nvfp4_pack(bf16_dev(w.x_bits, dev), round_mode=mode, sr_state=st)
    want_p = onv.pack_rows(w.x_bits, sr_seed=case["sr_seed"], sr_counter_base=case["base"],
                           sr_mode="element" if mode in (1, 3) else "stream", sr_rule="carry" if mode >= 3 else "threshold")
    assert_bytes_equal(host(packed), want_p, f"SR pack mode {mode}")
    plan = mtb.ep_route_plan(torch.from_numpy(w.topk_idx).to(dev), w.num_experts, w.alignment)
    ref = mtb.ep_nvfp4_direct_receive(packed, h, plan)
    got = {key: torch.empty_like(v) for key, v in ref.items()}
    got["col_scale"] = ref["col_scale"].clone()
    rs = torch.tensor([case["sr_seed"] ^ 0x5A5A, case["base"] + 17], dtype=torch.int64, device=dev)
    words = "stream" if case["seed"] % 2 else "element"   # both word mappings of the receive's codes
    mtb.ep_nvfp4_direct_receive_sr(packed, h, plan, got, rs, stream_words=words == "stream")
    want = orecv.direct_receive(want_p, h, w.topk_idx, w.num_experts, w.alignment,
                                sr=(case["sr_seed"] ^ 0x5A5A, case["base"] + 17), sr_mode=words)
    off = int(host(plan["offsets"])[-1])
    n = h * off
    assert_bytes_equal(host(got["col_codes"])[: n // 2], want["col_codes"][: n // 2], "SR columnwise codes")
    assert_bytes_equal(host(got["col_scales"])[: n // 16], want["col_scales"][: n // 16], "SR columnwise scales")
