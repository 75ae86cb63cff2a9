"""A seeded sweep of random small dispatch shapes, every output compared with the
oracle byte for byte: the pack, the routing plan, the direct receive in both
columnwise layouts, the unpack of the routed rows and (for 32-row alignments)
the MXFP4 receive.  The shapes are drawn once from a fixed seed: ragged token
counts, widths from one to many 256-column tiles with partial last tiles,
expert counts up to 80 with empty experts, every alignment the plan accepts up
to 256, and unused (-1) slots."""

import numpy as np
import pytest
import torch

import moe_token_block_amd as mtb
import workloads
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
