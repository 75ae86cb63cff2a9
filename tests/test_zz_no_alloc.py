"""The allocation-free entry point dswiglu_nvfp4_quant_noalloc, called through
the C ABI, against dswiglu_nvfp4_quant (the same computation with a caller
workspace): every output byte for byte, on two calls in a row, the second with
a smaller input (the static scratch keeps the first call's contents)."""

import ctypes

import numpy as np
import pytest
import torch

import moe_token_block_amd as mtb
import workloads

from gpu_util import require_gpu, bf16_dev, host, i32_dev, assert_bytes_equal

pytestmark = pytest.mark.gpu


def _outputs(t, f, e, dev, fill):
    cap = t + 15 * e
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    return dict(dx=torch.full((t, 2 * f), fill, dtype=torch.bfloat16, device=dev),
                amax=torch.full((e,), fill, **f32), row_codes=torch.full((t, f), fill, **u8),
                row_scales=torch.full((t, 2 * f // 16), fill, **u8), row_scale=torch.full((e,), fill, **f32),
                col_codes=torch.full((2 * f * cap // 2,), fill, **u8),
                col_scales=torch.full((2 * f * cap // 16,), fill, **u8), col_scale=torch.full((e,), fill, **f32))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_equals_workspace_entry_point(order):
    dev = require_gpu()
    lib = mtb.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    for seed, counts, ffn in ((101, [300, 0, 129, 57, 1], 256), (102, [17, 5], 128)):
        w = workloads.small_dswiglu(seed, counts, ffn)
        pre, dy, cnt = bf16_dev(w.preact_bits, dev), bf16_dev(w.dy_bits, dev), i32_dev(w.counts, dev)
        t, f, e = int(sum(counts)), ffn, len(counts)
        print(f"noalloc counts={counts} ffn={ffn}", flush=True)
        ref = mtb.dswiglu_nvfp4_quant(pre, dy, cnt)
        out = _outputs(t, f, e, dev, 77)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = lib.dswiglu_nvfp4_quant_noalloc(P(pre), P(dy), t, f, P(cnt), e, P(out["dx"]), P(out["amax"]),
                                             P(out["row_codes"]), P(out["row_scales"]), P(out["row_scale"]),
                                             P(out["col_codes"]), P(out["col_scales"]), P(out["col_scale"]), stream)
        assert st == 0, mtb.ep_status_string(st)
        torch.cuda.synchronize(dev)
        n = 2 * f * sum((c + 15) // 16 * 16 for c in counts)
        for key in ("dx", "amax", "row_codes", "row_scales", "row_scale", "col_scale"):
            assert_bytes_equal(host(out[key]), host(ref[key]), f"noalloc {key} (counts {counts})")
        assert_bytes_equal(host(out["col_codes"])[: n // 2], host(ref["col_codes"])[: n // 2],
                           f"noalloc col_codes (counts {counts})")
        assert_bytes_equal(host(out["col_scales"])[: n // 16], host(ref["col_scales"])[: n // 16],
                           f"noalloc col_scales (counts {counts})")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    dev = require_gpu()
    lib = mtb.lib()
    big = 1_100_000                     # its workspace needs more than EP_NOALLOC_SCRATCH_BYTES
    assert lib.dswiglu_workspace_bytes(big, 8) > mtb.EP_NOALLOC_SCRATCH_BYTES
    assert lib.dswiglu_workspace_bytes(1_000_000, 1024) <= mtb.EP_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.uint8, device=dev)
    p = ctypes.c_void_p(dummy.data_ptr())
    st = lib.dswiglu_nvfp4_quant_noalloc(p, p, big, 64, p, 8, p, p, p, p, p, p, p, p, None)
    assert st == mtb.EP_ERR_SCRATCH           # refused on the host: nothing launched
    torch.cuda.synchronize(dev)
