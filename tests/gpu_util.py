"""Helpers for the GPU parity tests: host <-> device transfer and the comparison bars."""

import numpy as np
import torch

from oracle import formats as F


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (run them with -m gpu on an MI355X)")
    return torch.device("cuda:0")


def bf16_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def i32_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)
    if bad[0].size:
        idx = tuple(b[:5] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} of {got.size} differ; first at {idx}: "
                             f"got {got[idx]} want {want[idx]}")


def tolerant_codes(got_codes, want_codes, got_sc, want_sc, what, frac=1e-4, block=16):
    """The bar for values derived from FP32 amaxes / post-RHT values: block scales
    differ by at most one E4M3 step in at most ``frac`` of blocks; where the scales
    agree, E2M1 codes differ by at most one grid step in at most ``frac`` of
    elements; where they differ, the decoded values are within one grid step at
    the larger scale.  Codes are unpacked 4-bit codes [..., 16 * nblocks] laid
    out block-major along the last axis, scales [..., nblocks]; ``block`` elements
    per scale (16 for NVFP4, 32 for MXFP4, whose scale steps are powers of two)."""
    gc = np.asarray(got_codes, dtype=np.int64)
    wc = np.asarray(want_codes, dtype=np.int64)
    gs = np.asarray(got_sc, dtype=np.int64)
    ws = np.asarray(want_sc, dtype=np.int64)
    assert gc.shape == wc.shape and gs.shape == ws.shape, what
    nblk = gs.size
    sdiff = np.abs(gs - ws)
    assert sdiff.max(initial=0) <= 1, f"{what}: a block scale differs by {sdiff.max()} E4M3 steps"
    assert (sdiff > 0).sum() <= max(0, frac * nblk), f"{what}: {(sdiff > 0).sum()} of {nblk} block scales differ"
    same = np.repeat((sdiff == 0).reshape(gs.shape), block, axis=-1)
    # one grid step: same sign and adjacent magnitude index (or +-0 vs the smallest step)
    gv = F.e2m1_value(gc.astype(np.uint8)) * 2
    wv = F.e2m1_value(wc.astype(np.uint8)) * 2
    gi = np.where(gv < 0, -1, 1) * (gc & 7)
    wi = np.where(wv < 0, -1, 1) * (wc & 7)
    code_diff = np.abs(gi - wi)
    cd = code_diff[same]
    assert cd.max(initial=0) <= 1, f"{what}: an E2M1 code differs by {cd.max()} steps"
    n_bad = (gc != wc).sum()
    assert n_bad <= frac * gc.size, f"{what}: {n_bad} of {gc.size} codes differ"
    return int(n_bad), int((sdiff > 0).sum())
