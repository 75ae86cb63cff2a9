"""bench.py's algorithmic byte counts (distinct inputs read once + outputs,
padding rows excluded) against the per-configuration figures worked out by hand
from the formats: packed row = 9H/16 + 4 bytes, MXFP8 row = H + H/32, grouped
operands of R = T*k routed rows.  Host only."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _mb(x):
    return round(x / 1e6, 1)


def test_dispatch_bytes_per_configuration():
    # config 2: 4096 x 4096, top-2 of 8, alignment 16
    T, H, k, E = 4096, 4096, 2, 8
    b = bench.dispatch_bytes(T, H, k, E, T * k + E * 15, T * k)
    assert _mb(b["nvfp4_pack"]) == 43.0            # 2 B in + 2308 B per row out
    assert _mb(b["mxfp8_pack"]) == 50.9            # 2 B in + 1 + 1/32 B out per element
    assert _mb(b["nvfp4_direct_receive"]) == 47.3  # rows once in + rowwise + columnwise out
    assert _mb(b["mxfp8_receive"]) == 51.9
    # config 3: 16384 x 7168, top-8 of 32
    T, H, k, E = 16384, 7168, 8, 32
    b = bench.dispatch_bytes(T, H, k, E, T * k + E * 15, T * k)
    assert _mb(b["nvfp4_pack"]) == 301.0
    assert _mb(b["nvfp4_direct_receive"]) == 1124.1
    assert b["nvfp4_direct_receive_kblock"] == b["nvfp4_direct_receive"]   # same bytes, re-placed
    # MXFP4 receive: rows once in + rowwise and columnwise codes (H/2) and scales (H/32) per grouped row
    assert b["mxfp4_receive"] == T * (9 * H // 16 + 4) + (T * k + E * 15) * 4 + (E + 1) * 4 + 2 * T * k * (H // 2 + H // 32)
    assert b["mxfp4_receive_kblock"] == b["mxfp4_receive"]
    # the unpack of the routed rows: packed rows once in, R rows of BF16 out
    assert b["nvfp4_unpack"] == T * (9 * H // 16 + 4) + T * k * 4 + T * k * H * 2
    assert _mb(b["nvfp4_unpack_tokens"]) == 301.0   # one row per token
    # config 4: 32768 x 4096, top-2 of 16
    T, H, k, E = 32768, 4096, 2, 16
    b = bench.dispatch_bytes(T, H, k, E, T * k + E * 15, T * k)
    assert _mb(b["nvfp4_pack_sr"]) == 344.1
    assert _mb(b["nvfp4_direct_receive"]) == 378.1


def test_dswiglu_bytes_and_kernel_split():
    T, F, E = 14841, 2048, 8
    split = bench.dswiglu_kernel_bytes(T, F, E)
    assert _mb(split["k_dswiglu_epilogue"]) == 303.9   # preact + dy in, dX out
    assert _mb(split["k_fc1_quant"]) == 190.0          # dX in, both NVFP4 operands out
    # the call counts dX once (written, not re-read) and reads the per-expert counts:
    # the two kernels' bytes minus one dX, plus the counts
    assert bench.dswiglu_bytes(T, F, E) == sum(split.values()) - T * 2 * F * 2 + E * 4


def test_source_hash_ignores_comments():
    assert bench._code_only("int a; // note\n/* block\n comment */ int  b;\n") == "inta;intb;"
