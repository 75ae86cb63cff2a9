"""Host-side checks of the C-ABI library (CPU, no GPU needed): it builds, loads,
exports every symbol the header declares, and rejects invalid arguments with
the documented status codes before launching anything."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_token_block.h")


@pytest.fixture(scope="module")
def lib():
    from moe_token_block_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    import moe_token_block_amd as m
    return m.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", src, flags=re.M)) - {"defined"})


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("ep_nvfp4_pack", "ep_nvfp4_unpack", "ep_nvfp4_direct_receive", "ep_mxfp8_pack",
              "dswiglu_nvfp4_quant", "ep_route_plan", "ep_mxfp8_direct_receive"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from moe_token_block_amd import LIB_PATH, EXPORTS
    names = _declared()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    assert not [e for e in exported if e.startswith("_Z")], "C++ symbols leak from the ABI library"


def test_helpers(lib):
    import moe_token_block_amd as m
    assert m.ep_abi_version() == 1
    assert m.ep_nvfp4_packed_row_bytes(1024) == 580          # 512 code bytes + 64 scales + 4
    assert m.ep_nvfp4_packed_row_bytes(100) == -2
    assert m.ep_route_capacity(4096, 2, 8, 16) == 8312
    assert lib.ep_route_capacity(1, 1, 1, 24) == -3
    assert m.ep_rht_sign_mask() == 0xE8D5
    assert m.ep_status_string(-4).startswith("r_cap")
    assert lib.dswiglu_workspace_bytes(10, 8) == 72 + 48  # offsets + row maxima padded to 4 rows


@pytest.mark.skipif(torch.cuda.is_available(), reason="passes fake pointers: only where no GPU exists")
def test_argument_validation_before_launch(lib):
    P = ctypes.c_void_p(0x1000)          # never dereferenced: every call below must fail validation
    N = None
    assert lib.ep_nvfp4_pack(P, 4, 100, P, 0, N, N) == -2           # hidden % 64
    assert lib.ep_nvfp4_pack(P, 4, 32768, P, 0, N, N) == -2         # hidden too large
    assert lib.ep_nvfp4_pack(P, -1, 128, P, 0, N, N) == -2
    assert lib.ep_nvfp4_pack(N, 4, 128, P, 0, N, N) == -1
    assert lib.ep_nvfp4_pack(P, 4, 128, P, 1, N, N) == -1           # SR without state
    assert lib.ep_nvfp4_pack(P, 4, 128, P, 7, N, N) == -5
    assert lib.ep_nvfp4_pack(P, 4, 128, P, 5, N, N) == -5           # past the last SR mode
    assert lib.ep_nvfp4_pack(P, 4, 128, P, 3, N, N) == -1           # carry-form SR without state
    assert lib.ep_nvfp4_pack_scatter(P, 4, 128, 33, P, 4, 64, P, P, P, P, P, N) == -8   # top_k > 32
    assert lib.ep_nvfp4_pack_scatter(P, 4, 100, 2, P, 4, 64, P, P, P, P, P, N) == -2    # hidden % 64
    assert lib.ep_nvfp4_pack_scatter(P, 4, 128, 2, P, 0, 64, P, P, P, P, P, N) == -2    # no experts
    assert lib.ep_nvfp4_pack_scatter(P, 4, 128, 2, N, 4, 64, P, P, P, P, P, N) == -1    # no dst_row
    assert lib.ep_nvfp4_columnwise_grouped(P, P, P, 100, 4, 64, P, P, P, P, N) == -2
    assert lib.ep_nvfp4_columnwise_grouped(P, P, P, 128, 1025, 64, P, P, P, P, N) == -2
    assert lib.ep_nvfp4_columnwise_grouped(P, P, P, 128, 4, 64, N, P, P, P, N) == -1
    assert lib.ep_nvfp4_pack(P, 0, 128, N, 0, N, N) == 0            # empty: nothing to do
    assert lib.ep_mxfp8_pack(P, 4, 48, P, P, N) == -2
    assert lib.ep_nvfp4_unpack(P, 4, 128, N, 5, P, N) == -2         # rows_out != rows_in without a map
    assert lib.ep_route_plan(P, 0, 10, 2, 4, 24, 100, P, P, P, P, P, 1 << 20, P, N) == -3
    assert lib.ep_route_plan(P, 0, 10, 2, 4, 16, 59, P, P, P, P, P, 1 << 20, P, N) == -4
    assert lib.ep_route_plan(P, 3, 10, 2, 4, 16, 80, P, P, P, P, P, 1 << 20, P, N) == -5
    assert lib.ep_route_plan(P, 0, 10, 2, 4, 16, 80, P, P, P, P, P, 4, P, N) == -7
    assert lib.ep_route_plan(P, 0, 10, 2, 2000, 16, 80000, P, P, P, P, P, 1 << 30, P, N) == -2
    assert lib.ep_nvfp4_direct_receive(P, 4, 128, 2, 64, N, P, P, P, P, N, N, N, N) == -1
    assert lib.ep_nvfp4_direct_receive(P, 4, 128, 1025, 64, P, P, P, P, P, N, N, N, N) == -2
    assert lib.ep_nvfp4_direct_receive(P, 4, 128, 2, 64, P, P, P, P, P, P, N, P, N) == -1
    # packed rows are addressed with 31-bit offsets: fewer than 2^24 tokens, under 2 GiB of rows
    assert lib.ep_nvfp4_direct_receive(P, 1 << 24, 64, 2, 64, P, P, P, P, P, P, P, P, N) == -8
    assert lib.ep_nvfp4_direct_receive_kblock(P, 532083, 7168, 2, 64, P, P, P, P, P, P, P, P, N) == -8
    assert lib.ep_nvfp4_direct_receive_scaled(P, 532082, 7168, 2, 64, N, P, P, P, P, P, P, P, N) == -1
    assert lib.ep_nvfp4_columnwise_grouped(P, P, P, 7168, 2, 599187, P, P, P, P, N) == -8
    assert lib.dswiglu_nvfp4_quant(P, P, 10, 100, P, 2, P, P, P, P, P, P, P, P, P, 16, N) == -2
    assert lib.ep_mxfp4_direct_receive(P, 4, 128, 2, 16, 64, P, P, P, P, P, P, N) == -3   # alignment not a multiple of 32
    assert lib.ep_nvfp4_direct_receive_sr(P, 4, 128, 2, 64, P, P, P, P, P, P, P, P, N, N) == -1   # sr_state NULL
    assert lib.dswiglu_nvfp4_quant_sr(P, P, 10, 128, P, 2, P, P, P, P, P, P, P, P, P, 4096, N, N) == -1
    assert lib.ep_mxfp4_direct_receive(P, 4, 128, 2, 48, 64, P, P, P, P, P, P, N) == -3
    assert lib.ep_mxfp4_direct_receive(P, 4, 100, 2, 32, 64, P, P, P, P, P, P, N) == -2   # hidden not a multiple of 64
    assert lib.ep_mxfp4_direct_receive(P, 4, 128, 2, 32, 64, P, P, P, P, N, P, N) == -1   # col_codes NULL
    assert lib.ep_mxfp4_direct_receive(P, 4, 128, 2, 32, 64, N, P, P, P, P, P, N) == -1   # offsets NULL
    assert lib.ep_mxfp4_direct_receive_kblock(P, 4, 128, 2, 16, 64, P, P, P, P, P, P, N) == -3  # alignment
    assert lib.ep_mxfp4_direct_receive_kblock(P, 1 << 24, 64, 2, 32, 64, P, P, P, P, P, P, N) == -8
    assert lib.ep_mxfp4_kblock_tile(P, P, 128, 0, 256, 0, 16, N, N) == -1                     # out NULL
    assert lib.ep_mxfp4_kblock_tile(P, P, 128, 0, 288, 0, 16, P, N) == -2                     # len > 256
    assert lib.ep_mxfp4_kblock_tile(P, P, 128, 16, 256, 0, 16, P, N) == -2                    # block_row off the grid
    assert lib.ep_mxfp4_kblock_tile(P, P, 128, 0, 48, 0, 16, P, N) == -2                      # len off the grid
    assert lib.ep_mxfp4_kblock_tile(P, P, 128, 0, 256, 120, 0, P, N) == -2                    # columns past hidden
    assert lib.dswiglu_nvfp4_quant(P, P, 10, 128, P, 2, P, P, P, P, P, P, P, P, P, 4, N) == -7
    # the one-call receive checks both halves before its first launch
    R = (P, P, P, P, P, P, P, P, P, P)   # counts .. col_scale
    assert lib.ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, 2, 4, 16, 59, *R, P, 1 << 20, P, N) == -4  # r_cap
    assert lib.ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, 2, 4, 24, 100, *R, P, 1 << 20, P, N) == -3
    assert lib.ep_nvfp4_direct_receive_topk(P, 10, 100, P, 0, 2, 4, 16, 80, *R, P, 1 << 20, P, N) == -2
    assert lib.ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, 2, 4, 16, 80, P, P, P, P, N, P, P, P, P, P,
                                            P, 1 << 20, P, N) == -1                                   # row_codes
    assert lib.ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, 2, 4, 16, 80, *R, P, 4, P, N) == -7     # workspace
    assert lib.ep_receive_workspace_bytes(10, 2, 4) == lib.ep_route_workspace_bytes(10, 2, 4)
    # the allocation-free dSwiGLU refuses sizes beyond its static scratch before anything else
    assert lib.dswiglu_nvfp4_quant_noalloc(P, P, 1_100_000, 64, P, 8, P, P, P, P, P, P, P, P, N) == -9
    assert lib.dswiglu_nvfp4_quant_noalloc(P, P, -1, 64, P, 8, P, P, P, P, P, P, P, P, N) == -2
    assert lib.dswiglu_nvfp4_quant(P, P, 10, 128, P, 2, P, P, P, P, P, P, P, P, ctypes.c_void_p(0x1008), 4096, N) == -7  # misaligned


def test_binding_refuses_cpu_and_wrong_dtypes(lib):
    import moe_token_block_amd as m
    with pytest.raises((ValueError, TypeError)):
        m.ep_nvfp4_pack(torch.zeros((4, 64), dtype=torch.bfloat16))          # CPU tensor: no CPU path
    with pytest.raises((ValueError, TypeError)):
        m.ep_nvfp4_pack(torch.zeros((4, 64), dtype=torch.float32))


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "moe_token_block_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, f)
