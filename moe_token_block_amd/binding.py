"""Python binding of the C ABI in ``include/moe_token_block.h``.

Argument marshalling only: every step of the path runs in the gfx950 kernels
of ``libmoe_token_block.so``.  PyTorch provides device memory and the stream;
each call runs on the input tensor's device and that device's current stream
(P1, commit messages: launch stream, allocations and the stochastic-rounding
state follow the input tensor's device).  There is no CPU fallback: if the
library is missing, every entry point raises.
"""

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_token_block.so")

EP_ROUND_NEAREST, EP_ROUND_SR_ELEMENT, EP_ROUND_SR_STREAM = 0, 1, 2
EP_ROUND_SR_ELEMENT_CARRY, EP_ROUND_SR_STREAM_CARRY = 3, 4
EP_IDX_INT32, EP_IDX_INT64 = 0, 1
EP_DEVERR_EXPERT_ID = 1
EP_ERR_SCRATCH = -9
EP_NOALLOC_SCRATCH_BYTES = 4 << 20

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGS = {
    "ep_abi_version": (_I32, []),
    "ep_status_string": (ctypes.c_char_p, [_I32]),
    "ep_nvfp4_packed_row_bytes": (_I64, [_I64]),
    "ep_route_capacity": (_I64, [_I64, _I64, _I64, _I64]),
    "ep_route_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "ep_rht_sign_mask": (ctypes.c_uint32, []),
    "dswiglu_workspace_bytes": (_SZ, [_I64, _I64]),
    "ep_nvfp4_pack": (_I32, [_P, _I64, _I64, _P, _I32, _P, _P]),
    "ep_mxfp8_pack": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "ep_nvfp4_unpack": (_I32, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "ep_route_plan": (_I32, [_P, _I32, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "ep_nvfp4_direct_receive": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ep_receive_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "ep_nvfp4_direct_receive_topk": (_I32, [_P, _I64, _I64, _P, _I32, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                                            _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "ep_nvfp4_expert_scale": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P]),
    "ep_nvfp4_direct_receive_scaled": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ep_mxfp8_direct_receive": (_I32, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "ep_nvfp4_direct_receive_kblock": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ep_mxfp4_direct_receive": (_I32, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "ep_mxfp4_direct_receive_kblock": (_I32, [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "ep_mxfp4_kblock_tile": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "ep_nvfp4_direct_receive_sr": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ep_nvfp4_direct_receive_sr_stream": (_I32, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ep_nvfp4_pack_scatter": (_I32, [_P, _I64, _I64, _I64, _P, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "ep_nvfp4_columnwise_grouped": (_I32, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "dswiglu_nvfp4_quant": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dswiglu_nvfp4_quant_sr": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "dswiglu_nvfp4_quant_sr_stream": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P,
                                             _P]),
    "dswiglu_nvfp4_quant_noalloc": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
}

EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m moe_token_block_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class EpError(RuntimeError):
    pass


def _check(status, what):
    if status != 0:
        msg = lib().ep_status_string(status).decode()
        raise EpError(f"{what}: status {status} ({msg})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("tensors must live on a GPU (no CPU path)")
    return t.device


def _need(t, dtype, name, dev=None, shape=None, numel=None):
    """Checks a tensor handed to the library: dtype, contiguity, device, and its
    size -- an exact ``shape``, or at least ``numel`` elements.  The C ABI gets
    raw pointers, so this is the only place a buffer too small for the sizes
    passed with it can be caught before a kernel writes past its end."""
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")


def _row_bytes(hidden, what):
    rb = lib().ep_nvfp4_packed_row_bytes(hidden)
    _check(rb if rb < 0 else 0, what)
    return rb


def _packed(packed, hidden, dev, what):
    """A packed-row tensor [rows, 9*hidden/16 + 4] (uint8)."""
    _need(packed, torch.uint8, "packed", dev)
    rb = _row_bytes(hidden, what)
    if packed.dim() != 2 or packed.shape[1] != rb:
        raise ValueError(f"{what}: packed has shape {tuple(packed.shape)}, rows of {rb} bytes expected "
                         f"for hidden {hidden}")
    return packed.shape[0]


def _plan(plan, dev, tokens=None):
    """Sizes of a routing plan as its tensors hold them."""
    e, r_cap = int(plan["num_experts"]), int(plan["r_cap"])
    _need(plan["offsets"], torch.int32, "plan offsets", dev, shape=(e + 1,))
    _need(plan["counts"], torch.int32, "plan counts", dev, shape=(e,))
    _need(plan["src_row"], torch.int32, "plan src_row", dev, shape=(r_cap,))
    _need(plan["dst_row"], torch.int32, "plan dst_row", dev)
    if tokens is not None and plan["dst_row"].shape[0] != tokens:
        raise ValueError(f"the plan routes {plan['dst_row'].shape[0]} tokens, the input has {tokens}")
    return e, r_cap


def _receive_out(out, r_cap, hidden, e, dev, columnwise=True, scale_div=16, col_scale=True):
    """Checks the grouped-operand buffers of a receive: rowwise codes / scales /
    t for r_cap rows, columnwise codes and scales for r_cap * hidden elements,
    the per-expert decode scales."""
    _need(out["row_codes"], torch.uint8, "row_codes", dev, numel=r_cap * (hidden // 2))
    _need(out["row_scales"], torch.uint8, "row_scales", dev, numel=r_cap * (hidden // scale_div))
    if "row_t" in out:
        _need(out["row_t"], torch.float32, "row_t", dev, numel=r_cap)
    if columnwise:
        _need(out["col_codes"], torch.uint8, "col_codes", dev, numel=r_cap * hidden // 2)
        _need(out["col_scales"], torch.uint8, "col_scales", dev, numel=r_cap * hidden // scale_div)
        if col_scale:
            _need(out["col_scale"], torch.float32, "col_scale", dev, numel=e)


# ------------------------------------------------------------------ helpers
def ep_abi_version():
    return lib().ep_abi_version()


def ep_status_string(status):
    return lib().ep_status_string(status).decode()


def ep_nvfp4_packed_row_bytes(hidden):
    return lib().ep_nvfp4_packed_row_bytes(hidden)


def ep_route_capacity(tokens, top_k, num_experts, alignment):
    r = lib().ep_route_capacity(tokens, top_k, num_experts, alignment)
    _check(r if r < 0 else 0, "ep_route_capacity")
    return r


def ep_rht_sign_mask():
    return lib().ep_rht_sign_mask()


# ------------------------------------------------------------------ pack / unpack
def ep_nvfp4_pack(x, round_mode=EP_ROUND_NEAREST, sr_state=None, out=None):
    """BF16 rows [T, H] -> packed NVFP4 rows uint8 [T, 9H/16 + 4].

    ``sr_state``: int64 device tensor [2] = {seed, counter_base} for the
    stochastic modes (a pre-quantized or non-BF16 input is refused)."""
    dev = _dev(x)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    t, h = x.shape
    rb = _row_bytes(h, "ep_nvfp4_pack")
    if out is None:
        out = torch.empty((t, rb), dtype=torch.uint8, device=dev)
    _need(out, torch.uint8, "out", dev, shape=(t, rb))
    if round_mode != EP_ROUND_NEAREST:
        if sr_state is None:
            raise ValueError("stochastic rounding needs sr_state")
        _need(sr_state, torch.int64, "sr_state", dev, numel=2)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_pack(_ptr(x), t, h, _ptr(out), round_mode, _ptr(sr_state), _stream(dev)),
               "ep_nvfp4_pack")
    return out


def ep_nvfp4_unpack(packed, hidden, src_row=None, out=None):
    """Packed rows -> BF16 [rows_out, H]; with ``src_row`` (int32 [rows_out]) output
    row g decodes packed row src_row[g] (-1: zeros)."""
    dev = _dev(packed)
    rows_in = _packed(packed, hidden, dev, "ep_nvfp4_unpack")
    rows_out = rows_in if src_row is None else src_row.numel()
    if src_row is not None:
        _need(src_row, torch.int32, "src_row", dev)
    if out is None:
        out = torch.empty((rows_out, hidden), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out", dev, numel=rows_out * hidden)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_unpack(_ptr(packed), rows_in, hidden, _ptr(src_row), rows_out, _ptr(out), _stream(dev)),
               "ep_nvfp4_unpack")
    return out


def ep_mxfp8_pack(x, out=None):
    """BF16 rows [T, H] -> (data uint8 [T, H], scales uint8 [T, H/32]) carved from one
    data-then-scales buffer (returned as the third element)."""
    dev = _dev(x)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    t, h = x.shape
    if h % 32:
        raise ValueError("hidden must be a multiple of 32")
    if out is None:
        out = torch.empty(t * h + t * (h // 32), dtype=torch.uint8, device=dev)
    _need(out, torch.uint8, "out", dev, numel=t * h + t * (h // 32))
    data = out[: t * h].view(t, h)
    scales = out[t * h : t * h + t * (h // 32)].view(t, h // 32)
    with torch.cuda.device(dev):
        _check(lib().ep_mxfp8_pack(_ptr(x), t, h, _ptr(data), _ptr(scales), _stream(dev)), "ep_mxfp8_pack")
    return data, scales, out


# ------------------------------------------------------------------ routing / receive
def _topk(topk_idx):
    if topk_idx.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_idx must be int32 or int64")
    if not topk_idx.is_contiguous() or topk_idx.dim() != 2:
        raise ValueError("topk_idx must be a contiguous [tokens, top_k] tensor")
    return EP_IDX_INT64 if topk_idx.dtype == torch.int64 else EP_IDX_INT32


def _plan_buffers(t, k, num_experts, r_cap, dev, out, d_error):
    i32 = dict(dtype=torch.int32, device=dev)
    if out is not None:
        counts, offsets, dst_row, src_row = out["counts"], out["offsets"], out["dst_row"], out["src_row"]
        if d_error is None:
            d_error = out["d_error"]
    else:
        counts = torch.empty(num_experts, **i32)
        offsets = torch.empty(num_experts + 1, **i32)
        dst_row = torch.empty((t, k), **i32)
        src_row = torch.empty(r_cap, **i32)
    if d_error is None:
        d_error = torch.zeros(1, **i32)
    _need(counts, torch.int32, "counts", dev, shape=(num_experts,))
    _need(offsets, torch.int32, "offsets", dev, shape=(num_experts + 1,))
    _need(dst_row, torch.int32, "dst_row", dev, numel=t * k)
    _need(src_row, torch.int32, "src_row", dev, shape=(r_cap,))
    _need(d_error, torch.int32, "d_error", dev, numel=1)
    return dict(counts=counts, offsets=offsets, dst_row=dst_row, src_row=src_row, d_error=d_error, r_cap=r_cap,
                num_experts=num_experts)


def ep_route_plan(topk_idx, num_experts, alignment=16, r_cap=None, d_error=None, workspace=None, out=None):
    """Routing plan of topk_idx [T, k] (int32 or int64): dict of counts, offsets,
    dst_row, src_row (device int32), d_error (device int32 [1]) and r_cap.
    ``out``: a plan returned earlier for the same sizes, refilled in place."""
    dev = _dev(topk_idx)
    idt = _topk(topk_idx)
    t, k = topk_idx.shape
    cap = ep_route_capacity(t, k, num_experts, alignment)
    r_cap = cap if r_cap is None else r_cap
    plan = _plan_buffers(t, k, num_experts, r_cap, dev, out, d_error)
    wsb = lib().ep_route_workspace_bytes(t, k, num_experts)
    if workspace is None:
        workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", dev, numel=wsb)
    with torch.cuda.device(dev):
        _check(lib().ep_route_plan(_ptr(topk_idx), idt, t, k, num_experts, alignment, r_cap, _ptr(plan["counts"]),
                                   _ptr(plan["offsets"]), _ptr(plan["dst_row"]), _ptr(plan["src_row"]),
                                   _ptr(workspace), workspace.numel(), _ptr(plan["d_error"]), _stream(dev)),
               "ep_route_plan")
    plan["alignment"] = alignment
    return plan


def _receive_buffers(r_cap, hidden, e, dev, columnwise=True):
    u8 = dict(dtype=torch.uint8, device=dev)
    out = dict(row_codes=torch.empty((r_cap, hidden // 2), **u8),
               row_scales=torch.empty((r_cap, hidden // 16), **u8),
               row_t=torch.empty(r_cap, dtype=torch.float32, device=dev))
    if columnwise:
        out.update(col_codes=torch.empty(r_cap * hidden // 2, **u8),
                   col_scales=torch.empty(r_cap * hidden // 16, **u8),
                   col_scale=torch.empty(e, dtype=torch.float32, device=dev))
    return out


def ep_nvfp4_direct_receive(packed, hidden, plan, columnwise=True, out=None):
    """Grouped rowwise (+ RHT columnwise) NVFP4 operands from packed rows and a
    routing plan (from ``ep_route_plan``)."""
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, "ep_nvfp4_direct_receive")
    e, r_cap = _plan(plan, dev)
    if out is None:
        out = _receive_buffers(r_cap, hidden, e, dev, columnwise)
    columnwise = out.get("col_codes") is not None
    _receive_out(out, r_cap, hidden, e, dev, columnwise)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_direct_receive(
            _ptr(packed), t, hidden, e, r_cap, _ptr(plan["offsets"]), _ptr(plan["src_row"]),
            _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["row_t"]),
            _ptr(out.get("col_codes")), _ptr(out.get("col_scales")), _ptr(out.get("col_scale")),
            _stream(dev)), "ep_nvfp4_direct_receive")
    return out


def ep_receive_workspace_bytes(tokens, top_k, num_experts):
    return lib().ep_receive_workspace_bytes(tokens, top_k, num_experts)


def ep_nvfp4_direct_receive_topk(packed, hidden, topk_idx, num_experts, alignment=16, columnwise=True, r_cap=None,
                                 out=None, plan=None, workspace=None, d_error=None):
    """The receive in one call from top-k indices [T, k] (int32 or int64): returns
    (plan, operands), the plan refilled in ``plan`` if given."""
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, "ep_nvfp4_direct_receive_topk")
    idt = _topk(topk_idx)
    if topk_idx.device != dev or topk_idx.shape[0] != t:
        raise ValueError("topk_idx must be [tokens, top_k] on the packed rows' device")
    k = topk_idx.shape[1]
    cap = ep_route_capacity(t, k, num_experts, alignment)
    r_cap = cap if r_cap is None else r_cap
    plan = _plan_buffers(t, k, num_experts, r_cap, dev, plan, d_error)
    plan["alignment"] = alignment
    if out is None:
        out = _receive_buffers(r_cap, hidden, num_experts, dev, columnwise)
    columnwise = out.get("col_codes") is not None
    _receive_out(out, r_cap, hidden, num_experts, dev, columnwise)
    wsb = lib().ep_receive_workspace_bytes(t, k, num_experts)
    if workspace is None:
        workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", dev, numel=wsb)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_direct_receive_topk(
            _ptr(packed), t, hidden, _ptr(topk_idx), idt, k, num_experts, alignment, r_cap, _ptr(plan["counts"]),
            _ptr(plan["offsets"]), _ptr(plan["dst_row"]), _ptr(plan["src_row"]), _ptr(out["row_codes"]),
            _ptr(out["row_scales"]), _ptr(out["row_t"]), _ptr(out.get("col_codes")), _ptr(out.get("col_scales")),
            _ptr(out.get("col_scale")), _ptr(workspace), workspace.numel(), _ptr(plan["d_error"]), _stream(dev)),
            "ep_nvfp4_direct_receive_topk")
    return plan, out


def ep_nvfp4_direct_receive_kblock(packed, hidden, plan, out):
    """The one-pass receive with the columnwise operand in 256-row K-blocks
    (out["col_scale"] already holding D_e, as for ep_nvfp4_direct_receive_scaled)."""
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, "ep_nvfp4_direct_receive_kblock")
    e, r_cap = _plan(plan, dev)
    _receive_out(out, r_cap, hidden, e, dev)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_direct_receive_kblock(
            _ptr(packed), t, hidden, e, r_cap, _ptr(plan["offsets"]),
            _ptr(plan["src_row"]), _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["row_t"]),
            _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(out["col_scale"]), _stream(dev)),
            "ep_nvfp4_direct_receive_kblock")
    return out


def ep_mxfp4_direct_receive(packed, hidden, plan, out=None, kblock=False):
    """MXFP4 rowwise and RHT columnwise grouped operands (E2M1 codes, one E8M0 scale
    per 32 elements) from NVFP4 packed rows and a routing plan whose alignment is a
    multiple of 32; ``kblock`` lays the columnwise operand out in 256-row K-blocks
    (``ep_mxfp4_direct_receive_kblock``)."""
    name = "ep_mxfp4_direct_receive_kblock" if kblock else "ep_mxfp4_direct_receive"
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, name)
    e, r_cap = _plan(plan, dev)
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        out = dict(row_codes=torch.empty((r_cap, hidden // 2), **u8), row_scales=torch.empty((r_cap, hidden // 32), **u8),
                   col_codes=torch.empty(r_cap * hidden // 2, **u8), col_scales=torch.empty(r_cap * hidden // 32, **u8))
    _receive_out(out, r_cap, hidden, e, dev, scale_div=32, col_scale=False)
    with torch.cuda.device(dev):
        _check(getattr(lib(), name)(
            _ptr(packed), t, hidden, e, plan.get("alignment", 16), r_cap,
            _ptr(plan["offsets"]), _ptr(plan["src_row"]), _ptr(out["row_codes"]), _ptr(out["row_scales"]),
            _ptr(out["col_codes"]), _ptr(out["col_scales"]), _stream(dev)), name)
    return out


def ep_mxfp4_kblock_tile(col_codes, col_scales, hidden, block_row, length, ha, hb, out=None):
    """One 16 x 16 tile, computed by gfx950's block-scaled matrix instruction on the
    K-blocked MXFP4 operand as stored: out[i, j] = sum_k A[ha+i, k] A[hb+j, k] over the
    K-block of grouped rows [block_row, block_row + length)."""
    dev = _dev(col_codes)
    _need(col_codes, torch.uint8, "col_codes", dev)
    _need(col_scales, torch.uint8, "col_scales", dev)
    if col_codes.numel() < hidden * (block_row + length) // 2 or col_scales.numel() < hidden * (block_row + length) // 32:
        raise ValueError("ep_mxfp4_kblock_tile: the operand buffers do not hold the K-block")
    if out is None:
        out = torch.empty((16, 16), dtype=torch.float32, device=dev)
    _need(out, torch.float32, "out", dev, numel=256)
    with torch.cuda.device(dev):
        _check(lib().ep_mxfp4_kblock_tile(_ptr(col_codes), _ptr(col_scales), hidden, block_row, length, ha, hb,
                                          _ptr(out), _stream(dev)), "ep_mxfp4_kblock_tile")
    return out


def ep_nvfp4_pack_scatter(x, plan, out=None):
    """BF16 token rows [T, H] packed straight into the grouped rowwise operand of a
    routing plan (each token once, written to its top-k grouped rows; padding rows
    zeroed): the same bytes as ep_nvfp4_pack followed by the rowwise receive."""
    dev = _dev(x)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    t, h = x.shape
    _row_bytes(h, "ep_nvfp4_pack_scatter")
    e, r_cap = _plan(plan, dev, tokens=t)
    k = plan["dst_row"].shape[1] if plan["dst_row"].dim() == 2 else 1
    if plan["dst_row"].numel() != t * k:
        raise ValueError("plan dst_row must hold tokens * top_k entries")
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        out = dict(row_codes=torch.empty((r_cap, h // 2), **u8), row_scales=torch.empty((r_cap, h // 16), **u8),
                   row_t=torch.empty(r_cap, dtype=torch.float32, device=dev))
    _receive_out(out, r_cap, h, e, dev, columnwise=False)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_pack_scatter(_ptr(x), t, h, k, _ptr(plan["dst_row"]), e, r_cap, _ptr(plan["counts"]),
                                           _ptr(plan["offsets"]), _ptr(out["row_codes"]), _ptr(out["row_scales"]),
                                           _ptr(out["row_t"]), _stream(dev)), "ep_nvfp4_pack_scatter")
    return out


def ep_nvfp4_columnwise_grouped(rowwise, hidden, plan, out=None):
    """D_e and the RHT columnwise operand from a grouped rowwise operand
    (``rowwise``: dict with row_codes, row_scales, row_t): the same bytes as the
    direct receive's columnwise outputs."""
    dev = _dev(rowwise["row_codes"])
    _row_bytes(hidden, "ep_nvfp4_columnwise_grouped")
    e, r_cap = _plan(plan, dev)
    _receive_out(rowwise, r_cap, hidden, e, dev, columnwise=False)
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        out = dict(col_codes=torch.empty(r_cap * hidden // 2, **u8), col_scales=torch.empty(r_cap * hidden // 16, **u8),
                   col_scale=torch.empty(e, dtype=torch.float32, device=dev))
    _need(out["col_codes"], torch.uint8, "col_codes", dev, numel=r_cap * hidden // 2)
    _need(out["col_scales"], torch.uint8, "col_scales", dev, numel=r_cap * hidden // 16)
    _need(out["col_scale"], torch.float32, "col_scale", dev, numel=e)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_columnwise_grouped(
            _ptr(rowwise["row_codes"]), _ptr(rowwise["row_scales"]), _ptr(rowwise["row_t"]), hidden, e, r_cap,
            _ptr(plan["offsets"]), _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(out["col_scale"]),
            _stream(dev)), "ep_nvfp4_columnwise_grouped")
    return out


def ep_nvfp4_expert_scale(packed, hidden, plan, col_scale=None):
    """D_e = 4 * max t over each expert's rows -> float32 [E] (the first half of the receive)."""
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, "ep_nvfp4_expert_scale")
    e, r_cap = _plan(plan, dev)
    if col_scale is None:
        col_scale = torch.empty(e, dtype=torch.float32, device=dev)
    _need(col_scale, torch.float32, "col_scale", dev, numel=e)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_expert_scale(_ptr(packed), t, hidden, e, r_cap,
                                           _ptr(plan["offsets"]), _ptr(plan["src_row"]), _ptr(col_scale),
                                           _stream(dev)), "ep_nvfp4_expert_scale")
    return col_scale


def ep_nvfp4_direct_receive_scaled(packed, hidden, plan, out):
    """The one-pass receive kernel alone, with out["col_scale"] already holding D_e."""
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, "ep_nvfp4_direct_receive_scaled")
    e, r_cap = _plan(plan, dev)
    _receive_out(out, r_cap, hidden, e, dev)
    with torch.cuda.device(dev):
        _check(lib().ep_nvfp4_direct_receive_scaled(
            _ptr(packed), t, hidden, e, r_cap, _ptr(plan["offsets"]),
            _ptr(plan["src_row"]), _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["row_t"]),
            _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(out["col_scale"]), _stream(dev)),
            "ep_nvfp4_direct_receive_scaled")
    return out


def ep_nvfp4_direct_receive_sr(packed, hidden, plan, out, sr_state, stream_words=False):
    """The one-pass receive with stochastic columnwise codes; out["col_scale"] must
    hold D_e (ep_nvfp4_expert_scale); sr_state: device int64 [seed, counter_base];
    ``stream_words`` takes each position's word from the four-word Philox stream
    (``ep_nvfp4_direct_receive_sr_stream``) instead of a block per position."""
    name = "ep_nvfp4_direct_receive_sr_stream" if stream_words else "ep_nvfp4_direct_receive_sr"
    dev = _dev(packed)
    t = _packed(packed, hidden, dev, name)
    e, r_cap = _plan(plan, dev)
    _receive_out(out, r_cap, hidden, e, dev)
    _need(sr_state, torch.int64, "sr_state", dev, numel=2)
    with torch.cuda.device(dev):
        _check(getattr(lib(), name)(
            _ptr(packed), t, hidden, e, r_cap, _ptr(plan["offsets"]),
            _ptr(plan["src_row"]), _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["row_t"]),
            _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(out["col_scale"]), _ptr(sr_state), _stream(dev)),
            name)
    return out


def ep_mxfp8_direct_receive(data, scales, plan, out=None):
    """Grouped MXFP8 rows: grouped row g holds the data and scale bytes of token
    src_row[g] (zero bytes for padding)."""
    dev = _dev(data)
    _need(data, torch.uint8, "data", dev)
    if data.dim() != 2 or data.shape[1] % 32:
        raise ValueError("data must be [tokens, hidden] with hidden a multiple of 32")
    t, h = data.shape
    _need(scales, torch.uint8, "scales", dev, shape=(t, h // 32))
    _, r_cap = _plan(plan, dev)
    if out is None:
        out = (torch.empty((r_cap, h), dtype=torch.uint8, device=dev),
               torch.empty((r_cap, h // 32), dtype=torch.uint8, device=dev))
    _need(out[0], torch.uint8, "grouped data", dev, numel=r_cap * h)
    _need(out[1], torch.uint8, "grouped scales", dev, numel=r_cap * (h // 32))
    with torch.cuda.device(dev):
        _check(lib().ep_mxfp8_direct_receive(_ptr(data), _ptr(scales), t, h, r_cap, _ptr(plan["src_row"]),
                                             _ptr(out[0]), _ptr(out[1]), _stream(dev)), "ep_mxfp8_direct_receive")
    return out


# ------------------------------------------------------------------ dSwiGLU
def _dswiglu_out(out, t, f, e, dev):
    cap = t + 15 * e
    if out["dx"] is not None:
        _need(out["dx"], torch.bfloat16, "dx", dev, numel=t * 2 * f)
    for name, n in (("amax", e), ("row_scale", e), ("col_scale", e)):
        _need(out[name], torch.float32, name, dev, numel=n)
    _need(out["row_codes"], torch.uint8, "row_codes", dev, numel=t * f)
    _need(out["row_scales"], torch.uint8, "row_scales", dev, numel=t * (2 * f // 16))
    _need(out["col_codes"], torch.uint8, "col_codes", dev, numel=2 * f * cap // 2)
    _need(out["col_scales"], torch.uint8, "col_scales", dev, numel=2 * f * cap // 16)


def _dswiglu_args(preact, dy, counts, out, materialize_dx):
    dev = _dev(preact)
    _need(dy, torch.bfloat16, "dy", dev)
    if dy.dim() != 2:
        raise ValueError("dy must be [tokens, ffn]")
    t, f = dy.shape
    _need(preact, torch.bfloat16, "preact", dev, shape=(t, 2 * f))
    _need(counts, torch.int32, "counts", dev)
    if counts.dim() != 1:
        raise ValueError("counts must be [num_experts]")
    e = counts.shape[0]
    cap = t + 15 * e
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        out = dict(dx=torch.empty((t, 2 * f), dtype=torch.bfloat16, device=dev) if materialize_dx else None,
                   amax=torch.empty(e, **f32),
                   row_codes=torch.empty((t, f), **u8), row_scales=torch.empty((t, 2 * f // 16), **u8),
                   row_scale=torch.empty(e, **f32), col_codes=torch.empty(2 * f * cap // 2, **u8),
                   col_scales=torch.empty(2 * f * cap // 16, **u8), col_scale=torch.empty(e, **f32))
    _dswiglu_out(out, t, f, e, dev)
    args = (_ptr(preact), _ptr(dy), t, f, _ptr(counts), e, _ptr(out["dx"]), _ptr(out["amax"]),
            _ptr(out["row_codes"]), _ptr(out["row_scales"]), _ptr(out["row_scale"]),
            _ptr(out["col_codes"]), _ptr(out["col_scales"]), _ptr(out["col_scale"]))
    return dev, t, e, out, args


def dswiglu_nvfp4_quant_noalloc(preact, dy, counts, out, materialize_dx=True):
    """dswiglu_nvfp4_quant without a workspace: the library's static per-GPU
    scratch serves instead (the caller passes every output; calls that overlap
    on one GPU race)."""
    dev, t, e, out, args = _dswiglu_args(preact, dy, counts, out, materialize_dx)
    with torch.cuda.device(dev):
        _check(lib().dswiglu_nvfp4_quant_noalloc(*args, _stream(dev)), "dswiglu_nvfp4_quant_noalloc")
    return out


def dswiglu_nvfp4_quant(preact, dy, counts, out=None, workspace=None, materialize_dx=True, sr_state=None,
                        stream_words=False):
    """Grouped dSwiGLU epilogue + FC1-gradient NVFP4 operands; rows expert-major,
    ``counts`` a device int32 [E] tensor.  Returns a dict of output tensors.
    ``materialize_dx=False``: no BF16 dX is written (out["dx"] is None); the
    quantizer recomputes dX from preact and dy.  ``sr_state`` (device int64
    [seed, counter_base]): stochastic FC1-gradient codes, each position's Philox
    word its own block's or, with ``stream_words``, from the four-word stream."""
    dev, t, e, out, args = _dswiglu_args(preact, dy, counts, out, materialize_dx)
    wsb = lib().dswiglu_workspace_bytes(t, e)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", dev, numel=wsb)
    with torch.cuda.device(dev):
        args = args + (_ptr(workspace), workspace.numel())
        if sr_state is not None:
            _need(sr_state, torch.int64, "sr_state", dev, numel=2)
            name = "dswiglu_nvfp4_quant_sr_stream" if stream_words else "dswiglu_nvfp4_quant_sr"
            _check(getattr(lib(), name)(*args, _ptr(sr_state), _stream(dev)), name)
            return out
        _check(lib().dswiglu_nvfp4_quant(*args, _stream(dev)), "dswiglu_nvfp4_quant")
    return out
