"""Benchmark of the block-scaled token codec hot path on one MI355X.

Headline step: one pass of the path over the DeepSeek-V3-shaped one-GPU share
(16384 tokens x hidden 7168 BF16 ~ N(0, 0.5^2) * 10^U(-2,2) per token, top-8
of 32 experts from N(0,1) logits, 16-row aligned slots):

  route plan -> NVFP4 pack -> per-expert decode scale D_e -> direct receive
  (rowwise operand + 16-point-RHT columnwise operand, K-blocked: each
  expert's 256-row K-blocks one contiguous region) -> unpack of the received
  rows to BF16.

value = algorithmic bytes (distinct inputs read once + outputs, padding rows
excluded) of the step / step time, in GB/s.  Inputs are resident in HBM
before the timed region; the timed region is K eager steps on one stream,
and HIP events on that stream bracket every call of every timed step.  It
follows the configuration's per-call passes at once, and before its W warm-up
steps untimed steps run for --settle-s seconds (0.1 by default): the GPU's
clock needs tens of milliseconds of a sustained load to settle, and the
receive runs up to ~40% slower during that transient (measured).

``kernels`` lists every call of the path at each of the five configurations
(their own seeded inputs): its HIP-event time per launch (eager passes, each
after a read of a 1 GiB buffer that evicts the 256 MB MALL), algorithmic GB/s
and the fraction of the 8 TB/s HBM peak, and -- from the committed rocprofv3
counter summary, when the call's kernels are unchanged since -- its measured
traffic.  The stochastic-rounding packs are reported against VALU issue.

``cpu_baseline``: the oracle (plain numpy, test infrastructure) timed on the
host on config-3 tokens, one process and one process per core.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
       [--configs 1,2,3,4,5] [--workload cfgN] [--only CALL --workload cfgN]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantize/pack/receive GB/s (in+out) on 1 MI355X; % of HBM peak"
HBM_PEAK_GBS = 8000.0
# VALU issue: 256 CUs, each issuing one wave64 vector instruction per clock
# (four 16-lane SIMDs, four clocks per wave64 instruction each), at 2.4 GHz
VALU_PEAK_GIPS = 256 * 2.4
CPU_SAMPLE_TOKENS = 4096        # one process: about 10 s of oracle work on one host core
CPU_CHUNK_TOKENS = 1024         # one process per core: each on its own chunk

# ---------------------------------------------------------------------------- calls
# source files each call's kernels are built from (a counter summary is used
# only while these are unchanged) and the kernels it launches
_COMMON = ("common.h", "launch.h")
CALLS = {
    "route_plan": (("route.hip",), ["k_route_single (<= 16K entries)", "k_route_count + k_route_scan + k_route_scatter"]),
    "nvfp4_pack": (("pack.hip",), ["k_nvfp4_pack_wg (H >= 4096)", "k_nvfp4_pack"]),
    "nvfp4_pack_sr": (("pack.hip",), ["k_nvfp4_pack_sr_rows (H <= 4096)", "k_nvfp4_pack_sr"]),
    "nvfp4_pack_sr_stream": (("pack.hip",), ["k_nvfp4_pack_sr_rows (H <= 4096)", "k_nvfp4_pack_sr"]),
    "mxfp8_pack": (("pack.hip",), ["k_mxfp8_pack"]),
    "nvfp4_expert_scale": (("receive.hip",), ["k_expert_scale"]),
    "nvfp4_direct_receive": (("receive.hip",), ["k_nvfp4_receive"]),
    "nvfp4_direct_receive_kblock": (("receive.hip",), ["k_nvfp4_receive (K-blocked columnwise layout)"]),
    "nvfp4_direct_receive_sr": (("receive.hip",), ["k_nvfp4_receive (stochastic columnwise codes)"]),
    "nvfp4_direct_receive_sr_stream": (("receive.hip",), ["k_nvfp4_receive (stochastic codes, stream words)"]),
    "mxfp4_receive": (("receive.hip",), ["k_mxfp4_receive"]),
    "mxfp4_receive_kblock": (("receive.hip",), ["k_mxfp4_receive (K-blocked columnwise layout)"]),
    "nvfp4_pack_scatter": (("pack.hip",), ["k_nvfp4_pack_wg / k_nvfp4_pack (scatter)", "k_zero_padding"]),
    "nvfp4_columnwise_grouped": (("receive.hip",), ["k_expert_scale_grouped", "k_nvfp4_receive (grouped rows)"]),
    "mxfp8_receive": (("unpack.hip",), ["k_mxfp8_receive"]),
    "nvfp4_unpack": (("unpack.hip",), ["k_nvfp4_unpack"]),
    "nvfp4_unpack_tokens": (("unpack.hip",), ["k_nvfp4_unpack (one row per token, no gather)"]),
    "dswiglu_nvfp4_quant": (("dswiglu.hip",), ["k_dswiglu_epilogue", "k_dswiglu_reduce", "k_fc1_quant"]),
    "dswiglu_nvfp4_quant_nodx": (("dswiglu.hip",), ["k_dswiglu_epilogue (max only)", "k_dswiglu_reduce",
                                                    "k_fc1_quant (recompute)"]),
    "dswiglu_nvfp4_quant_sr": (("dswiglu.hip",), ["k_dswiglu_epilogue", "k_dswiglu_reduce",
                                                  "k_fc1_quant (stochastic codes)"]),
    "dswiglu_nvfp4_quant_sr_stream": (("dswiglu.hip",), ["k_dswiglu_epilogue", "k_dswiglu_reduce",
                                                         "k_fc1_quant (stochastic codes, stream words)"]),
}
VALU_BOUND = ("nvfp4_pack_sr", "nvfp4_pack_sr_stream")
SR_ELEMENT_CARRY, SR_STREAM_CARRY = 3, 4      # EP_ROUND_SR_ELEMENT_CARRY, EP_ROUND_SR_STREAM_CARRY


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--reps", type=int, default=20, help="eager passes per configuration for the per-call times")
    p.add_argument("--settle-s", type=float, default=STEP_SETTLE_S,
                   help="untimed steps for this many seconds before the warm-up steps (0: none)")
    p.add_argument("--configs", default="1,2,3,4,5", help="configurations listed under 'kernels'")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=CPU_SAMPLE_TOKENS)
    p.add_argument("--json-out", default=None)
    p.add_argument("--workload", default=None, choices=["cfg1", "cfg2", "cfg3", "cfg4", "cfg5"],
                   help="profiling aid: time only this configuration's calls (same JSON shape)")
    p.add_argument("--counters-pass", action="store_true",
                   help="profiling aid (with --workload): each call --steps times between marker kernels")
    p.add_argument("--only", default=None, choices=["copy"],
                   help="with --counters-pass: a 1 GiB device copy instead (the counter reference)")
    p.add_argument("--copy-bytes", type=int, default=1 << 30,
                   help="with --only copy: bytes per copy (a multiple of 16); below 1 GiB each launch "
                        "follows the MALL-evicting read, as the calls' launches do")
    return p.parse_args()


def row_bytes(h):
    return 9 * h // 16 + 4


# ---------------------------------------------------------------------------- algorithmic bytes
def dispatch_bytes(T, H, k, E, r_cap, R):
    """Distinct input bytes read once + output bytes of each dispatch-side call
    (R routed rows, padding rows excluded)."""
    rb = row_bytes(H)
    b = {}
    b["route_plan"] = T * k * 4 + E * 4 + (E + 1) * 4 + T * k * 4 + r_cap * 4
    b["nvfp4_pack"] = T * H * 2 + T * rb
    b["nvfp4_pack_sr"] = b["nvfp4_pack_sr_stream"] = T * H * 2 + T * rb + 16
    b["nvfp4_expert_scale"] = R * 4 + r_cap * 4 + (E + 1) * 4 + E * 4
    b["nvfp4_direct_receive"] = (T * rb + r_cap * 4 + (E + 1) * 4 + E * 4
                                 + R * (H // 2 + H // 16 + 4) + R * (H // 2 + H // 16))
    b["nvfp4_direct_receive_kblock"] = b["nvfp4_direct_receive_sr"] = b["nvfp4_direct_receive"]
    b["mxfp4_receive"] = T * rb + r_cap * 4 + (E + 1) * 4 + 2 * R * (H // 2 + H // 32)
    b["mxfp4_receive_kblock"] = b["mxfp4_receive"]     # the same bytes, placed per K-block
    b["nvfp4_pack_scatter"] = T * H * 2 + T * k * 4 + R * rb
    b["nvfp4_columnwise_grouped"] = R * rb + (E + 1) * 4 + R * (H // 2 + H // 16) + E * 4
    b["mxfp8_pack"] = T * H * 2 + T * H + T * (H // 32)
    b["mxfp8_receive"] = T * (H + H // 32) + r_cap * 4 + R * (H + H // 32)
    b["nvfp4_unpack"] = T * rb + R * 4 + R * H * 2
    b["nvfp4_unpack_tokens"] = T * rb + T * H * 2
    return b


def dswiglu_kernel_bytes(T, F, E, dx=True):
    """The same bytes split over the call's two main kernels: the epilogue reads
    preact and dy and writes dX (when materialized) and the per-row maxima; the
    quantizer reads dX (or preact and dy again) and writes both operands."""
    ops = 2 * T * (F + 2 * F // 16) + 3 * E * 4
    epi = T * 2 * F * 2 + T * F * 2 + (T * 2 * F * 2 if dx else 0)
    quant = (T * 2 * F * 2 if dx else T * 2 * F * 2 + T * F * 2) + ops
    return {"k_dswiglu_epilogue": epi, "k_fc1_quant": quant}


def dswiglu_bytes(T, F, E, dx=True, sr=False):
    """Inputs (preact [T,2F], dy [T,F], counts) read once + outputs (dX if written,
    the per-expert amax and scales, rowwise and columnwise codes and scales)."""
    b = T * 2 * F * 2 + T * F * 2 + E * 4 + 3 * E * 4 + 2 * T * (F + 2 * F // 16)
    if dx:
        b += T * 2 * F * 2
    if sr:
        b += 16
    return b


# ---------------------------------------------------------------------------- paths
class Call:
    def __init__(self, name, fn, nbytes, in_step=True, elements=None, kernel_bytes=None):
        self.name, self.fn, self.bytes, self.in_step, self.elements = name, fn, nbytes, in_step, elements
        self.kernel_bytes = kernel_bytes     # {kernel name part: its algorithmic bytes} for multi-kernel calls


class Path:
    """One configuration's calls over its own seeded inputs, outputs pre-allocated.
    ``step`` holds the calls of the configuration's path in order; the other
    calls are variants of a step call (other layouts, formats, rounding modes)
    timed on the same inputs."""

    def __init__(self, n, dev, w=None):
        import torch
        import moe_token_block_amd as m
        import workloads
        self.n = n
        self.dev = dev
        w = w if w is not None else workloads.CONFIGS[n]()
        self.w = w
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        self.calls = []
        self.outputs = {}        # every buffer a call writes (graph-replay test)
        if n == 5:
            T, F, E = w.preact_bits.shape[0], w.dy_bits.shape[1], len(w.counts)
            pre, dy = bf(w.preact_bits), bf(w.dy_bits)
            counts = torch.from_numpy(w.counts).to(dev)
            cap = T + 15 * E
            mk = lambda dx: dict(dx=torch.empty((T, 2 * F), dtype=torch.bfloat16, device=dev) if dx else None,
                                 amax=torch.empty(E, **f32), row_codes=torch.empty((T, F), **u8),
                                 row_scales=torch.empty((T, 2 * F // 16), **u8), row_scale=torch.empty(E, **f32),
                                 col_codes=torch.empty(2 * F * cap // 2, **u8),
                                 col_scales=torch.empty(2 * F * cap // 16, **u8), col_scale=torch.empty(E, **f32))
            out, out_nodx = mk(True), mk(False)
            self.outputs.update({f"dsw.{k}": v for k, v in out.items()})
            self.outputs.update({f"dsw_nodx.{k}": v for k, v in out_nodx.items() if v is not None})
            ws = torch.empty(m.lib().dswiglu_workspace_bytes(T, E), **u8)
            sr = torch.tensor([1234, 0], dtype=torch.int64, device=dev)
            self._add("dswiglu_nvfp4_quant", lambda: m.dswiglu_nvfp4_quant(pre, dy, counts, out=out, workspace=ws),
                      dswiglu_bytes(T, F, E), elements=T * 2 * F, kernel_bytes=dswiglu_kernel_bytes(T, F, E))
            self._add("dswiglu_nvfp4_quant_nodx",
                      lambda: m.dswiglu_nvfp4_quant(pre, dy, counts, out=out_nodx, workspace=ws),
                      dswiglu_bytes(T, F, E, dx=False), in_step=False, elements=T * 2 * F,
                      kernel_bytes=dswiglu_kernel_bytes(T, F, E, dx=False))
            self._add("dswiglu_nvfp4_quant_sr",
                      lambda: m.dswiglu_nvfp4_quant(pre, dy, counts, out=out, workspace=ws, sr_state=sr),
                      dswiglu_bytes(T, F, E, sr=True), in_step=False, elements=T * 2 * F,
                      kernel_bytes=dswiglu_kernel_bytes(T, F, E))
            self._add("dswiglu_nvfp4_quant_sr_stream",
                      lambda: m.dswiglu_nvfp4_quant(pre, dy, counts, out=out, workspace=ws, sr_state=sr,
                                                    stream_words=True),
                      dswiglu_bytes(T, F, E, sr=True), in_step=False, elements=T * 2 * F,
                      kernel_bytes=dswiglu_kernel_bytes(T, F, E))
            self.desc = dict(workload=w.name, tokens=T, ffn=F, experts=E)
            return
        T, H = w.x_bits.shape
        k, E, A = w.topk_idx.shape[1], w.num_experts, w.alignment
        R = T * k
        x = bf(w.x_bits)
        topk = torch.from_numpy(w.topk_idx).to(dev)
        r_cap = m.ep_route_capacity(T, k, E, A)
        ws = torch.empty(max(m.lib().ep_route_workspace_bytes(T, k, E), 4), **u8)
        derr = torch.zeros(1, dtype=torch.int32, device=dev)
        plan = m.ep_route_plan(topk, E, A, d_error=derr, workspace=ws)
        packed = torch.empty((T, row_bytes(H)), **u8)
        recv = dict(row_codes=torch.empty((r_cap, H // 2), **u8), row_scales=torch.empty((r_cap, H // 16), **u8),
                    row_t=torch.empty(r_cap, **f32), col_codes=torch.empty(r_cap * H // 2, **u8),
                    col_scales=torch.empty(r_cap * H // 16, **u8), col_scale=torch.empty(E, **f32))
        b = dispatch_bytes(T, H, k, E, r_cap, R)
        self.outputs.update({f"plan.{nm}": plan[nm] for nm in ("counts", "offsets", "dst_row", "src_row", "d_error")})
        self.outputs["packed"] = packed
        self.outputs.update({f"recv.{nm}": v for nm, v in recv.items()})
        G = int(plan["offsets"][-1].item())     # grouped rows, padding included: the columnwise transform's rows
        self._add("route_plan", lambda: m.ep_route_plan(topk, E, A, d_error=derr, workspace=ws, out=plan),
                  b["route_plan"])
        if n == 4:
            st = torch.tensor([w.sr_seed, w.sr_counter_base], dtype=torch.int64, device=dev)
            self._add("nvfp4_pack_sr", lambda: m.ep_nvfp4_pack(x, SR_ELEMENT_CARRY, st, out=packed),
                      b["nvfp4_pack_sr"], elements=T * H)
            self._add("nvfp4_pack_sr_stream", lambda: m.ep_nvfp4_pack(x, SR_STREAM_CARRY, st, out=packed),
                      b["nvfp4_pack_sr_stream"], in_step=False, elements=T * H)
            # the step's receive reads the element-mode rows: pack them again after the variant
            self._add("nvfp4_pack_sr", lambda: m.ep_nvfp4_pack(x, SR_ELEMENT_CARRY, st, out=packed),
                      b["nvfp4_pack_sr"], in_step=False, elements=T * H, record=False)
        else:
            self._add("nvfp4_pack", lambda: m.ep_nvfp4_pack(x, out=packed), b["nvfp4_pack"], elements=T * H)
        self._add("nvfp4_expert_scale",
                  lambda: m.ep_nvfp4_expert_scale(packed, H, plan, col_scale=recv["col_scale"]), b["nvfp4_expert_scale"])
        # the step's receive writes the K-blocked columnwise layout (each 256-row
        # K-block of an expert one contiguous [H, 128 B] region, the tiles a
        # K-tiled grouped GEMM reads); the compact per-expert layout is a variant
        self._add("nvfp4_direct_receive_kblock", lambda: m.ep_nvfp4_direct_receive_kblock(packed, H, plan, recv),
                  b["nvfp4_direct_receive_kblock"], elements=G * H)
        self._add("nvfp4_direct_receive", lambda: m.ep_nvfp4_direct_receive_scaled(packed, H, plan, recv),
                  b["nvfp4_direct_receive"], in_step=False, elements=G * H)
        if n == 2:
            mx = torch.empty(T * H + T * H // 32, **u8)
            mx_out = (torch.empty((r_cap, H), **u8), torch.empty((r_cap, H // 32), **u8))
            self.outputs.update({"mx": mx, "mx_out.data": mx_out[0], "mx_out.scales": mx_out[1]})
            self._add("mxfp8_pack", lambda: m.ep_mxfp8_pack(x, out=mx), b["mxfp8_pack"])
            self._add("mxfp8_receive", lambda: m.ep_mxfp8_direct_receive(
                mx[: T * H].view(T, H), mx[T * H:].view(T, H // 32), plan, out=mx_out), b["mxfp8_receive"])
        if n in (1, 3):
            off = plan["offsets"].cpu().numpy()
            src = plan["src_row"].cpu().numpy()
            src_valid = torch.from_numpy(np.ascontiguousarray(src[: off[-1]][src[: off[-1]] >= 0])).to(dev)
            unpacked = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
            self.outputs["unpacked"] = unpacked
            self._add("nvfp4_unpack", lambda: m.ep_nvfp4_unpack(packed, H, src_row=src_valid, out=unpacked),
                      b["nvfp4_unpack"], elements=R * H)
            # the per-token form (each packed row once, no gather): one row per token
            unpacked_t = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            self.outputs["unpacked_tokens"] = unpacked_t
            self._add("nvfp4_unpack_tokens", lambda: m.ep_nvfp4_unpack(packed, H, out=unpacked_t),
                      b["nvfp4_unpack_tokens"], in_step=False, elements=T * H)
        if n == 4:
            srr = torch.tensor([1234, 1 << 40], dtype=torch.int64, device=dev)
            self._add("nvfp4_direct_receive_sr", lambda: m.ep_nvfp4_direct_receive_sr(packed, H, plan, recv, srr),
                      b["nvfp4_direct_receive_sr"], in_step=False, elements=G * H)
            self._add("nvfp4_direct_receive_sr_stream",
                      lambda: m.ep_nvfp4_direct_receive_sr(packed, H, plan, recv, srr, stream_words=True),
                      b["nvfp4_direct_receive_sr"], in_step=False, elements=G * H)
        if n in (2, 3):
            A32 = max(A, 32)
            plan32 = m.ep_route_plan(topk, E, A32)
            r32 = plan32["r_cap"]
            mx4 = dict(row_codes=torch.empty((r32, H // 2), **u8), row_scales=torch.empty((r32, H // 32), **u8),
                       col_codes=torch.empty(r32 * H // 2, **u8), col_scales=torch.empty(r32 * H // 32, **u8))
            G32 = int(plan32["offsets"][-1].item())   # grouped rows at the 32-row alignment
            self._add("mxfp4_receive", lambda: m.ep_mxfp4_direct_receive(packed, H, plan32, out=mx4),
                      dispatch_bytes(T, H, k, E, r32, R)["mxfp4_receive"], in_step=False, elements=G32 * H)
            mx4k = {nm: torch.empty_like(v) for nm, v in mx4.items()}
            self.outputs.update({f"mx4k.{nm}": v for nm, v in mx4k.items()})
            self._add("mxfp4_receive_kblock",
                      lambda: m.ep_mxfp4_direct_receive(packed, H, plan32, out=mx4k, kblock=True),
                      dispatch_bytes(T, H, k, E, r32, R)["mxfp4_receive_kblock"], in_step=False, elements=G32 * H)
            fused = dict(row_codes=torch.empty((r_cap, H // 2), **u8), row_scales=torch.empty((r_cap, H // 16), **u8),
                         row_t=torch.empty(r_cap, **f32), col_codes=torch.empty(r_cap * H // 2, **u8),
                         col_scales=torch.empty(r_cap * H // 16, **u8), col_scale=torch.empty(E, **f32))
            self.outputs.update({f"mx4.{nm}": v for nm, v in mx4.items()})
            self.outputs.update({f"fused.{nm}": v for nm, v in fused.items()})
            self._add("nvfp4_pack_scatter", lambda: m.ep_nvfp4_pack_scatter(x, plan, out=fused),
                      b["nvfp4_pack_scatter"], in_step=False)
            self._add("nvfp4_columnwise_grouped", lambda: m.ep_nvfp4_columnwise_grouped(fused, H, plan, out=fused),
                      b["nvfp4_columnwise_grouped"], in_step=False)
        self.desc = dict(workload=w.name, tokens=T, hidden=H, experts=E, top_k=k, alignment=A)

    def _add(self, name, fn, nbytes, in_step=True, elements=None, record=True, kernel_bytes=None):
        c = Call(name, fn, nbytes, in_step, elements, kernel_bytes)
        c.record = record
        c.dev = self.dev
        self.calls.append(c)

    def step_calls(self):
        return [c for c in self.calls if c.in_step]


def evict_mall(buf):
    """Read a 1 GiB buffer (4x the 256 MB MALL) before an eager pass of per-call
    timings: the pass then starts with its inputs in HBM and no write-backs of
    earlier work ahead of its own traffic (a 1 GiB fill instead would leave 256
    MB of dirty lines for the first calls to write back), and the GPU is busy
    while the host enqueues the pass, so each event pair brackets GPU time."""
    buf.amax()


SETTLE_S = 0.06     # untimed warm-up of each configuration's per-call passes
STEP_SETTLE_S = 0.1  # untimed steps before the timed region's warm-up steps


def settle(calls, flush=None, seconds=SETTLE_S):
    """Untimed passes of ``calls`` (each after the MALL-evicting read when a flush
    buffer is given) for at least ``seconds`` of GPU time.  The GPU's clock
    settles only after tens of milliseconds of a sustained load: measured on
    config 3, the receive runs at ~400 us per call right after an idle pause or
    a change of load and ~270-290 us once settled, over 20-40 steps; a timed
    phase that starts before that would time the transient."""
    import torch
    t0 = time.monotonic()
    while True:
        if flush is not None:
            evict_mall(flush)
        for c in calls:
            c.fn()
        torch.cuda.synchronize()
        if time.monotonic() - t0 >= seconds:
            return


def time_calls(path, reps, flush):
    """Per-call HIP-event times (ms per launch) over ``reps`` eager passes of all
    the path's calls, each pass after the MALL-evicting read (after ``settle``)."""
    import torch
    calls = path.calls
    settle(calls, flush)                              # warm-up passes
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(reps)]
    for r in range(reps):
        evict_mall(flush)
        for j, c in enumerate(calls):
            ev[r][j][0].record()
            c.fn()
            ev[r][j][1].record()
    torch.cuda.synchronize()
    out = {}
    for j, c in enumerate(calls):
        if getattr(c, "record", True) and c.name not in out:
            out[c.name] = float(np.mean([ev[r][j][0].elapsed_time(ev[r][j][1]) for r in range(reps)]))
    return out


def time_step(path, steps, warmup, settle_s=STEP_SETTLE_S):
    """The timed region: ``steps`` eager passes of the step's calls on the current
    stream, HIP events on that stream around every call; returns the wall time
    per step and each call's mean event time over the timed steps.  Before the
    ``warmup`` steps, untimed steps run for ``settle_s`` seconds so that the
    timed steps see the GPU's settled clock (``settle``)."""
    import torch
    calls = path.step_calls()
    if settle_s > 0:
        settle(calls, None, settle_s)
    for _ in range(warmup):
        for c in calls:
            c.fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(steps)]
    # marker kernels (a torch random fill, used nowhere else) before and after the
    # timed region: in a kernel trace, the dispatches between them are the timed steps'
    marker = torch.empty(64, dtype=torch.float32, device=calls[0].dev)
    marker.random_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for j, c in enumerate(calls):
            ev[s][j][0].record()
            c.fn()
            ev[s][j][1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    marker.random_()
    torch.cuda.synchronize()
    per = {}
    for j, c in enumerate(calls):
        per.setdefault(c.name, []).extend(ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(steps))
    return ms_step, {k: float(np.mean(v)) for k, v in per.items()}


# ---------------------------------------------------------------------------- counters
def _code_only(text):
    """Source text without comments and whitespace (a comment edit changes no kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def kernel_source_hash(call):
    """Hash of the code (comments and whitespace dropped) of the sources the
    call's kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_token_block_amd", "csrc")
    for f in sorted(CALLS[call][0] + _COMMON):
        h.update(_code_only(open(os.path.join(csrc, f)).read()).encode())
    return h.hexdigest()[:16]


def counters_of(cfg, call):
    """The committed counter record of one call at one configuration (per launch:
    HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by the copy reference, DRAM
    request bytes, issued VALU instructions), or None when the call's kernels
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("calls", {}).get(f"cfg{cfg}/{call}")
    if rec is None or rec.get("source_hash") != kernel_source_hash(call):
        return None
    return rec


def kernel_time_of(cfg, call):
    """The committed kernel-only time of one call at one configuration (the sum of
    its dispatches' traced durations per launch), or None when the call's kernels
    changed since the trace was taken."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("calls", {}).get(f"cfg{cfg}/{call}")
    if rec is None or rec.get("source_hash") != kernel_source_hash(call):
        return None
    return rec


def entry(cfg, call, nbytes, ms, elements=None, kernel_bytes=None):
    """One call's figures: HIP-event time per launch and the algorithmic rate
    against the HBM peak; from the committed profiles (while the call's kernels
    are unchanged): the traced kernel-only time and rate, the HBM and DRAM bytes
    the counters saw, and the issued VALU instructions against the VALU issue
    peak at the kernel-only time."""
    gbs = nbytes / (ms / 1e3) / 1e9
    e = dict(ms=round(ms, 5), bytes=nbytes, gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
    kt = kernel_time_of(cfg, call)
    if kt:
        kgbs = nbytes / (kt["us_per_launch"] / 1e6) / 1e9
        e.update(kernel_us=kt["us_per_launch"], kernel_gbs=round(kgbs, 1), kernel_frac=round(kgbs / HBM_PEAK_GBS, 4))
        if kernel_bytes:
            split = {}
            for part, kb in kernel_bytes.items():
                us = sum(v for k, v in kt["kernels"].items() if part in k)
                if us > 0:
                    split[part] = dict(us=round(us, 3), bytes=kb,
                                       frac=round(kb / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 4))
            e["kernel_split"] = split
    cnt = counters_of(cfg, call)
    e["traffic"] = cnt.get("hbm_bytes") if cnt else None
    if cnt and cnt.get("dram_bytes") is not None:
        e["dram_bytes"] = cnt["dram_bytes"]
        e["dram_ratio"] = round(cnt["dram_bytes"] / nbytes, 3)
    valu = cnt.get("valu_insts") if cnt else None
    if valu:
        t = kt["us_per_launch"] / 1e6 if kt else ms / 1e3
        gips = valu / t / 1e9
        e.update(valu_insts=valu, valu_gips=round(gips, 1), valu_frac=round(gips / VALU_PEAK_GIPS, 4))
        if elements:
            e["valu_per_element"] = round(valu * 64 / elements, 2)
    if call in VALU_BOUND:
        e["bound"] = "alu"
    return e


# ---------------------------------------------------------------------------- CPU baseline
def _oracle_cfg3(x_bits, topk, E, A, H):
    """The oracle's path of one sample of config-3 tokens: route plan, pack, direct
    receive (rowwise + columnwise, re-laid in K-blocks), unpack of the received
    rows; returns
    (seconds, algorithmic bytes)."""
    from oracle import nvfp4, receive
    from oracle.routing import route_plan
    t0 = time.perf_counter()
    plan = route_plan(topk, E, A)
    packed = nvfp4.pack_rows(x_bits)
    r = receive.direct_receive(packed, H, topk, E, A)
    receive.kblock_layout(r["col_codes"], r["col_scales"], r["offsets"], H)
    off, src = plan["offsets"], plan["src_row"]
    nvfp4.unpack_rows(packed, H, src[: off[-1]][src[: off[-1]] >= 0])
    dt = time.perf_counter() - t0
    T, k = topk.shape
    b = dispatch_bytes(T, H, k, E, src.shape[0], T * k)
    return dt, sum(b[c] for c in ("route_plan", "nvfp4_pack", "nvfp4_expert_scale", "nvfp4_direct_receive_kblock",
                                  "nvfp4_unpack"))


def _oracle_worker(args):
    return _oracle_cfg3(*args)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, n_tok, n_chunk=CPU_CHUNK_TOKENS):
    """The oracle as it stands on the host, before anything touches the GPU: one
    single-threaded process on tokens [0, n_tok) of config 3, then one
    single-threaded process per core (at most 16, whatever the affinity mask
    shows), each on its own n_chunk tokens (their own routing).
    The worker processes are spawned with OMP/OpenBLAS/MKL threads set to 1, so
    each uses exactly one core."""
    import multiprocessing as mp
    E, A, H = w.num_experts, w.alignment, w.x_bits.shape[1]
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = "1"                     # inherited by the spawned workers
    ctx = mp.get_context("spawn")
    # pools are closed and joined, not terminated: the workers then exit on
    # their own, with no signal (a profiler's signal handler in a terminated
    # worker has held up the parent's join)
    pool = ctx.Pool(1)
    try:
        dt1, b1 = pool.apply(_oracle_worker, ((w.x_bits[:n_tok], w.topk_idx[:n_tok], E, A, H),))
    finally:
        pool.close()
        pool.join()
    ncore = max(1, min(len(os.sched_getaffinity(0)), 16, w.x_bits.shape[0] // n_chunk))
    jobs = [(w.x_bits[i * n_chunk:(i + 1) * n_chunk], w.topk_idx[i * n_chunk:(i + 1) * n_chunk], E, A, H)
            for i in range(ncore)]
    t0 = time.perf_counter()
    pool = ctx.Pool(ncore)
    try:
        res = pool.map(_oracle_worker, jobs)
        dtn = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    bn = sum(r[1] for r in res)
    return {"value": round(bn / dtn / 1e9, 4), "unit": "GB/s", "cores": ncore, "kind": "oracle",
            "sample": f"config 3 ({w.name}): route plan, NVFP4 pack, direct receive (rowwise + RHT columnwise, "
                      f"K-blocked), "
                      f"unpack; {ncore} processes, each on its own {n_chunk} tokens ({ncore * n_chunk} tokens, "
                      f"{dtn:.1f} s wall incl. process start)",
            "single_core": {"value": round(b1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"tokens [0, {n_tok}) of config 3, {dt1:.1f} s, one thread"},
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model()}


# ---------------------------------------------------------------------------- output
def headline(path3, ms_step, per, steps, warmup, kernels, cpu, copy=None, settle_s=STEP_SETTLE_S):
    calls = path3.step_calls()
    total = sum(c.bytes for c in calls)
    dom = max(per, key=lambda nm: per[nm])
    c = next(c for c in calls if c.name == dom)
    gbs = c.bytes / (per[dom] / 1e3) / 1e9
    cnt = counters_of(3, dom)
    roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                traffic=cnt.get("hbm_bytes") if cnt else None, kernel=dom, kernels=CALLS[dom][1],
                bytes_per_launch=c.bytes, ms_per_launch=round(per[dom], 5),
                dominant_by="largest per-launch time in the timed step")
    if cnt and cnt.get("dram_bytes") is not None:
        roof["dram_bytes"] = cnt["dram_bytes"]
    if cnt and cnt.get("valu_insts"):
        # the same launch against the VALU issue peak: the receive's decode, 16-point
        # RHT and quotients are instruction-bound before they are HBM-bound
        gips = cnt["valu_insts"] / (per[dom] / 1e3) / 1e9
        roof["valu_issue"] = dict(insts_per_launch=cnt["valu_insts"], achieved=round(gips, 1), peak=VALU_PEAK_GIPS,
                                  unit="G wave-instructions/s", frac=round(gips / VALU_PEAK_GIPS, 4))
    return {
        "metric": METRIC, "value": round(total / (ms_step / 1e3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "settle_s": settle_s, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": dict(path3.desc, workload=path3.desc["workload"] + ": route plan + NVFP4 pack + D_e + direct "
                       "receive (rowwise + RHT columnwise in K-blocks) + unpack of the received rows",
                       bytes_per_step=total, step_calls=[c.name for c in calls],
                       step_ms={nm: round(v, 5) for nm, v in per.items()}),
        "roofline": roof,
        "kernels": kernels,
        "copy_reference": copy,
        "cpu_baseline": cpu,
    }


def copy_reference(dev, reps=10):
    """A 1 GiB device-to-device copy (torch's copy kernel) timed with HIP events:
    the rate a plain streaming kernel reaches on this GPU, for context."""
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    nbytes = 2 * a.numel() * 4
    del a, b
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "ms": round(ms, 4), "gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
            "frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "kind": "torch device-to-device copy, 1 GiB"}


def config_kernels(n, path, per):
    out = {}
    for c in path.calls:
        if c.name in per and c.name not in out:
            out[c.name] = entry(n, c.name, c.bytes, per[c.name], c.elements, c.kernel_bytes)
            if not c.in_step:
                out[c.name]["variant"] = True
    return dict(workload=path.desc["workload"], calls=out)


def main_counters_pass(args, dev):
    """Counter-collection aid (run under rocprofv3 --pmc): every call of --workload
    once, then for each call a marker kernel (a torch random fill, used nowhere
    else) followed by --steps launches of the call, each after the MALL-evicting
    read (a torch reduction).  A profile's dispatches between two markers that
    are not the reduction are that call's.  --only copy: --steps
    device-to-device copies of --copy-bytes (1 GiB: the reference that scales
    the memory counters; smaller: the kernel-only time a plain copy of a call's
    size takes, each launch after the MALL-evicting read) after one marker
    instead."""
    import torch
    marker = torch.empty(64, dtype=torch.float32, device=dev)
    if args.only == "copy":
        if args.copy_bytes <= 0 or args.copy_bytes % 16 != 0 or args.copy_bytes > (1 << 30):
            raise SystemExit("--copy-bytes must be a positive multiple of 16, at most 1 GiB")
        a = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev) if args.copy_bytes < (1 << 30) else None
        torch.cuda.synchronize()
        marker.random_()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            if flush is not None:
                evict_mall(flush)
            b.copy_(a)
        torch.cuda.synchronize()
        marker.random_()
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                          "launches": args.steps}))
        return
    n = int(args.workload[3:])
    path = Path(n, dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    for c in path.calls:
        c.fn()
    segments = []
    for c in path.calls:
        torch.cuda.synchronize()
        marker.random_()
        torch.cuda.synchronize()
        reps = args.steps if getattr(c, "record", True) else 1
        for _ in range(reps):
            evict_mall(flush)
            c.fn()
        segments.append(dict(call=c.name if getattr(c, "record", True) else None, launches=reps, bytes=c.bytes,
                             elements=c.elements, kernel_bytes=c.kernel_bytes,
                             source_hash=kernel_source_hash(c.name)))
    torch.cuda.synchronize()
    marker.random_()
    torch.cuda.synchronize()
    print(json.dumps({"counters_pass": args.workload, "segments": segments}))


def emit(out, args):
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def progress(msg):
    """One line on stderr as each phase of the run ends (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU only; --gpus must be 1 "
                                   "(multi-GPU expert-parallel transport is not implemented)"}))
        sys.exit(2)
    import workloads
    configs = [int(c) for c in args.configs.split(",") if c]
    if args.workload:
        configs = [int(args.workload[3:])]
    w3 = workloads.config3() if (args.workload is None or args.workload == "cfg3") and not args.counters_pass \
        else None
    cpu = None
    if w3 is not None and not args.no_cpu_baseline and args.workload is None:
        cpu = cpu_baseline(w3, args.cpu_sample_tokens)           # on the host, before the GPU is touched
        progress(f"oracle baseline: {cpu['value']} {cpu['unit']}")
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.counters_pass:
        return main_counters_pass(args, dev)
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB: 4x the MALL
    # torch sets its GPU random generator up on first use (the marker kernel that
    # time_step launches before its timed steps), and GPU work right after that
    # runs slower for a while (measured: the first timed step 772 us against 726
    # us once it had been used): done here, before anything is timed
    torch.empty(64, dtype=torch.float32, device=dev).random_()
    torch.cuda.synchronize()
    kernels = {}
    head = None
    for n in configs:
        path = Path(n, dev, w3 if n == 3 else None)
        per = time_calls(path, args.reps, flush)
        headline_cfg = n == 3 and args.workload in (None, "cfg3")
        step = None
        if headline_cfg or args.workload is not None:
            # the timed step follows the per-call passes at once (the host-side work
            # of config_kernels comes after it): no idle pause for the clock to drop in
            step = time_step(path, args.steps, args.warmup, args.settle_s)
        kernels[f"cfg{n}"] = config_kernels(n, path, per)
        progress(f"config {n}: {len(per)} calls timed")
        if headline_cfg:
            head = (path,) + step
            progress(f"step timed: {step[0] * 1e3:.1f} us")
        elif args.workload is not None:
            calls = path.step_calls()
            ms_step, step_per = step
            total = sum(c.bytes for c in calls)
            emit({"metric": METRIC, "value": round(total / (ms_step / 1e3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
                  "steps": args.steps, "warmup": args.warmup, "settle_s": args.settle_s,
                  "ms_per_step": round(ms_step, 4),
                  "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
                  "data": "synthetic", "config": dict(path.desc, bytes_per_step=total),
                  "step_ms": {nm: round(v, 5) for nm, v in step_per.items()}, "kernels": kernels,
                  "cpu_baseline": None}, args)
            return
        del path
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if head is None:
        p3 = Path(3, dev, w3)
        head = (p3,) + time_step(p3, args.steps, args.warmup, args.settle_s)
    path3, ms_step, step_per = head
    emit(headline(path3, ms_step, step_per, args.steps, args.warmup, kernels, cpu, copy_reference(dev), args.settle_s),
         args)


if __name__ == "__main__":
    main()
