"""Benchmark of the block-scaled token codec hot path on one MI355X.

One step is one pass of the whole path over one batch of the dispatch workload
(4096 tokens x hidden 4096 BF16 ~ N(0,1), top-2 of 8 experts with
Zipf(1.2)-skewed routing and expert 7 empty, 16-row aligned slots):

  route plan -> NVFP4 pack -> NVFP4 direct receive (rowwise + RHT columnwise)
  -> MXFP8 pack -> MXFP8 receive -> unpack of the received rows to BF16
  -> combine backward: stochastic-rounding NVFP4 pack of a same-shaped
     gradient (Student-t(3) * 1e-3, Philox seed 1234) + its direct receive
  -> grouped dSwiGLU epilogue + FC1-gradient NVFP4 quantization over the
     routed rows (ffn 2048; preact ~ N(0,1), dy ~ N(0, 1e-2^2)).

value = algorithmic bytes (distinct inputs read once + outputs, padding rows
excluded) of all kernels of a step / step time, in GB/s.  Inputs are resident
in HBM before the timed region.  Per-call durations come from HIP events on
the stream the kernels run on.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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

HBM_PEAK_GBS = 8000.0
# Philox multiplies: 256 CUs x 64 lanes x 2.4 GHz, one 32x32->64-bit multiply
# (v_mad_u64_u32) per lane per clock (its measured issue rate on gfx950)
ALU_PEAK_TMULS = 256 * 64 * 2.4e9 / 1e12
PHILOX_MULS_PER_ELEMENT = 20          # ten rounds of two multiplies, one Philox call per element

# source files each call's kernels are built from (a counter summary is used
# only while these are unchanged)
_COMMON = ("common.h", "launch.h")
CALL_SOURCES = {
    "route_plan": ("route.hip",),
    "nvfp4_pack": ("pack.hip",), "nvfp4_pack_sr": ("pack.hip",), "mxfp8_pack": ("pack.hip",),
    "nvfp4_expert_scale": ("receive.hip",), "nvfp4_expert_scale_grad": ("receive.hip",),
    "nvfp4_direct_receive": ("receive.hip",), "nvfp4_direct_receive_grad": ("receive.hip",),
    "mxfp8_receive": ("unpack.hip",), "nvfp4_unpack": ("unpack.hip",),
    "dswiglu_nvfp4_quant": ("dswiglu.hip",),
    "nvfp4_pack_scatter": ("pack.hip",), "nvfp4_columnwise_grouped": ("receive.hip",),
    "nvfp4_direct_receive_kblock": ("receive.hip",), "dswiglu_nvfp4_quant_nodx": ("dswiglu.hip",),
    "mxfp4_receive": ("receive.hip",), "nvfp4_direct_receive_sr": ("receive.hip",),
    "dswiglu_nvfp4_quant_sr": ("dswiglu.hip",),
}
# the kernels each call launches (as named in a rocprofv3 kernel trace)
CALL_KERNELS = {
    "route_plan": ["k_route_single (<= 16K entries) or k_route_count + k_route_scan + k_route_scatter"],
    "nvfp4_pack": ["k_nvfp4_pack_wg (H >= 4096) or k_nvfp4_pack"], "nvfp4_pack_sr": ["k_nvfp4_pack_sr_rows (H <= 4096) or k_nvfp4_pack_sr"],
    "mxfp8_pack": ["k_mxfp8_pack"], "nvfp4_expert_scale": ["k_expert_scale"],
    "nvfp4_expert_scale_grad": ["k_expert_scale"], "nvfp4_direct_receive": ["k_nvfp4_receive"],
    "nvfp4_direct_receive_grad": ["k_nvfp4_receive"], "mxfp8_receive": ["k_mxfp8_receive"],
    "nvfp4_unpack": ["k_nvfp4_unpack"],
    "dswiglu_nvfp4_quant": ["k_dswiglu_epilogue", "k_dswiglu_reduce", "k_fc1_quant"],
    "nvfp4_pack_scatter": ["k_nvfp4_pack_wg / k_nvfp4_pack (scatter)", "k_zero_padding"],
    "nvfp4_columnwise_grouped": ["k_expert_scale_grouped", "k_nvfp4_receive (grouped rows)"],
    "nvfp4_direct_receive_kblock": ["k_nvfp4_receive (K-blocked columnwise layout)"],
    "dswiglu_nvfp4_quant_nodx": ["k_dswiglu_epilogue (max only)", "k_dswiglu_reduce", "k_fc1_quant (recompute)"],
    "mxfp4_receive": ["k_mxfp4_receive"],
    "nvfp4_direct_receive_sr": ["k_nvfp4_receive (stochastic columnwise codes)"],
    "dswiglu_nvfp4_quant_sr": ["k_dswiglu_epilogue", "k_dswiglu_reduce", "k_fc1_quant (stochastic codes)"],
}
# the combine-backward SR pack: one Philox4x32-10 word per element at counter
# row*hidden + col (element mode), carry-form decision (the hardware converter)
SR_MODE = 3  # EP_ROUND_SR_ELEMENT_CARRY
STEP_NAMES = ["route_plan", "nvfp4_pack", "nvfp4_expert_scale", "nvfp4_direct_receive", "mxfp8_pack",
              "mxfp8_receive", "nvfp4_unpack", "nvfp4_pack_sr", "nvfp4_expert_scale_grad",
              "nvfp4_direct_receive_grad", "dswiglu_nvfp4_quant"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=4096)
    p.add_argument("--json-out", default=None)
    p.add_argument("--only", default=None,
                   help="profiling aid: run only this call of the path (or 'copy': a 1 GiB device copy, the "
                        "reference for memory counters) --steps times, eagerly, and print what ran")
    p.add_argument("--workload", default="dispatch",
                   choices=["dispatch", "cfg1", "cfg2", "cfg3", "cfg4", "cfg5", "cfg2f", "cfg3f", "cfg2k", "cfg3k",
                            "cfg5r", "cfg2m", "cfg3m", "cfg4s", "cfg5s"],
                   help="dispatch (default): the full step on the 4096x4096 dispatch workload; cfgN: that "
                        "configuration's own path, for per-kernel figures")
    return p.parse_args()


# ---------------------------------------------------------------------------- bytes
def row_bytes(h):
    return 9 * h // 16 + 4


def algorithmic_bytes(T, H, k, E, r_cap, R, Tg, F):
    """Distinct input bytes read once + output bytes, per call of the step.
    R = routed rows (T*k), Tg = rows of the grouped MLP (= R), padding excluded."""
    rb = row_bytes(H)
    b = {}
    b["route_plan"] = T * k * 4 + E * 4 + (E + 1) * 4 + T * k * 4 + r_cap * 4
    b["nvfp4_pack"] = T * H * 2 + T * rb
    b["nvfp4_expert_scale"] = R * 4 + r_cap * 4 + (E + 1) * 4 + E * 4
    b["nvfp4_direct_receive"] = (T * rb + r_cap * 4 + (E + 1) * 4 + E * 4
                                 + R * (H // 2 + H // 16 + 4) + R * (H // 2 + H // 16))
    b["mxfp8_pack"] = T * H * 2 + T * H + T * (H // 32)
    b["mxfp8_receive"] = T * (H + H // 32) + r_cap * 4 + R * (H + H // 32)
    b["nvfp4_unpack"] = T * rb + R * 4 + R * H * 2
    b["nvfp4_pack_sr"] = T * H * 2 + T * rb + 16
    b["nvfp4_expert_scale_grad"] = b["nvfp4_expert_scale"]
    b["nvfp4_direct_receive_grad"] = b["nvfp4_direct_receive"]
    b["dswiglu_nvfp4_quant"] = (Tg * 2 * F * 2 + Tg * F * 2 + E * 4                 # epilogue in
                                + Tg * 2 * F * 2 + E * 4                            # dX out, amax
                                + Tg * 2 * F * 2                                    # quant reads dX
                                + 2 * Tg * (F + 2 * F // 16) + 2 * E * 4)            # row + col operands
    return b


# ---------------------------------------------------------------------------- inputs
def make_inputs(dev):
    import torch
    import workloads
    w = workloads.config2()
    T, H = w.x_bits.shape
    k = w.topk_idx.shape[1]
    rng = [np.random.default_rng(s) for s in np.random.SeedSequence(7).spawn(3)]
    grad = workloads.to_bf16_bits(rng[0].standard_t(3, size=(T, H)) * 1e-3)
    F = 2048
    R = T * k
    pre = workloads.to_bf16_bits(rng[1].standard_normal((R, 2 * F), dtype=np.float32))
    dy = workloads.to_bf16_bits(rng[2].standard_normal((R, F), dtype=np.float32) * np.float32(1e-2))

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    return dict(w=w, T=T, H=H, k=k, E=w.num_experts, A=w.alignment, F=F, R=R,
                x=bf(w.x_bits), grad=bf(grad), preact=bf(pre), dy=bf(dy),
                topk=torch.from_numpy(w.topk_idx).to(dev),
                sr=torch.tensor([1234, 0], dtype=torch.int64, device=dev),
                host=dict(x=w.x_bits, grad=grad, pre=pre, dy=dy, topk=w.topk_idx))


def evict_mall(buf):
    """Read a 1 GiB buffer (4x the 256 MB MALL) before an eager pass of per-call
    timings.  The read evicts what the MALL holds and writes back its dirty lines, so
    the pass starts with its inputs in HBM and no write-backs of earlier work ahead of
    its own traffic (a 1 GiB fill instead leaves 256 MB of dirty lines that the first
    calls pay for: a plain 128 MiB read after a fill runs at 2.6 TB/s, after this read
    at 6.0); it also keeps the GPU busy while the host enqueues the pass, so each event
    pair brackets GPU time only.  One read per pass, not one per call: a read right
    before every call made each call about 2 us slower, small ones included (7.8 ->
    10.4 us for the expert-scale pass), a cold start that the calls of a step do not
    see."""
    buf.amax()


# ---------------------------------------------------------------------------- the step
class Step:
    """Pre-allocated outputs; ``run`` launches one pass of the path."""

    def __init__(self, inp):
        import torch
        import moe_token_block_amd as m
        self.m = m
        self.inp = inp
        dev = inp["x"].device
        T, H, k, E, A, F, R = (inp[s] for s in ("T", "H", "k", "E", "A", "F", "R"))
        self.r_cap = m.ep_route_capacity(T, k, E, A)
        self.ws = torch.empty(max(m.lib().ep_route_workspace_bytes(T, k, E), 4), dtype=torch.uint8, device=dev)
        self.derr = torch.zeros(1, dtype=torch.int32, device=dev)
        self.plan = m.ep_route_plan(inp["topk"], E, A, d_error=self.derr, workspace=self.ws)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.packed = torch.empty((T, row_bytes(H)), **u8)
        self.packed_g = torch.empty((T, row_bytes(H)), **u8)
        mk = lambda: dict(row_codes=torch.empty((self.r_cap, H // 2), **u8),
                          row_scales=torch.empty((self.r_cap, H // 16), **u8),
                          row_t=torch.empty(self.r_cap, dtype=torch.float32, device=dev),
                          col_codes=torch.empty(self.r_cap * H // 2, **u8),
                          col_scales=torch.empty(self.r_cap * H // 16, **u8),
                          col_scale=torch.empty(E, dtype=torch.float32, device=dev))
        self.recv, self.recv_g = mk(), mk()
        self.mx = torch.empty(T * H + T * H // 32, **u8)
        self.mx_out = (torch.empty((self.r_cap, H), **u8), torch.empty((self.r_cap, H // 32), **u8))
        self.unpacked = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        # the unpack decodes the routed rows in grouped order (padding rows skipped)
        off = self.plan["offsets"].cpu().numpy()
        src = self.plan["src_row"].cpu().numpy()
        self.src_valid = torch.from_numpy(np.ascontiguousarray(src[: off[-1]][src[: off[-1]] >= 0])).to(dev)
        self.counts = self.plan["counts"]
        self.dsw_ws = torch.empty(m.lib().dswiglu_workspace_bytes(R, E), **u8)
        cap = R + 15 * E
        f32 = dict(dtype=torch.float32, device=dev)
        self.dsw = dict(dx=torch.empty((R, 2 * F), dtype=torch.bfloat16, device=dev), amax=torch.empty(E, **f32),
                        row_codes=torch.empty((R, F), **u8), row_scales=torch.empty((R, 2 * F // 16), **u8),
                        row_scale=torch.empty(E, **f32), col_codes=torch.empty(2 * F * cap // 2, **u8),
                        col_scales=torch.empty(2 * F * cap // 16, **u8), col_scale=torch.empty(E, **f32))
        self.names = list(STEP_NAMES)
        self.flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB: 4x the MALL

    def calls(self):
        m, i = self.m, self.inp
        H, E, A = i["H"], i["E"], i["A"]
        return [
            lambda: m.ep_route_plan(i["topk"], E, A, d_error=self.derr, workspace=self.ws, out=self.plan),
            lambda: m.ep_nvfp4_pack(i["x"], out=self.packed),
            lambda: m.ep_nvfp4_expert_scale(self.packed, H, self.plan, col_scale=self.recv["col_scale"]),
            lambda: m.ep_nvfp4_direct_receive_scaled(self.packed, H, self.plan, self.recv),
            lambda: m.ep_mxfp8_pack(i["x"], out=self.mx),
            lambda: m.ep_mxfp8_direct_receive(self.mx[: i["T"] * H].view(i["T"], H),
                                              self.mx[i["T"] * H:].view(i["T"], H // 32), self.plan, out=self.mx_out),
            lambda: m.ep_nvfp4_unpack(self.packed, H, src_row=self.src_valid, out=self.unpacked),
            lambda: m.ep_nvfp4_pack(i["grad"], SR_MODE, i["sr"], out=self.packed_g),
            lambda: m.ep_nvfp4_expert_scale(self.packed_g, H, self.plan, col_scale=self.recv_g["col_scale"]),
            lambda: m.ep_nvfp4_direct_receive_scaled(self.packed_g, H, self.plan, self.recv_g),
            lambda: m.dswiglu_nvfp4_quant(i["preact"], i["dy"], self.counts, out=self.dsw, workspace=self.dsw_ws),
        ]

    def run_concurrent(self):
        """The same calls as ``run``: the route plan first (every later call needs it
        or its counts), then four independent chains on their own streams (default
        priority) joined back into the calling stream -- the dSwiGLU chain, the
        combine-backward chain and the MXFP8 chain on three side streams, in that
        launch order, then the NVFP4 dispatch chain on the calling stream.  One fork
        and one join, no other cross-stream waits: measured 1.5% faster than starting
        the packs beside the route plan with a wait on it in every chain (each
        cross-stream wait costs a dependency resolution in the graph).  The longest
        chain (dSwiGLU) first: 182 -> 177 us against the order combine backward,
        MXFP8, dSwiGLU; every order with it first is within 1.5 us of the best."""
        import torch
        c = self.calls()
        main = torch.cuda.current_stream()
        if not hasattr(self, "side"):
            self.side = [torch.cuda.Stream() for _ in range(3)]
        c[0]()                                       # route plan
        for st in self.side:
            st.wait_stream(main)
        with torch.cuda.stream(self.side[2]):
            c[10]()                                  # dSwiGLU + FC1-grad quantization (needs the counts)
        with torch.cuda.stream(self.side[0]):
            c[7](); c[8](); c[9]()                   # SR pack, expert scale, receive of the gradient rows
        with torch.cuda.stream(self.side[1]):
            c[4](); c[5]()                           # MXFP8 pack and receive
        c[1](); c[2](); c[3](); c[6]()               # NVFP4 pack, expert scale, receive, unpack
        for st in self.side:
            main.wait_stream(st)

    def run(self, events=None):
        calls = self.calls()
        if events is not None:
            evict_mall(self.flush)
        for j, c in enumerate(calls):
            if events is not None:
                events[j][0].record()
            c()
            if events is not None:
                events[j][1].record()


# ---------------------------------------------------------------------------- per-config paths
class ConfigStep:
    """The path of one configuration on its own inputs (for per-kernel figures):
    cfg1/cfg3: route -> pack -> expert scale -> direct receive -> unpack of the grouped rows;
    cfg2: route -> pack -> expert scale -> direct receive -> MXFP8 pack -> MXFP8 receive;
    cfg4: route -> SR pack -> expert scale -> direct receive; cfg5: dSwiGLU + FC1-grad quant."""

    def __init__(self, which, dev):
        import torch
        import moe_token_block_amd as m
        import workloads
        self.m = m
        fused, kblock, recompute = which.endswith("f"), which.endswith("k"), which.endswith("r")
        mxfp4, sr_grad = which.endswith("m"), which.endswith("s")
        n = int(which[3:-1] if fused or kblock or recompute or mxfp4 or sr_grad else which[3:])
        w = workloads.CONFIGS[n]()
        self.w, self.n = w, n
        u8 = dict(dtype=torch.uint8, device=dev)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        self.flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        self.names, self.calls_, self.bytes = [], [], {}
        self.elements = None
        if n == 5:
            T, F, E = w.preact_bits.shape[0], w.dy_bits.shape[1], len(w.counts)
            self.pre, self.dy = bf(w.preact_bits), bf(w.dy_bits)
            self.counts = torch.from_numpy(w.counts).to(dev)
            cap = T + 15 * E
            f32 = dict(dtype=torch.float32, device=dev)
            self.out = dict(dx=None if recompute else torch.empty((T, 2 * F), dtype=torch.bfloat16, device=dev),
                            amax=torch.empty(E, **f32),
                            row_codes=torch.empty((T, F), **u8), row_scales=torch.empty((T, 2 * F // 16), **u8),
                            row_scale=torch.empty(E, **f32), col_codes=torch.empty(2 * F * cap // 2, **u8),
                            col_scales=torch.empty(2 * F * cap // 16, **u8), col_scale=torch.empty(E, **f32))
            self.ws = torch.empty(m.lib().dswiglu_workspace_bytes(T, E), **u8)
            if sr_grad:
                self.sr5 = torch.tensor([1234, 0], dtype=torch.int64, device=dev)
                self._add("dswiglu_nvfp4_quant_sr",
                          lambda: m.dswiglu_nvfp4_quant(self.pre, self.dy, self.counts, out=self.out, workspace=self.ws,
                                                        sr_state=self.sr5),
                          T * 2 * F * 2 + T * F * 2 + T * 2 * F * 2 + E * 4 + T * 2 * F * 2 + 2 * T * (F + 2 * F // 16)
                          + 2 * E * 4)
                self.desc = dict(workload=w.name + " (stochastic FC1-grad codes)", tokens=T, ffn=F, experts=E)
                return
            if recompute:
                # no dX written: inputs read once + the quantized operands and the maxima
                self._add("dswiglu_nvfp4_quant_nodx",
                          lambda: m.dswiglu_nvfp4_quant(self.pre, self.dy, self.counts, out=self.out, workspace=self.ws),
                          T * 2 * F * 2 + T * F * 2 + E * 4 + 2 * T * (F + 2 * F // 16) + 2 * E * 4)
            else:
                self._add("dswiglu_nvfp4_quant",
                          lambda: m.dswiglu_nvfp4_quant(self.pre, self.dy, self.counts, out=self.out, workspace=self.ws),
                          T * 2 * F * 2 + T * F * 2 + T * 2 * F * 2 + E * 4 + T * 2 * F * 2 + 2 * T * (F + 2 * F // 16)
                          + 2 * E * 4)
            self.desc = dict(workload=w.name + (" (dX not materialized)" if recompute else ""), tokens=T, ffn=F,
                             experts=E)
            return
        T, H = w.x_bits.shape
        k, E, A = w.topk_idx.shape[1], w.num_experts, w.alignment
        R = T * k
        self.elements = T * H
        self.x = bf(w.x_bits)
        self.topk = torch.from_numpy(w.topk_idx).to(dev)
        r_cap = m.ep_route_capacity(T, k, E, A)
        self.ws = torch.empty(max(m.lib().ep_route_workspace_bytes(T, k, E), 4), **u8)
        self.derr = torch.zeros(1, dtype=torch.int32, device=dev)
        self.plan = m.ep_route_plan(self.topk, E, A, d_error=self.derr, workspace=self.ws)
        self.packed = torch.empty((T, row_bytes(H)), **u8)
        self.recv = dict(row_codes=torch.empty((r_cap, H // 2), **u8), row_scales=torch.empty((r_cap, H // 16), **u8),
                         row_t=torch.empty(r_cap, dtype=torch.float32, device=dev),
                         col_codes=torch.empty(r_cap * H // 2, **u8), col_scales=torch.empty(r_cap * H // 16, **u8),
                         col_scale=torch.empty(E, dtype=torch.float32, device=dev))
        b = algorithmic_bytes(T, H, k, E, r_cap, R, R, 0)
        self._add("route_plan", lambda: m.ep_route_plan(self.topk, E, A, d_error=self.derr, workspace=self.ws,
                                                        out=self.plan), b["route_plan"])
        if mxfp4:
            # the MXFP4 receive of the same packed rows (alignment 32: 32-row columnwise blocks)
            A32 = max(A, 32)
            r_cap32 = m.ep_route_capacity(T, k, E, A32)
            self.plan32 = m.ep_route_plan(self.topk, E, A32)
            self.mx4 = dict(row_codes=torch.empty((r_cap32, H // 2), **u8), row_scales=torch.empty((r_cap32, H // 32), **u8),
                            col_codes=torch.empty(r_cap32 * H // 2, **u8), col_scales=torch.empty(r_cap32 * H // 32, **u8))
            self._add("nvfp4_pack", lambda: m.ep_nvfp4_pack(self.x, out=self.packed), b["nvfp4_pack"])
            self._add("mxfp4_receive", lambda: m.ep_mxfp4_direct_receive(self.packed, H, self.plan32, out=self.mx4),
                      T * row_bytes(H) + r_cap32 * 4 + (E + 1) * 4 + 2 * R * (H // 2 + H // 32))
            self.desc = dict(workload=w.name + " (MXFP4 receive, alignment 32)", tokens=T, hidden=H, experts=E,
                             top_k=k, alignment=A32)
            return
        if fused:
            # sender-side fused dispatch: pack straight into the grouped rows, then
            # the columnwise operand from those contiguous rows
            rb = row_bytes(H)
            self._add("nvfp4_pack_scatter", lambda: m.ep_nvfp4_pack_scatter(self.x, self.plan, out=self.recv),
                      T * H * 2 + R * rb)
            self._add("nvfp4_columnwise_grouped", lambda: m.ep_nvfp4_columnwise_grouped(self.recv, H, self.plan,
                                                                                        out=self.recv),
                      R * rb + R * (H // 2 + H // 16) + E * 4)
            self.desc = dict(workload=w.name + " (fused dispatch)", tokens=T, hidden=H, experts=E, top_k=k, alignment=A)
            return
        if n == 4:
            self.sr = torch.tensor([w.sr_seed, w.sr_counter_base], dtype=torch.int64, device=dev)
            self._add("nvfp4_pack_sr", lambda: m.ep_nvfp4_pack(self.x, SR_MODE, self.sr, out=self.packed),
                      b["nvfp4_pack_sr"])
        else:
            self._add("nvfp4_pack", lambda: m.ep_nvfp4_pack(self.x, out=self.packed), b["nvfp4_pack"])
        self._add("nvfp4_expert_scale", lambda: m.ep_nvfp4_expert_scale(self.packed, H, self.plan,
                                                                        col_scale=self.recv["col_scale"]),
                  b["nvfp4_expert_scale"])
        if sr_grad:
            self.sr_recv = torch.tensor([w.sr_seed or 1234, 1 << 40], dtype=torch.int64, device=dev)
            self._add("nvfp4_direct_receive_sr",
                      lambda: m.ep_nvfp4_direct_receive_sr(self.packed, H, self.plan, self.recv, self.sr_recv),
                      b["nvfp4_direct_receive"])
        elif kblock:
            self._add("nvfp4_direct_receive_kblock",
                      lambda: m.ep_nvfp4_direct_receive_kblock(self.packed, H, self.plan, self.recv),
                      b["nvfp4_direct_receive"])
        else:
            self._add("nvfp4_direct_receive",
                      lambda: m.ep_nvfp4_direct_receive_scaled(self.packed, H, self.plan, self.recv),
                      b["nvfp4_direct_receive"])
        if n == 2:
            self.mx = torch.empty(T * H + T * H // 32, **u8)
            self.mx_out = (torch.empty((r_cap, H), **u8), torch.empty((r_cap, H // 32), **u8))
            self._add("mxfp8_pack", lambda: m.ep_mxfp8_pack(self.x, out=self.mx), b["mxfp8_pack"])
            self._add("mxfp8_receive", lambda: m.ep_mxfp8_direct_receive(
                self.mx[: T * H].view(T, H), self.mx[T * H:].view(T, H // 32), self.plan, out=self.mx_out),
                b["mxfp8_receive"])
        if n in (1, 3):
            off = self.plan["offsets"].cpu().numpy()
            src = self.plan["src_row"].cpu().numpy()
            self.src_valid = torch.from_numpy(np.ascontiguousarray(src[: off[-1]][src[: off[-1]] >= 0])).to(dev)
            self.unpacked = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
            self._add("nvfp4_unpack", lambda: m.ep_nvfp4_unpack(self.packed, H, src_row=self.src_valid,
                                                                out=self.unpacked), b["nvfp4_unpack"])
        self.desc = dict(workload=w.name, tokens=T, hidden=H, experts=E, top_k=k, alignment=A)

    def _add(self, name, fn, nbytes):
        self.names.append(name)
        self.calls_.append(fn)
        self.bytes[name] = nbytes

    def calls(self):
        return self.calls_

    def run(self, events=None):
        if events is not None:
            evict_mall(self.flush)
        for j, c in enumerate(self.calls_):
            if events is not None:
                events[j][0].record()
            c()
            if events is not None:
                events[j][1].record()


# ---------------------------------------------------------------------------- CPU baseline
def cpu_baseline(inp, n_tok):
    """The oracle, as it stands, on the first n_tok tokens of the same workload (their
    routing, their gradient rows, and the grouped dSwiGLU rows they route to)."""
    from oracle import nvfp4, receive, mxfp8, dswiglu
    from oracle.routing import route_plan
    h = inp["host"]
    H, E, A, F, k = inp["H"], inp["E"], inp["A"], inp["F"], inp["k"]
    x = h["x"][:n_tok]
    topk = h["topk"][:n_tok]
    grad = h["grad"][:n_tok]
    R = n_tok * k
    pre, dy = h["pre"][:R], h["dy"][:R]
    t0 = time.perf_counter()
    plan = route_plan(topk, E, A)
    packed = nvfp4.pack_rows(x)
    receive.direct_receive(packed, H, topk, E, A)
    d, s = mxfp8.pack_rows(x)
    mxfp8.grouped_receive(d, s, plan["src_row"])
    nvfp4.unpack_rows(packed, H, plan["src_row"][plan["src_row"] >= 0])
    pg = nvfp4.pack_rows(grad, sr_seed=1234, sr_rule="carry")
    receive.direct_receive(pg, H, topk, E, A)
    counts = plan["counts"]
    dx = dswiglu.dswiglu(pre, dy)
    dswiglu.fc1_grad_quant(dx, counts, dswiglu.expert_amax(dx, counts))
    dt = time.perf_counter() - t0
    r_cap = plan["src_row"].shape[0]
    total = sum(algorithmic_bytes(n_tok, H, k, E, r_cap, R, R, F).values())
    return dict(value=round(total / dt / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"first {n_tok} tokens of the workload (their routing, gradient rows and "
                       f"{R} grouped dSwiGLU rows); {dt:.1f} s single-threaded numpy")


def kernel_source_hash(call):
    """Hash of the sources the call's kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_token_block_amd", "csrc")
    for f in sorted(CALL_SOURCES[call] + _COMMON):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(call, workload="dispatch"):
    """HBM bytes per launch of one call from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy reference), or None when the
    call's kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("workload") != workload:
        return None
    k = d.get("calls", {}).get(call)
    if k is None or k.get("source_hash") != kernel_source_hash(call):
        return None
    return k.get("hbm_bytes_per_launch")


def roofline_of(call, nbytes, ms, elements=None, workload="dispatch"):
    """Roofline record of one call: HBM-bound calls against 8 TB/s; the
    stochastic-rounding pack, bound by its Philox arithmetic, against the
    multiply issue rate."""
    if call == "nvfp4_pack_sr" and elements is not None:
        tmul = elements * PHILOX_MULS_PER_ELEMENT / (ms / 1e3) / 1e12
        return dict(bound="alu", achieved=round(tmul, 3), peak=round(ALU_PEAK_TMULS, 2), unit="Tmul/s",
                    frac=round(tmul / ALU_PEAK_TMULS, 4), traffic=traffic_from_profile(call, workload),
                    kernel=call, kernels=CALL_KERNELS[call], bytes_per_launch=nbytes, ms_per_launch=round(ms, 5))
    gbs = nbytes / (ms / 1e3) / 1e9
    return dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4),
                traffic=traffic_from_profile(call, workload), kernel=call, kernels=CALL_KERNELS[call],
                bytes_per_launch=nbytes, ms_per_launch=round(ms, 5))


def time_step(step, args):
    """K graph replays of one captured step (the timed region), then per-call HIP
    events in eager passes, each pass preceded by a MALL-evicting read (evict_mall)."""
    import torch
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    # the timed region: K replays of one captured step (no host work per kernel)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
        if hasattr(step, "run_concurrent"):
            step.run_concurrent()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        if hasattr(step, "run_concurrent"):
            step.run_concurrent()
        else:
            step.run()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # per-call durations: HIP events on the launch stream around every call of
    # eager steps (each preceded by the read described in evict_mall)
    n = len(step.names)
    reps = max(5, min(args.steps, 50))
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
          for _ in range(reps)]
    for r in range(reps):
        step.run(ev[r])
    torch.cuda.synchronize()
    per_ms = {name: float(np.mean([ev[r][j][0].elapsed_time(ev[r][j][1]) for r in range(reps)]))
              for j, name in enumerate(step.names)}
    return ms_step, per_ms


def main_config(args, dev):
    import torch
    step = ConfigStep(args.workload, dev)
    ms_step, per_ms = time_step(step, args)
    total = sum(step.bytes.values())
    kernels = {nm: dict(ms=round(per_ms[nm], 5), bytes=step.bytes[nm],
                        gbs=round(step.bytes[nm] / (per_ms[nm] / 1e3) / 1e9, 1),
                        frac=round(step.bytes[nm] / (per_ms[nm] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)) for nm in step.names}
    for nm in step.names:
        kernels[nm]["traffic"] = traffic_from_profile(nm, args.workload)
    dom = max(step.names, key=lambda nm: per_ms[nm])
    out = {"metric": "quantize/pack/receive GB/s (in+out) on 1 MI355X; % of HBM peak",
           "value": round(total / (ms_step / 1e3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16->nvfp4/mxfp8", "data": "synthetic",
           "config": dict(step.desc, bytes_per_step=total),
           "roofline": roofline_of(dom, step.bytes[dom], per_ms[dom], elements=step.elements,
                                   workload=args.workload),
           "kernels": kernels, "cpu_baseline": None}
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


def main_only(args, dev):
    """Counter-collection aid: run the calls before ONLY once each, launch a
    marker kernel (a torch random fill, used nowhere else), then run ONLY
    --steps times; a profile's dispatches after the marker are ONLY's.
    ONLY = 'copy' runs a 1 GiB device-to-device copy instead (the reference
    that scales the memory counters)."""
    import torch
    marker = torch.empty(64, dtype=torch.float32, device=dev)
    if args.only == "copy":
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        marker.random_()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                          "launches": args.steps}))
        return
    step = ConfigStep(args.workload, dev) if args.workload != "dispatch" else Step(make_inputs(dev))
    j = step.names.index(args.only)
    calls = step.calls()
    for c in calls[:j]:
        c()
    torch.cuda.synchronize()
    marker.random_()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        calls[j]()
    torch.cuda.synchronize()
    if hasattr(step, "bytes"):
        nbytes = step.bytes[args.only]
    else:
        i = step.inp
        nbytes = algorithmic_bytes(i["T"], i["H"], i["k"], i["E"], step.r_cap, i["R"], i["R"], i["F"])[args.only]
    print(json.dumps({"only": args.only, "workload": args.workload, "launches": args.steps,
                      "algorithmic_bytes_per_launch": nbytes}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1 "
                                   "(multi-GPU expert-parallel transport is not part of it)"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.only is not None:
        return main_only(args, dev)
    if args.workload != "dispatch":
        return main_config(args, dev)
    inp = make_inputs(dev)
    step = Step(inp)
    ms_step, per_ms = time_step(step, args)
    T, H, k, E, R, F = (inp[s] for s in ("T", "H", "k", "E", "R", "F"))
    by = algorithmic_bytes(T, H, k, E, step.r_cap, R, R, F)
    total = sum(by.values())
    value = total / (ms_step / 1e3) / 1e9
    kernels = {nm: dict(ms=round(per_ms[nm], 5), bytes=by[nm], gbs=round(by[nm] / (per_ms[nm] / 1e3) / 1e9, 1),
                        frac=round(by[nm] / (per_ms[nm] / 1e3) / 1e9 / HBM_PEAK_GBS, 4)) for nm in step.names}
    for nm in step.names:
        kernels[nm]["traffic"] = traffic_from_profile(nm)
    # the dominant kernel: the call with the largest share of the step's time
    dom = max(step.names, key=lambda nm: per_ms[nm])
    roofline = roofline_of(dom, by[dom], per_ms[dom], elements=T * H)
    roofline["dominant_by"] = "largest per-call time in the step"
    out = {
        "metric": "quantize/pack/receive GB/s (in+out) on 1 MI355X; % of HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->nvfp4/mxfp8", "data": "synthetic",
        "config": {"workload": "dispatch-4096x4096-e8-top2-zipf1.2 (+ SR combine-bwd grads, grouped dSwiGLU ffn 2048)",
                   "tokens": T, "hidden": H, "experts": E, "top_k": k, "alignment": inp["A"],
                   "bytes_per_step": total, "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    else:
        out["cpu_baseline"] = None
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
