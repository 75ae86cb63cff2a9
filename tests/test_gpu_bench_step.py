"""The benchmark's timed step -- the route plan, then four chains on their own
streams captured in one HIP graph -- gives, on every replay, the outputs of the
same calls run eagerly one after another on one stream.

This is the configuration ``bench.py`` times (the config-2 dispatch workload
with its gradient rows and grouped dSwiGLU rows).  The eager outputs themselves
are checked against the oracle by the parity tests; here every output of the
step is compared byte for byte between the eager pass and three graph replays,
with every output zeroed (eager fill kernels) before each replay, so a replay
that skipped or raced a kernel would show.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _defined(step):
    """Every output of the step, cut to the part the calls define."""
    inp = step.inp
    H, F, E = inp["H"], inp["F"], inp["E"]
    off = int(step.plan["offsets"][-1])
    out = {}
    for name in ("counts", "offsets", "dst_row", "src_row", "d_error"):
        out["plan." + name] = step.plan[name]
    out["packed"] = step.packed
    out["packed_g"] = step.packed_g
    for tag, r in (("recv", step.recv), ("recv_g", step.recv_g)):
        out[tag + ".row_codes"] = r["row_codes"][:off]
        out[tag + ".row_scales"] = r["row_scales"][:off]
        out[tag + ".row_t"] = r["row_t"][:off]
        out[tag + ".col_codes"] = r["col_codes"][: H * off // 2]
        out[tag + ".col_scales"] = r["col_scales"][: H * off // 16]
        out[tag + ".col_scale"] = r["col_scale"]
    out["mx"] = step.mx
    out["mx_out.data"], out["mx_out.scales"] = step.mx_out
    out["unpacked"] = step.unpacked[: step.src_valid.numel()]
    counts = step.counts.cpu().numpy().astype(np.int64)
    rows, padded = int(counts.sum()), int(((counts + 15) // 16 * 16).sum())
    d = step.dsw
    for name in ("dx", "row_codes", "row_scales"):
        out["dsw." + name] = d[name][:rows]
    for name in ("amax", "row_scale", "col_scale"):
        out["dsw." + name] = d[name]
    out["dsw.col_codes"] = d["col_codes"][: 2 * F * padded // 2]
    out["dsw.col_scales"] = d["col_scales"][: 2 * F * padded // 16]
    return out


def _bytes(t):
    return t.contiguous().view(torch.uint8).reshape(-1)


def test_bench_step_graph_replays_match_eager():
    import bench
    dev = torch.device("cuda:0")
    inp = bench.make_inputs(dev)
    step = bench.Step(inp)
    print("bench step: eager reference pass", flush=True)
    step.run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in _defined(step).items()}
    # capture as the benchmark does: a warm-up of both forms on a side stream, then the graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
        step.run_concurrent()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run_concurrent()
    for rep in range(3):
        for v in _defined(step).values():
            v.zero_()
        torch.cuda.synchronize()
        print(f"bench step: graph replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = _defined(step)
        for k, want in ref.items():
            assert torch.equal(_bytes(got[k]), _bytes(want)), (rep, k)
