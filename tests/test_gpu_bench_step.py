"""Every call the benchmark times, captured in one HIP graph, gives on every
replay the outputs of the same calls run eagerly one after another on one
stream.

The calls are those of ``bench.Path`` at the dispatch workload (4096 tokens x
hidden 4096, top-2 of 8 experts: route plan, packs, receives in every layout
and format, the fused scatter path) and at the FC1-gradient workload (the
dSwiGLU epilogue with both quantizers, with and without dX, stochastic codes
too).  The eager outputs are checked against the oracle by the parity tests;
here every buffer the calls write is zeroed (eager fill kernels, outside the
graph) before the eager pass and before each of three replays, and compared
byte for byte, so a replay that skipped or raced a kernel, or a call that
cannot be captured (a host synchronisation, an allocation outside the graph's
pool), would show.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.contiguous().view(torch.uint8).reshape(-1)


def _zero(path):
    for v in path.outputs.values():
        v.zero_()
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", [2, 5])
def test_bench_calls_graph_replays_match_eager(cfg):
    import bench
    dev = torch.device("cuda:0")
    path = bench.Path(cfg, dev)
    calls = path.calls
    print(f"bench calls, config {cfg}: eager reference pass ({len(calls)} calls)", flush=True)
    _zero(path)
    for c in calls:
        c.fn()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in path.outputs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream, as capture requires
        for c in calls:
            c.fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c.fn()
    for rep in range(3):
        _zero(path)
        print(f"bench calls, config {cfg}: graph replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for k, want in ref.items():
            assert torch.equal(_bytes(path.outputs[k]), _bytes(want)), (cfg, rep, k)
