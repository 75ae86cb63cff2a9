"""rocprofv3 summaries of the bench workloads, written under profiles/.

Run on a machine with an MI355X and rocprofv3, from the repository root; this
process itself never touches the GPU (every GPU run is a rocprofv3 child).

  python rocprof_summaries.py traffic [--workload dispatch] [--raw DIR]
      For every call of the step: one FETCH_SIZE run and one WRITE_SIZE run
      (one counter per run) of `bench.py --only CALL`; the dispatches after
      bench's marker kernel are CALL's.  A 1 GiB device copy measured the same
      way gives the scale of each counter (bytes moved / counter KiB).
      -> profiles/traffic_counters.json (per call: KiB per launch as read,
      scaled HBM bytes per launch, the hash of the call's kernel sources).
  python rocprof_summaries.py trace [--workload dispatch] [--raw DIR] [--steps K]
      Kernel-trace statistics of a bench run -> profiles/kernel_trace_<workload>.md
"""

import argparse
import csv
import datetime
import json
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports no GPU state)

WORKLOAD_NAMES = {"dispatch": "dispatch_4096x4096_e8_top2", "cfg1": "roundtrip_256x1024_e4_top1",
                  "cfg2": "dispatch_4096x4096_e8_top2_cfg", "cfg3": "dsv3_16384x7168_e32_top8",
                  "cfg4": "combine_bwd_sr_32768x4096_e16_top2", "cfg5": "dswiglu_fc1grad_14841x2x2048_e8"}


def run(cmd, timeout):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd="/tmp", timeout=timeout, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, env=dict(os.environ, TMPDIR="/tmp"))
    if r.returncode != 0:
        print(r.stdout[-4000:])
        raise SystemExit(f"failed ({r.returncode}): {' '.join(cmd)}")
    return r.stdout


def pmc_pass(counter, only, workload, steps, raw):
    out = os.path.join(raw, f"pmc_{only}_{counter}")
    cmd = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", out, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), "--only", only, "--workload", workload,
           "--steps", str(steps)]
    run(cmd, 240)
    rows = list(csv.DictReader(open(os.path.join(out, "run_counter_collection.csv"))))
    per = {}
    names = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d] = per.get(d, 0.0) + float(r["Counter_Value"])  # summed over the counter's dimensions
        names[d] = r["Kernel_Name"]
    marks = [d for d, n in names.items() if "distribution" in n or "random" in n.lower()]
    if not marks:
        raise SystemExit(f"marker kernel not found in {out}")
    after = sorted(d for d in per if d > max(marks))
    kib = sum(per[d] for d in after) / steps
    kernels = sorted({names[d].split("(")[0].replace("void ", "") for d in after})
    shown = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", "OUT", "-o", "run", "--", "python3",
             "bench.py", "--only", only, "--workload", workload, "--steps", str(steps)]
    return kib, kernels, " ".join(shown)


def traffic(args):
    raw = args.raw or tempfile.mkdtemp(prefix="mtb_pmc_")
    steps = 5
    ref = {}
    cmds = []
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        kib, _, cmd = pmc_pass(ctr, "copy", "dispatch", steps, raw)
        ref[ctr] = (1 << 30) / (kib * 1024.0)  # bytes moved per counted byte
        cmds.append(cmd)
    names = bench.STEP_NAMES if args.workload == "dispatch" else args.calls.split(",")
    calls = {}
    for nm in names:
        f, kernels, c1 = pmc_pass("FETCH_SIZE", nm, args.workload, steps, raw)
        w, _, c2 = pmc_pass("WRITE_SIZE", nm, args.workload, steps, raw)
        cmds += [c1, c2]
        calls[nm] = dict(kernels=kernels, fetch_kib_per_launch=round(f, 1), write_kib_per_launch=round(w, 1),
                         hbm_bytes_per_launch=int(f * 1024 * ref["FETCH_SIZE"] + w * 1024 * ref["WRITE_SIZE"]),
                         source_hash=bench.kernel_source_hash(nm))
    doc = dict(workload=args.workload, date=datetime.date.today().isoformat(),
               method="FETCH_SIZE and WRITE_SIZE in separate rocprofv3 --pmc runs, KiB summed over each "
                      "dispatch's dimensions, averaged over the launches after bench's marker; each scaled by "
                      "bytes/counted-byte of a 1 GiB device-to-device copy",
               copy_reference=dict(fetch_scale=round(ref["FETCH_SIZE"], 4), write_scale=round(ref["WRITE_SIZE"], 4)),
               calls=calls, commands=cmds)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


def trace(args):
    raw = args.raw or tempfile.mkdtemp(prefix="mtb_trace_")
    out = os.path.join(raw, f"trace_{args.workload}")
    bench_args = ["--workload", args.workload, "--steps", str(args.steps), "--warmup", "3", "--no-cpu-baseline"]
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", out, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py")] + bench_args
    text = run(cmd, 600)
    line = next((ln for ln in text.splitlines() if ln.startswith("{\"metric\"")), None)
    rows = list(csv.DictReader(open(os.path.join(out, "run_kernel_stats.csv"))))
    shown = " ".join(["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", "OUT", "-o", "run",
                      "--", "python3", "bench.py"] + bench_args)
    md = [f"# Kernel trace: bench.py --workload {args.workload}", "",
          "Command (from the repository root, via `python rocprof_summaries.py trace --workload "
          f"{args.workload}`):", "", "```", shown, "```", "",
          "All dispatches of the run: warm-up, the graph replays of the timed region and the eager per-call "
          "passes (each pass preceded by a 1 GiB read that evicts the MALL; the reduce_kernel row).", "",
          "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                  f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    # the eager per-call passes: every dispatch from the first 1 GiB read on runs alone
    # (one stream, nothing concurrent), so these durations compare with the bench's
    # per-call figures; the graph replays before them overlap calls on four streams
    trace_rows = list(csv.DictReader(open(os.path.join(out, "run_kernel_trace.csv"))))
    trace_rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(r["Kernel_Name"].split("(")[0].replace("void ", ""),
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in trace_rows]
    first_sweep = next((i for i, (n, us) in enumerate(dur) if "reduce_kernel" in n and us > 50.0), None)
    if first_sweep is not None:
        eager = {}
        for n, us in dur[first_sweep:]:
            if "reduce_kernel" in n or "fillBuffer" in n:     # the read and its reduction's semaphore clear
                continue
            eager.setdefault(n, []).append(us)
        md += ["", "Eager per-call passes only (each call alone, each pass after the MALL-evicting read; compare with the bench's "
               "per-call times below):", "", "| kernel | dispatches | avg us | min us |", "|---|---|---|---|"]
        for n, v in eager.items():
            md.append(f"| `{n}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} |")
    if line:
        d = json.loads(line)
        md += ["", "Bench line of the same profiled run (HIP-event per-call times, MALL flushed):", "",
               "| call | us | algorithmic MB | GB/s | frac of 8 TB/s |", "|---|---|---|---|---|"]
        for nm, k in d["kernels"].items():
            md.append(f"| {nm} | {k['ms'] * 1e3:.1f} | {k['bytes'] / 1e6:.1f} | {k['gbs']} | {k['frac']} |")
        md += ["", f"Step: {d['ms_per_step'] * 1e3:.1f} us, {d['value']} GB/s (graph replay)."]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{WORKLOAD_NAMES[args.workload]}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("wrote", path)


def main():
    p = argparse.ArgumentParser()
    p.add_argument("what", choices=["traffic", "trace"])
    p.add_argument("--workload", default="dispatch", choices=list(WORKLOAD_NAMES))
    p.add_argument("--calls", default="", help="comma-separated calls (non-dispatch workloads)")
    p.add_argument("--raw", default=None, help="directory for rocprofv3's raw output (default: a temp dir)")
    p.add_argument("--steps", type=int, default=50)
    args = p.parse_args()
    if args.raw:
        args.raw = os.path.abspath(args.raw)
        os.makedirs(args.raw, exist_ok=True)
    traffic(args) if args.what == "traffic" else trace(args)


if __name__ == "__main__":
    main()
