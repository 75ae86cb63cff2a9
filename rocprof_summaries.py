"""rocprofv3 summaries of the bench workloads, written under profiles/.

Run on a machine with an MI355X and rocprofv3, from the repository root; this
process itself never touches the GPU (every GPU run is a rocprofv3 child).

  python rocprof_summaries.py counters [--configs 1,2,3,4,5] [--raw DIR]
      Per configuration, three rocprofv3 --pmc runs of `bench.py --counters-pass
      --workload cfgN` (every call of the configuration, each K times between
      marker kernels, each launch after a MALL-evicting read): FETCH_SIZE;
      WRITE_SIZE; TCC_EA0_RDREQ_DRAM_sum + TCC_EA0_WRREQ_DRAM_sum +
      SQ_INSTS_VALU.  A 1 GiB device-to-device copy measured the same way gives
      the bytes per counted unit of each memory counter.
      -> profiles/counters.json (per call and configuration, per launch: the
      counters as read, HBM bytes = FETCH and WRITE scaled by the copy, DRAM
      request bytes scaled the same way, issued VALU instructions, and the hash
      of the call's kernel sources) and profiles/counters_cfgN.md.
  python rocprof_summaries.py kernels [--configs 1,2,3,4,5] [--raw DIR]
      Per configuration, rocprofv3 --kernel-trace of `bench.py --counters-pass
      --workload cfgN`: each call's kernel-only time per launch (its dispatches'
      durations summed) -> profiles/kernel_times.json, profiles/kernel_times_cfgN.md.
  python rocprof_summaries.py trace --workload cfgN|all [--raw DIR] [--steps K]
      Kernel-trace statistics of `bench.py --workload cfgN` (all: of the default
      `bench.py`, the command that prints the headline line), with the timed
      step's dispatches -> profiles/kernel_trace_<workload>.md
"""

import argparse
import csv
import datetime
import json
import os
import subprocess
import time
import sys
import tempfile

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports no GPU state)

WORKLOAD_NAMES = {"cfg1": "roundtrip_256x1024_e4_top1", "cfg2": "dispatch_4096x4096_e8_top2",
                  "cfg3": "dsv3_16384x7168_e32_top8", "cfg4": "combine_bwd_sr_32768x4096_e16_top2",
                  "cfg5": "dswiglu_fc1grad_14841x2x2048_e8"}
GROUPS = (("FETCH_SIZE",), ("WRITE_SIZE",), ("TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum", "SQ_INSTS_VALU"))


def run(cmd, timeout):
    """Run cmd, echoing its output line by line as it comes (a long profiled run
    shows its progress), and return that output."""
    print("+", " ".join(cmd), flush=True)
    t0 = time.monotonic()
    p = subprocess.Popen(cmd, cwd="/tmp", stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         env=dict(os.environ, TMPDIR="/tmp"))
    lines = []
    try:
        for line in p.stdout:
            lines.append(line)
            print("  " + line.rstrip()[:300], flush=True)
            if time.monotonic() - t0 > timeout:
                raise subprocess.TimeoutExpired(cmd, timeout)
        p.wait(timeout=max(1.0, timeout - (time.monotonic() - t0)))
    except subprocess.TimeoutExpired:
        p.kill()
        p.wait()
        raise SystemExit(f"timed out after {timeout} s: {' '.join(cmd)}")
    out = "".join(lines)
    if p.returncode != 0:
        raise SystemExit(f"failed ({p.returncode}): {' '.join(cmd)}")
    return out


def _is_marker(name):
    return "distribution" in name or "random" in name.lower()


def _is_evict(name):
    """The MALL-evicting read before each launch of a counters pass (a torch
    reduction, and the fill that initialises its one-element result), which
    belongs to no call: the library itself issues no fills."""
    return "reduce_kernel" in name or "fillBuffer" in name


def kernel_name(name):
    return name.split("(")[0].replace("void ", "")


def pmc_run(counters, workload, steps, raw, copy=False):
    """One rocprofv3 --pmc run of a counters pass; returns (per segment: {counter: value
    summed over the segment's dispatches and dimensions}, per segment kernel names,
    the pass's JSON line, the command as shown in the summaries)."""
    tag = "copy" if copy else workload
    out = os.path.join(raw, f"pmc_{tag}_{'_'.join(counters)}")
    bench_args = ["--counters-pass", "--steps", str(steps)] + (["--only", "copy"] if copy else ["--workload", workload])
    cmd = ["rocprofv3", "--pmc"] + list(counters) + ["--output-format", "csv", "-d", out, "-o", "run", "--",
                                                      sys.executable, os.path.join(ROOT, "bench.py")] + bench_args
    text = run(cmd, 600)
    line = json.loads(next(ln for ln in text.splitlines() if ln.startswith("{\"")))
    rows = list(csv.DictReader(open(os.path.join(out, "run_counter_collection.csv"))))
    disp = {}
    for r in rows:
        d = disp.setdefault(int(r["Dispatch_Id"]), dict(name=r["Kernel_Name"], ctr={}))
        d["ctr"][r["Counter_Name"]] = d["ctr"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(disp)
    marks = [i for i in ids if _is_marker(disp[i]["name"])]
    segs = []
    for a, b in zip(marks, marks[1:]):
        tot, names, per_k = {}, set(), {}
        for i in ids:
            if a < i < b and not _is_evict(disp[i]["name"]):
                nm = kernel_name(disp[i]["name"])
                names.add(nm)
                pk = per_k.setdefault(nm, {})
                for c, v in disp[i]["ctr"].items():
                    tot[c] = tot.get(c, 0.0) + v
                    pk[c] = pk.get(c, 0.0) + v
        segs.append((tot, sorted(names), per_k))
    shown = " ".join(["rocprofv3", "--pmc"] + list(counters) + ["--output-format", "csv", "-d", "OUT", "-o", "run",
                                                              "--", "python3", "bench.py"] + bench_args)
    return segs, line, shown


def counters(args):
    raw = args.raw or tempfile.mkdtemp(prefix="mtb_pmc_")
    steps = 5
    cmds = []
    ref = {}
    for g in GROUPS:
        segs, line, shown = pmc_run(g, None, steps, raw, copy=True)
        cmds.append(shown)
        tot = segs[0][0]
        for c in g:
            if c in ("FETCH_SIZE", "TCC_EA0_RDREQ_DRAM_sum"):
                ref[c] = line["bytes_read"] * steps / (tot[c] * (1024.0 if c == "FETCH_SIZE" else 1.0))
            elif c in ("WRITE_SIZE", "TCC_EA0_WRREQ_DRAM_sum"):
                ref[c] = line["bytes_written"] * steps / (tot[c] * (1024.0 if c == "WRITE_SIZE" else 1.0))
    path = os.path.join(args.out_dir, "counters.json")
    prev = os.path.join(ROOT, "profiles", "counters.json")
    doc = json.load(open(path if os.path.exists(path) else prev)) if os.path.exists(path) or os.path.exists(prev) \
        else {}
    calls = doc.get("calls", {})
    for n in [int(c) for c in args.configs.split(",") if c]:
        wl = f"cfg{n}"
        per = {}
        for g in GROUPS:
            segs, line, shown = pmc_run(g, wl, steps, raw)
            cmds.append(shown)
            for (tot, names, per_k), seg in zip(segs, line["segments"]):
                if seg["call"] is None:
                    continue
                rec = per.setdefault(seg["call"], dict(kernels=names, launches=seg["launches"],
                                                       algorithmic_bytes=seg["bytes"], source_hash=seg["source_hash"],
                                                       per_kernel={}))
                for c in g:
                    rec[c] = tot.get(c, 0.0) / seg["launches"]
                for k, kv in per_k.items():
                    kr = rec["per_kernel"].setdefault(k, {})
                    for c in g:
                        kr[c] = kv.get(c, 0.0) / seg["launches"]
        lines = [f"# Counters per launch: bench.py --counters-pass --workload {wl}", "",
                 f"Date {datetime.date.today().isoformat()}.  Each call {steps} times, each launch after a read of a "
                 "1 GiB buffer that evicts the MALL; values summed over the counter's dimensions and the call's "
                 "dispatches, divided by the launches.  HBM bytes = FETCH_SIZE KiB x 1024 x "
                 f"{ref['FETCH_SIZE']:.3f} + WRITE_SIZE KiB x 1024 x {ref['WRITE_SIZE']:.3f} (the bytes a 1 GiB "
                 "device copy moves per counted byte); DRAM bytes = the TCC_EA0 DRAM read/write requests scaled "
                 f"by the same copy ({ref['TCC_EA0_RDREQ_DRAM_sum']:.1f} / {ref['TCC_EA0_WRREQ_DRAM_sum']:.1f} "
                 "bytes per request).  Both count what leaves the L2 for the memory side; MALL hits are not "
                 "separated by any counter here.", "", "Commands (from the repository root):", "", "```"]
        lines += [c for c in cmds if wl in c or "copy" in c] + ["```", "",
                  "| call | kernels | algorithmic MB | HBM MB (fetch+write) | ratio | DRAM MB (rd+wr) | ratio | "
                  "VALU instr | VALU / element |", "|---|---|---|---|---|---|---|---|---|"]
        for call, rec in per.items():
            hbm = rec["FETCH_SIZE"] * 1024 * ref["FETCH_SIZE"] + rec["WRITE_SIZE"] * 1024 * ref["WRITE_SIZE"]
            dram = (rec["TCC_EA0_RDREQ_DRAM_sum"] * ref["TCC_EA0_RDREQ_DRAM_sum"]
                    + rec["TCC_EA0_WRREQ_DRAM_sum"] * ref["TCC_EA0_WRREQ_DRAM_sum"])
            rec.update(hbm_bytes=int(hbm), dram_bytes=int(dram), valu_insts=int(rec["SQ_INSTS_VALU"]))
            seg = next(s for s in line["segments"] if s["call"] == call)
            vpe = (f"{rec['valu_insts'] * 64 / seg['elements']:.1f}" if seg.get("elements") else "")
            lines.append(f"| {call} | {', '.join('`' + k + '`' for k in rec['kernels'])} | "
                         f"{rec['algorithmic_bytes'] / 1e6:.1f} | {hbm / 1e6:.1f} | {hbm / rec['algorithmic_bytes']:.2f} | "
                         f"{dram / 1e6:.1f} | {dram / rec['algorithmic_bytes']:.2f} | {rec['valu_insts']:.3g} | {vpe} |")
            for k, kr in rec["per_kernel"].items():
                khbm = kr["FETCH_SIZE"] * 1024 * ref["FETCH_SIZE"] + kr["WRITE_SIZE"] * 1024 * ref["WRITE_SIZE"]
                kdram = (kr["TCC_EA0_RDREQ_DRAM_sum"] * ref["TCC_EA0_RDREQ_DRAM_sum"]
                         + kr["TCC_EA0_WRREQ_DRAM_sum"] * ref["TCC_EA0_WRREQ_DRAM_sum"])
                kr.update(hbm_bytes=int(khbm), dram_bytes=int(kdram), valu_insts=int(kr["SQ_INSTS_VALU"]))
                if len(rec["per_kernel"]) > 1:
                    lines.append(f"| &nbsp;&nbsp;of which | `{k}` | | {khbm / 1e6:.1f} | | {kdram / 1e6:.1f} | | "
                                 f"{kr['valu_insts']:.3g} | |")
            calls[f"{wl}/{call}"] = rec
        with open(os.path.join(args.out_dir, f"counters_{wl}_{WORKLOAD_NAMES[wl]}.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    doc = dict(date=datetime.date.today().isoformat(),
               method="bench.py --counters-pass under rocprofv3 --pmc, three counter groups per configuration; "
                      "memory counters scaled by a 1 GiB device-to-device copy",
               copy_reference={k: round(v, 4) for k, v in ref.items()}, calls=calls)
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


def kernel_times(args):
    """Kernel-only times per call: rocprofv3 --kernel-trace of the counters pass
    (each call K times between marker kernels, each launch after the MALL-evicting
    read), the call's dispatches between two markers summed per launch."""
    raw = args.raw or tempfile.mkdtemp(prefix="mtb_ktimes_")
    steps = 10
    path = os.path.join(args.out_dir, "kernel_times.json")
    prev = os.path.join(ROOT, "profiles", "kernel_times.json")   # the configurations not re-run are kept
    doc = json.load(open(path if os.path.exists(path) else prev)) if os.path.exists(path) or os.path.exists(prev) \
        else {}
    calls = doc.get("calls", {})
    for n in [int(c) for c in args.configs.split(",") if c]:
        wl = f"cfg{n}"
        out = os.path.join(raw, f"ktimes_{wl}")
        bench_args = ["--counters-pass", "--steps", str(steps), "--workload", wl]
        cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", out, "-o", "run", "--",
               sys.executable, os.path.join(ROOT, "bench.py")] + bench_args
        text = run(cmd, 600)
        line = json.loads(next(ln for ln in text.splitlines() if ln.startswith("{\"")))
        rows = sorted(csv.DictReader(open(os.path.join(out, "run_kernel_trace.csv"))),
                      key=lambda r: int(r["Start_Timestamp"]))
        marks = [i for i, r in enumerate(rows) if _is_marker(r["Kernel_Name"])]
        shown = " ".join(["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", "OUT", "-o",
                          "run", "--", "python3", "bench.py"] + bench_args)
        md = [f"# Kernel-only time per call: bench.py --counters-pass --workload {wl}", "",
              f"Date {datetime.date.today().isoformat()}.  Command (from the repository root, via "
              f"`python rocprof_summaries.py kernels --configs {n}`):", "", "```", shown, "```", "",
              f"Each call {steps} times, each launch after a read of a 1 GiB buffer that evicts the MALL (the torch "
              "reduction, not counted); a call's time per launch is the sum of its dispatches' durations "
              "(start to end of each kernel, as the trace records them) summed per launch; the median launch and "
              "the interquartile range are reported, and GB/s is the algorithmic bytes over the median.", "",
              "| call | kernel | dispatches | median us | IQR us | call us per launch: median (IQR) | "
              "algorithmic MB | GB/s | frac of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
        for (a, b), seg in zip(zip(marks, marks[1:]), line["segments"]):
            if seg["call"] is None:
                continue
            per, launches = {}, []
            for r in rows[a + 1:b]:
                if _is_evict(r["Kernel_Name"]):
                    if "reduce_kernel" in r["Kernel_Name"]:
                        launches.append(0.0)        # each launch follows one evicting read
                    continue
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                per.setdefault(kernel_name(r["Kernel_Name"]), []).append(d)
                if launches:
                    launches[-1] += d
            lq = np.percentile(launches, [25, 50, 75]) if launches else [0.0, 0.0, 0.0]
            us = float(lq[1])                       # the median launch
            gbs = seg["bytes"] / (us / 1e6) / 1e9
            calls[f"{wl}/{seg['call']}"] = dict(source_hash=seg["source_hash"], launches=len(launches),
                                               us_per_launch=round(us, 3), us_p25=round(float(lq[0]), 3),
                                               us_p75=round(float(lq[2]), 3), algorithmic_bytes=seg["bytes"],
                                               kernels={k: round(float(np.median(v)), 3) for k, v in per.items()})
            first = True
            kb = seg.get("kernel_bytes") or {}
            for k, v in per.items():
                part = next((p for p in kb if p in k), None)
                if first:
                    tail = (f"{us:.2f} ({lq[0]:.2f}-{lq[2]:.2f}) | {seg['bytes'] / 1e6:.1f} | {gbs:.0f} | "
                            f"{gbs / bench.HBM_PEAK_GBS:.3f} |")
                elif part is not None:
                    kg = kb[part] / (float(np.median(v)) / 1e6) / 1e9
                    tail = f"(this kernel) | {kb[part] / 1e6:.1f} | {kg:.0f} | {kg / bench.HBM_PEAK_GBS:.3f} |"
                else:
                    tail = "| | | |"
                md.append(f"| {seg['call'] if first else ''} | `{k}` | {len(v)} | {float(np.median(v)):.2f} | "
                          f"{float(np.percentile(v, 25)):.2f}-{float(np.percentile(v, 75)):.2f} | " + tail)
                first = False
                if part is not None and k == next(iter(per)):
                    kg = kb[part] / (float(np.median(v)) / 1e6) / 1e9
                    md.append(f"| | (`{k}` alone) | | | | (this kernel) | {kb[part] / 1e6:.1f} | {kg:.0f} | "
                              f"{kg / bench.HBM_PEAK_GBS:.3f} |")
        with open(os.path.join(args.out_dir, f"kernel_times_{wl}_{WORKLOAD_NAMES[wl]}.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
    doc = dict(date=datetime.date.today().isoformat(),
               method="rocprofv3 --kernel-trace of bench.py --counters-pass; per call, the sum of its dispatches' "
                      "durations per launch", calls=calls)
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


def trace(args):
    raw = args.raw or tempfile.mkdtemp(prefix="mtb_trace_")
    out = os.path.join(raw, f"trace_{args.workload}")
    # "all": the bench's default command, exactly as the headline line is produced
    bench_args = [] if args.workload == "all" else \
        ["--workload", args.workload, "--steps", str(args.steps), "--warmup", "5", "--no-cpu-baseline"]
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", out, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py")] + bench_args
    text = run(cmd, 600)
    line = next((ln for ln in text.splitlines() if ln.startswith("{\"metric\"")), None)
    rows = list(csv.DictReader(open(os.path.join(out, "run_kernel_stats.csv"))))
    shown = " ".join(["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", "OUT", "-o", "run",
                      "--", "python3", "bench.py"] + bench_args)
    title = "bench.py (default: configurations 1-5 per call, the configuration-3 step timed)" \
        if args.workload == "all" else f"bench.py --workload {args.workload}"
    md = [f"# Kernel trace: {title}", "",
          f"Date {datetime.date.today().isoformat()}.  Command (from the repository root, via "
          f"`python rocprof_summaries.py trace --workload {args.workload}`):", "", "```", shown, "```", "",
          "All dispatches of the run: the per-call passes (each after a 1 GiB read that evicts the MALL: the "
          "reduce_kernel rows) and the eager steps of the timed region.", "",
          "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        md.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                  f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    # the timed region: the dispatches between the two marker kernels bench.time_step
    # launches right before and right after its timed steps
    trace_rows = list(csv.DictReader(open(os.path.join(out, "run_kernel_trace.csv"))))
    trace_rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(trace_rows) if _is_marker(r["Kernel_Name"])]
    per = {}
    for r in trace_rows[marks[-2] + 1:marks[-1]]:
        nm = r["Kernel_Name"].split("(")[0].replace("void ", "")
        per.setdefault(nm, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    md += ["", f"Timed region ({args.steps if args.workload != 'all' else 20} eager steps; the dispatches between "
           "the marker kernels bench.py launches right before and right after it):", "", "| kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
    for nm, v in per.items():
        md.append(f"| `{nm}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    if line:
        d = json.loads(line)
        md += ["", "Bench line of the same profiled run (HIP events):", "",
               "| call | us per launch (per-call passes) | algorithmic MB | GB/s | frac of 8 TB/s |",
               "|---|---|---|---|---|"]
        for cfg, v in d["kernels"].items():
            for nm, k in v["calls"].items():
                md.append(f"| {nm} | {k['ms'] * 1e3:.1f} | {k['bytes'] / 1e6:.1f} | {k['gbs']} | {k['frac']} |")
        step_ms = d.get("step_ms") or d.get("config", {}).get("step_ms", {})
        md += ["", f"Step (timed region): {d['ms_per_step'] * 1e3:.1f} us, {d['value']} GB/s; per call (HIP events) "
               + ", ".join(f"{nm} {v * 1e3:.1f} us" for nm, v in step_ms.items()) + "."]
    name = "bench_default_" + WORKLOAD_NAMES["cfg3"] if args.workload == "all" else WORKLOAD_NAMES[args.workload]
    path = os.path.join(args.out_dir, f"kernel_trace_{name}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("wrote", path)


def main():
    p = argparse.ArgumentParser()
    p.add_argument("what", choices=["counters", "kernels", "trace"])
    p.add_argument("--workload", default="cfg3", choices=list(WORKLOAD_NAMES) + ["all"])
    p.add_argument("--configs", default="1,2,3,4,5")
    p.add_argument("--raw", default=None, help="directory for rocprofv3's raw output (default: a temp dir)")
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"), help="where the summaries go")
    args = p.parse_args()
    args.out_dir = os.path.abspath(args.out_dir)
    os.makedirs(args.out_dir, exist_ok=True)
    if args.raw:
        args.raw = os.path.abspath(args.raw)
        os.makedirs(args.raw, exist_ok=True)
    {"counters": counters, "kernels": kernel_times, "trace": trace}[args.what](args)


if __name__ == "__main__":
    main()
