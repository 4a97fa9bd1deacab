#!/usr/bin/env python3
"""Summaries of rocprofv3 runs of bench.py, for profiles/ and for bench.py's
roofline `traffic` field.

Three modes, each reading the CSV output of one rocprofv3 run over a
`bench.py --workload W ...` command:

  --fetch F.csv --write W.csv --calib-mib N
      HBM traffic per launch from one `--pmc FETCH_SIZE` pass and one
      `--pmc WRITE_SIZE` pass. The calibration kernels bench.py runs after its
      timed region with --calib-copy-mib N (a torch fill that writes N MiB,
      then a torch add that reads N MiB and writes N MiB) give the
      counter-to-bytes factors: fetch factor = add's FETCH_SIZE / N MiB, write
      factor = fill's WRITE_SIZE / N MiB. Writes profiles/traffic_<W>.json
      (read by bench.py, which reports a GEMM's figure only while the source
      hash recorded here still matches) and profiles/traffic_<W>.md.
  --util U.csv
      One `--pmc MfmaUtil VALUBusy SQ_INSTS_VALU SQ_INSTS_MFMA` pass, per
      launch of the step: profiles/util_<W>.md.
  --trace T.csv [--stats S.csv] [--bench-line B.json] --steps K
      One `--kernel-trace --stats` pass: each launch of the step's average
      duration over all its dispatches and over the last K steps (the timed
      ones, when bench.py ran with --no-lowrank-overhead), the rocprofv3 stats
      table, and the bench.py line's event averages: profiles/trace_<W>_step.md.

The library's dispatches are labelled by their position in the step: bench.py
launches the same sequence every step (for a stream of layers, quantizer and
GEMM per layer, then the GEMV), so the k-th library dispatch is launch
k mod (launches per step). Several layers of the DiT block share one kernel
instantiation, so names alone would mix them.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))

# kernel-name substring -> source file
SOURCES = [("gemm_fp4_big_kernel", "gemm_fp4.hip"), ("gemm_w4a4_kernel", "gemm_w4a4.hip"),
           ("chain_reduce_kernel", "gemm_w4a4.hip"), ("splitk_reduce_kernel", "gemm_w4a4.hip"),
           ("gemm_nvfp4_kernel", "gemm_nvfp4.hip"),
           ("quantize_act_kernel", "quantize_act.hip"), ("awq_gemv", "awq_gemv.hip")]


def step_pattern(workload: str):
    """Labels of the library dispatches of one bench.py step, in order:
    (layer, entry point, kernel-name substring that must match). A fused MLP
    chain is the up-projection's GEMM (INT4 or FP4 kernel) and the reduce of
    its low-rank partials; the next layer then has no quantizer launch."""
    import bench
    import synth
    names = bench.WORKLOADS.get(workload, (workload,))
    chained = bench.CHAINS.get(workload, ())
    pat = []
    for i, name in enumerate(names):
        cfg = synth.CONFIGS[name]
        if i == 0 or names[i - 1] not in chained:
            pat.append((name, "svdq_quantize_act", "quantize_act_kernel"))
        if name in chained:
            pat.append((name, "svdq_gemm_w4a4_mlp", "gemm_"))
            if synth.CONFIGS[names[i + 1]].rank > 0:
                pat.append((name, "svdq_gemm_w4a4_mlp.reduce", "chain_reduce_kernel"))
        else:
            gk = "gemm_nvfp4_kernel" if cfg.fmt == "nvfp4_g16" else "gemm_"
            pat.append((name, bench.gemm_name(cfg), gk))
            if bench.splitk_bytes(cfg):   # the split-K GEMM adds its partials in a second kernel
                pat.append((name, "svdq_gemm_w4a4_splitk.reduce", "splitk_reduce_kernel"))
    return pat + [("gemv", "awq_gemv_w4a16", "awq_gemv")]


def library_dispatches(rows, name_key="Kernel_Name"):
    """Rows of library kernels (namespace svdq::) in dispatch order."""
    return [r for r in rows if "svdq::" in r[name_key]]


def label(dispatches, pattern, name_key="Kernel_Name"):
    """[(label tuple, [rows])]: one entry per launch occurrence, checking each
    dispatch's kernel against its slot. A launch made of several dispatches
    of one kernel (the quantizer's K split: a low-rank pass, then the codes)
    keeps them together: a dispatch that does not fit the next slot but fits
    the current one joins the current occurrence."""
    out = []
    s = 0
    for i, r in enumerate(dispatches):
        nxt = pattern[s % len(pattern)]
        if nxt[2] in r[name_key]:
            out.append((nxt, [r]))
            s += 1
        elif out and out[-1][0][2] in r[name_key]:
            out[-1][1].append(r)
        else:
            raise SystemExit(f"dispatch {i}: {r[name_key][:80]} does not match the step's slot {nxt}")
    return out


def source_of(kernel_name: str):
    for sub, src in SOURCES:
        if sub in kernel_name:
            return src
    return None


def source_sha(fname: str) -> str:
    p = os.path.join(ROOT, "bit_diffusion_transformer_act_amd", "csrc", fname)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def counter_per_dispatch(path: str, counter: str):
    """[{Kernel_Name, value}] in dispatch order (summed over the counter's instances)."""
    acc = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        if key not in acc:
            acc[key] = {"Kernel_Name": r["Kernel_Name"], "value": 0.0}
        acc[key]["value"] += float(r["Counter_Value"])
    return list(acc.values())


def short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def traffic(args, pattern):
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    calib_kib = args.calib_mib * 1024.0
    elem_f = [d["value"] for d in fetch if "elementwise" in d["Kernel_Name"]]
    elem_w = [d["value"] for d in write if "elementwise" in d["Kernel_Name"]]
    if len(elem_f) < 2 or len(elem_w) < 2:
        raise SystemExit("calibration kernels not found (run bench.py with --calib-copy-mib)")
    # the add reads N MiB (the largest fetch); the fill and the add each write N MiB
    f_factor = max(elem_f) / calib_kib
    w_factor = sorted(elem_w)[-1] / calib_kib

    fl = label(library_dispatches(fetch), pattern)
    wl = label(library_dispatches(write), pattern)
    per = collections.OrderedDict()
    for (lab, ds) in fl:
        per.setdefault(lab, {"f": [], "w": [], "kernel": ds[-1]["Kernel_Name"]})["f"].append(
            sum(d["value"] for d in ds))
    for (lab, ds) in wl:
        per[lab]["w"].append(sum(d["value"] for d in ds))

    layers = collections.OrderedDict()
    lines = [f"# HBM traffic per launch, workload {args.workload}", "",
             f"command: {args.command}", "",
             f"calibration: fetch factor {f_factor:.4f}, write factor {w_factor:.4f} "
             f"(torch add / fill of {args.calib_mib} MiB run by the same command); launches labelled by "
             "their position in the step", "",
             "| layer | entry point | kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | "
             "HBM write MB | total MB |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (layer, api, _), v in per.items():
        fk, wk = sum(v["f"]) / len(v["f"]), sum(v["w"]) / len(v["w"])
        rd, wr = fk / f_factor * 1024, wk / w_factor * 1024
        src = source_of(v["kernel"])
        rec = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "hbm_read_bytes": round(rd),
               "hbm_write_bytes": round(wr), "hbm_bytes_per_launch": round(rd + wr), "launches": len(v["f"]),
               "kernel": short(v["kernel"]), "source": src, "source_sha": source_sha(src)}
        layers.setdefault(layer, {"kernels": {}})["kernels"][api] = rec
        lines.append(f"| {layer} | {api} | `{short(v['kernel'])}` | {len(v['f'])} | {fk:.0f} | {wk:.0f} | "
                     f"{rd / 1e6:.1f} | {wr / 1e6:.1f} | {(rd + wr) / 1e6:.1f} |")
    # each layer's GEMM (the roofline's kernel) at the layer's top level
    for layer, d in layers.items():
        for api, rec in d["kernels"].items():
            if api.startswith("svdq_gemm") and not api.endswith(".reduce"):
                d.update({"source": rec["source"], "source_sha": rec["source_sha"],
                          "hbm_bytes_per_launch": rec["hbm_bytes_per_launch"], "entry_point": api})
    out = {"workload": args.workload, "calib_mib": args.calib_mib, "fetch_factor": round(f_factor, 4),
           "write_factor": round(w_factor, 4), "command": args.command}
    import bench
    if args.workload in bench.WORKLOADS:
        out["layers"] = layers
    else:
        d = layers[args.workload]
        out.update({k: d[k] for k in ("source", "source_sha", "hbm_bytes_per_launch")})
        out["kernels"] = d["kernels"]
    write_out(f"traffic_{args.workload}.json", json.dumps(out, indent=1))
    write_out(f"traffic_{args.workload}.md", "\n".join(lines) + "\n")
    print("\n".join(lines))


UTIL_COUNTERS = ("MfmaUtil", "VALUBusy", "SQ_INSTS_MFMA", "SQ_INSTS_VALU")


def util(args, pattern):
    """Per launch of the step: the average over its dispatches of each counter."""
    per_counter = {c: label(library_dispatches(counter_per_dispatch(args.util, c)), pattern)
                   for c in UTIL_COUNTERS}
    acc = collections.OrderedDict()
    for c, lst in per_counter.items():
        for lab, ds in lst:
            # busy percentages of a multi-dispatch launch: its last (main) dispatch's
            v = sum(d["value"] for d in ds) if c.startswith("SQ_") else ds[-1]["value"]
            acc.setdefault(lab, {"kernel": ds[-1]["Kernel_Name"], **{k: [] for k in UTIL_COUNTERS}})[c].append(v)
    lines = [f"# MFMA and VALU utilisation per launch, workload {args.workload}", "",
             f"command: {args.command}", "",
             "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs); VALUBusy = "
             "SQ_ACTIVE_INST_VALU / (CUs x GRBM_GUI_ACTIVE) (rocprofv3's derived counters, percent of "
             "the dispatch's active time); instruction counts are per launch, all waves; launches "
             "labelled by their position in the step.", "",
             "| layer | entry point | kernel | launches | MFMA busy % | VALU busy % | MFMA instr | VALU instr | "
             "VALU per MFMA |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (layer, api, _), c in acc.items():
        mean = {k: (sum(c[k]) / len(c[k]) if c[k] else 0.0) for k in UTIL_COUNTERS}
        nm, nv = mean["SQ_INSTS_MFMA"], mean["SQ_INSTS_VALU"]
        ratio = f"{nv / nm:.1f}" if nm else "-"
        lines.append(f"| {layer} | {api} | `{short(c['kernel'])}` | {len(c['MfmaUtil'])} | "
                     f"{mean['MfmaUtil']:.1f} | {mean['VALUBusy']:.1f} | {nm:.0f} | {nv:.0f} | {ratio} |")
    write_out(f"util_{args.workload}.md", "\n".join(lines) + "\n")
    print("\n".join(lines))


def trace(args, pattern):
    rows = list(csv.DictReader(open(args.trace)))
    key = "Kernel_Name"
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    lab = label(library_dispatches(rows, key), pattern)
    per = collections.OrderedDict()
    for (l, rs) in lab:
        per.setdefault(l, {"kernel": rs[-1][key], "us": []})["us"].append(
            sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs) / 1e3)
    lines = [f"# Kernel trace, workload {args.workload}", "",
             "Command (run from the repository root on one MI355X):", "", "```", args.command, "```", "",
             f"Every library dispatch, labelled by its position in the step. A launch ran once per step: "
             f"in the untimed pre-warm steps (150 ms of them), the warm-up steps and the {args.steps} timed "
             "steps; 'timed' averages the last of them, the steps whose HIP events bench.py reports.", "",
             "| layer | entry point | kernel | dispatches | avg us (all) | avg us (timed) | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    for (layer, api, _), v in per.items():
        us = v["us"]
        last = us[-args.steps:]
        lines.append(f"| {layer} | {api} | `{short(v['kernel'])}` | {len(us)} | {sum(us) / len(us):.2f} | "
                     f"{sum(last) / len(last):.2f} | {min(us):.2f} | {max(us):.2f} |")
    if args.stats:
        lines += ["", "rocprofv3's own `--stats` table (by kernel name; instantiations shared by several "
                  "layers are averaged together there):", "",
                  "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
        for r in csv.DictReader(open(args.stats)):
            lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f} |")
    if args.bench_line:
        b = json.loads(open(args.bench_line).read().strip().splitlines()[-1])
        lines += ["", "The same run's bench.py line (HIP events around every launch on the launch stream; "
                  "events add a few us to short kernels):", "", "| launch | avg us (events) | median us |",
                  "|---|---|---|"]
        for k, v in b["kernels"].items():
            lines.append(f"| {k} | {v['avg_us']} | {v['median_us']} |")
        lines += ["", f"value {b['value']} {b['unit']}, {b['ms_per_step']} ms per step; roofline: "
                  f"{json.dumps(b['roofline'])}"]
    write_out(f"trace_{args.workload}_step.md", "\n".join(lines) + "\n")
    print("\n".join(lines))


def write_out(name, text):
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write(text)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", help="counter_collection.csv of the FETCH_SIZE pass")
    ap.add_argument("--write", help="counter_collection.csv of the WRITE_SIZE pass")
    ap.add_argument("--calib-mib", type=int)
    ap.add_argument("--util", help="counter_collection.csv of the MfmaUtil / VALUBusy pass")
    ap.add_argument("--trace", help="kernel_trace.csv of the --kernel-trace pass")
    ap.add_argument("--stats", help="kernel_stats.csv of the same pass")
    ap.add_argument("--bench-line", help="the JSON line bench.py printed in the traced run")
    ap.add_argument("--steps", type=int, default=100, help="timed steps of the traced run")
    ap.add_argument("--command", default="", help="the profiled command, recorded verbatim")
    args = ap.parse_args()
    import sys
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    pattern = step_pattern(args.workload)
    if args.util:
        util(args, pattern)
    elif args.trace:
        trace(args, pattern)
    elif args.fetch and args.write and args.calib_mib:
        traffic(args, pattern)
    else:
        raise SystemExit("give --fetch, --write and --calib-mib, or --util, or --trace")


if __name__ == "__main__":
    main()
