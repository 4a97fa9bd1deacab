#!/usr/bin/env python3
"""HBM traffic per launch from rocprofv3 counter passes, for bench.py's
roofline `traffic` field.

Input: the counter_collection.csv of one `rocprofv3 --pmc FETCH_SIZE` pass and
one `--pmc WRITE_SIZE` pass over the same `bench.py --calib-copy-mib N` command.
The calibration kernels that command runs after its timed region (a torch fill
that writes N MiB, then a torch add that reads N MiB and writes N MiB) give the
counter-to-bytes factors: fetch factor = add's FETCH_SIZE / N MiB, write factor
= fill's WRITE_SIZE / N MiB. Each library kernel's average counters are divided
by those factors.

Writes profiles/traffic_<workload>.json (read by bench.py, which reports the
figure only while the GEMM source hash recorded here still matches) and prints
a short text summary.

With --util instead: the counter_collection.csv of one
`rocprofv3 --pmc MfmaUtil VALUBusy SQ_INSTS_VALU SQ_INSTS_MFMA` pass, summarised
per library kernel into profiles/util_<workload>.md (MFMA busy %, VALU busy %,
instruction counts per launch).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.abspath(__file__))
# entry point -> [(kernel-name substring, source file)]; the first that matches wins
KERNELS = {"svdq_gemm_w4a4": [("gemm_fp4_big_kernel", "gemm_fp4.hip"),
                              ("gemm_w4a4_kernel", "gemm_w4a4.hip")],
           "svdq_gemm_nvfp4": [("gemm_nvfp4_kernel", "gemm_nvfp4.hip")],
           "svdq_quantize_act": [("quantize_act_kernel", "quantize_act.hip")],
           "awq_gemv_w4a16": [("awq_gemv", "awq_gemv.hip")]}


def source_sha(fname: str) -> str:
    p = os.path.join(ROOT, "bit_diffusion_transformer_act_amd", "csrc", fname)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def per_dispatch(path: str, counter: str):
    """[(kernel name, value KiB)] in dispatch order."""
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    acc = collections.OrderedDict()
    for r in rows:
        key = int(r["Dispatch_Id"])
        name, v = acc.get(key, (r["Kernel_Name"], 0.0))
        acc[key] = (name, v + float(r["Counter_Value"]))
    return list(acc.values())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", help="counter_collection.csv of the FETCH_SIZE pass")
    ap.add_argument("--write", help="counter_collection.csv of the WRITE_SIZE pass")
    ap.add_argument("--calib-mib", type=int)
    ap.add_argument("--util", help="counter_collection.csv of the MfmaUtil / VALUBusy pass")
    ap.add_argument("--command", default="", help="the profiled command, recorded verbatim")
    args = ap.parse_args()
    if args.util:
        util(args)
        return
    if not (args.fetch and args.write and args.calib_mib):
        raise SystemExit("--fetch, --write and --calib-mib are required (or --util)")

    fetch = per_dispatch(args.fetch, "FETCH_SIZE")
    write = per_dispatch(args.write, "WRITE_SIZE")
    calib_kib = args.calib_mib * 1024.0

    elem_f = [v for n, v in fetch if "elementwise" in n]
    elem_w = [v for n, v in write if "elementwise" in n]
    if len(elem_f) < 2 or len(elem_w) < 2:
        raise SystemExit("calibration kernels not found (run bench.py with --calib-copy-mib)")
    # the add reads N MiB (largest fetch); the fill and the add each write N MiB
    f_factor = max(elem_f) / calib_kib
    w_factor = sorted(elem_w)[-1] / calib_kib

    out = {"workload": args.workload, "calib_mib": args.calib_mib,
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "command": args.command, "kernels": {}}
    lines = [f"# HBM traffic per launch, workload {args.workload}",
             f"command: {args.command}",
             f"calibration: fetch factor {f_factor:.4f}, write factor {w_factor:.4f} "
             f"(torch add / fill of {args.calib_mib} MiB)", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | total MB |",
             "|---|---|---|---|---|---|"]
    for api, cands in KERNELS.items():
        for sub, src in cands:
            fv = [v for n, v in fetch if sub in n]
            wv = [v for n, v in write if sub in n]
            if fv and wv:
                break
        else:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        rd, wr = fk / f_factor * 1024, wk / w_factor * 1024
        out["kernels"][api] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                               "hbm_read_bytes": round(rd), "hbm_write_bytes": round(wr),
                               "hbm_bytes_per_launch": round(rd + wr),
                               "launches": len(fv), "kernel": sub, "source": src,
                               "source_sha": source_sha(src)}
        lines.append(f"| {api} | {fk:.0f} | {wk:.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(rd + wr) / 1e6:.1f} |")
    g = out["kernels"].get("svdq_gemm_w4a4") or out["kernels"].get("svdq_gemm_nvfp4")
    if g:
        out["source"] = g["source"]
        out["source_sha"] = g["source_sha"]
        out["hbm_bytes_per_launch"] = g["hbm_bytes_per_launch"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))


UTIL_COUNTERS = ("MfmaUtil", "VALUBusy", "SQ_INSTS_MFMA", "SQ_INSTS_VALU")


def util(args):
    """Per library kernel: the average over its launches of each counter."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(args.util)):
        if r["Counter_Name"] in UTIL_COUNTERS:
            acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# MFMA and VALU utilisation per launch, workload {args.workload}", "",
             f"command: {args.command}", "",
             "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs); VALUBusy = "
             "SQ_ACTIVE_INST_VALU / (CUs x GRBM_GUI_ACTIVE) (rocprofv3's derived counters, percent of "
             "the dispatch's active time); instruction counts are per launch, all waves.", "",
             "| kernel | launches | MFMA busy % | VALU busy % | MFMA instr | VALU instr | VALU per MFMA |",
             "|---|---|---|---|---|---|---|"]
    for name, c in acc.items():
        short = name.split("(")[0].replace("void ", "")
        if not short.startswith("svdq::"):
            continue
        mean = {k: (sum(v) / len(v) if v else 0.0) for k, v in c.items()}
        nm, nv = mean.get("SQ_INSTS_MFMA", 0.0), mean.get("SQ_INSTS_VALU", 0.0)
        ratio = f"{nv / nm:.1f}" if nm else "-"
        lines.append(f"| `{short}` | {len(c.get('MfmaUtil', []))} | {mean.get('MfmaUtil', 0.0):.1f} | "
                     f"{mean.get('VALUBusy', 0.0):.1f} | {nm:.0f} | {nv:.0f} | {ratio} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"util_{args.workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
