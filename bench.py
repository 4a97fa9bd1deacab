#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 + low-rank linear layer and the AWQ W4A16
GEMV on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
svdq_quantize_act (smoothing + low-rank down + 4-bit activation quantizer),
svdq_gemm_w4a4 (4-bit GEMM + low-rank up + scales + bias [+ GELU]) on the
DiT QKV projection (M=4096 tokens, K=3072, N=9216, rank 32, INT4 group 64),
then awq_gemv_w4a16 on the modulation projection (M=1, K=3072, N=18432,
group 64). Inputs are resident in HBM before the timed region; R sets of
inputs and outputs are rotated so the working set (> 512 MB) cannot live in
the 256 MB Infinity Cache.

Prints ONE JSON line (rank 0). `value` is the layer's effective throughput
2*M*N*K / step time in TOPS (the GEMV's time is inside the step).
Per-kernel durations come from HIP events recorded on the launch stream
around every launch in the timed region.

Options: --gpus N (only 1 is supported: one GPU), --steps K, --warmup W,
--workload {qkv,qkv_normrope,mlp_up,mlp_down,mlp_down_m1024,attn_out,mlp_up_int4,block},
--no-cpu-baseline, --warm (no buffer rotation), --prewarm-ms T (untimed steps
for T ms before the W warm-up steps, default 150: after idle the clocks need
tens of ms of load to settle, and a short warm-up would time the ramp).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A4+lowrank GEMM effective TOPS & % MFMA peak; W4A16 GEMV HBM GB/s"
# dense MFMA peak of the contraction each format runs on: int8 (INT4 codes),
# MXFP4 (block-scaled FP4), fp16 (NVFP4 operands dequantized exactly to fp16)
PEAK_TOPS = {"int4_g64": 5000.0, "fp4_b32": 10100.0, "nvfp4_g16": 2500.0}
PEAK_NOTE = {"int4_g64": "INT4 runs on int8 MFMA: tera-ops against the 5.0 POP/s int8 peak",
             "fp4_b32": "FP4 against the 10.1 PFLOP/s MXFP4 peak",
             "nvfp4_g16": "NVFP4 operands dequantized exactly to fp16 (bf16 inputs and outputs, the pages' compute dtype): against the 2.5 PFLOP/s fp16 peak"}
SCALE_BYTES_PER_ROW = {"int4_g64": lambda K: (K // 64) * 2, "fp4_b32": lambda K: K // 32,
                       "nvfp4_g16": lambda K: K // 16}
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 600 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qkv",
                    choices=["qkv", "qkv_normrope", "mlp_up", "mlp_up_nvfp4", "mlp_down",
                             "mlp_down_m1024", "attn_out", "mlp_up_int4", "block", "mlp_pair",
                             "mlp_chain"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="no buffer rotation (cache-warm)")
    ap.add_argument("--rank", type=int, default=None, help="override the low-rank width")
    ap.add_argument("--prewarm-ms", type=float, default=150.0,
                    help="untimed steps for this long before the warm-up steps: the GPU's clocks "
                         "take tens of ms of sustained load to settle after idle")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def layer_bytes(cfg, r):
    M, K, N = cfg.M, cfg.K, cfg.N
    sbytes = SCALE_BYTES_PER_ROW[cfg.fmt](K)
    q = M * K * 2 + K * 4 + r * K * 2 + M * K // 2 + M * sbytes + M * r * 4   # lora_act is fp32
    g = (M * K // 2 + M * sbytes + M * r * 4 + N * K // 2 + N * sbytes + N * r * 2 + N * 2
         + M * N * 2)
    return q, g


def gemv_bytes(g, M=1):
    return g.N * g.K // 2 + 2 * g.N * (g.K // g.group) * 2 + M * g.K * 2 + M * g.N * 2


def kernel_source_hash(name):
    p = os.path.join(ROOT, "bit_diffusion_transformer_act_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per launch of the GEMM from committed rocprofv3 --pmc counters,
    only if the kernel's source file is unchanged since they were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        if d.get("source_sha") != kernel_source_hash(d["source"]):
            return None
    except (OSError, ValueError, KeyError):
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X; splitting the "
              "tokens across GPUs needs no exchange and is not run here. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_diffusion_transformer_act_amd as P
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    IO_DTYPE = {"int4_g64": torch.float16, "fp4_b32": torch.float16, "nvfp4_g16": torch.bfloat16}
    if P.svdq_device_check(0) != 0:
        print("cuda:0 is not a gfx950 (MI355X) device", file=sys.stderr)
        sys.exit(3)

    chain = args.workload == "mlp_chain"
    if args.workload == "block":
        names = list(synth.BLOCK_STREAM)
    elif args.workload in ("mlp_pair", "mlp_chain"):
        names = ["mlp_up_int4", "mlp_down"]      # the DiT MLP: INT4 up-projection + GELU, INT4 down
    else:
        names = [args.workload]
    cfgs = [synth.CONFIGS[n] for n in names]
    gcfg = synth.CONFIGS["gemv"]

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- one input set (host generation once), replicated on the device
    host_sets = []
    for cfg in cfgs:
        p = synth.random_quantized_layer(cfg, seed=0)
        r = cfg.rank if args.rank is None else args.rank
        host_sets.append((cfg, r, p))
    gp = synth.random_awq_layer(gcfg, seed=0)

    per_set = 0
    for cfg, r, _ in host_sets:
        qb, gb = layer_bytes(cfg, r)
        per_set += qb + gb
    per_set += gemv_bytes(gcfg)
    nsets = 1 if args.warm else max(2, -(-ROTATE_BYTES // per_set))

    sets = []
    for _ in range(nsets):
        layers = []
        for cfg, r, p in host_sets:
            # NVFP4 runs in bf16, the compute dtype the pages pair it with; the rest in fp16
            h = IO_DTYPE[cfg.fmt]
            L = {"cfg": cfg, "r": r, "X": t(p["X"]).to(h), "smooth_inv": t(p["smooth_inv"]),
                 "lora_down": t(p["lora_down"][:r]).to(h) if r else None,
                 "w_codes": t(p["w_codes"]), "w_scales": t(p["w_scales"]),
                 "lora_up": t(np.ascontiguousarray(p["lora_up"][:, :r])).to(h) if r else None,
                 "bias": t(p["bias"]).to(h)}
            sdt = torch.float16 if cfg.fmt == "int4_g64" else torch.uint8
            scols = SCALE_BYTES_PER_ROW[cfg.fmt](cfg.K) // (2 if cfg.fmt == "int4_g64" else 1)
            if cfg.fmt == "nvfp4_g16":
                L["act_gscale"] = float(p["act_gscale"])
                L["alpha"] = float(np.float32(p["act_gscale"]) * np.float32(p["w_gscale"]))
            L["codes"] = torch.empty((cfg.M, cfg.K // 2), dtype=torch.uint8, device=dev)
            L["scales"] = torch.empty((cfg.M, scols), dtype=sdt, device=dev)
            L["lora_act"] = torch.empty((cfg.M, r), dtype=torch.float32, device=dev) if r else None
            L["Y"] = torch.empty((cfg.M, cfg.N), dtype=h, device=dev)
            if cfg.epilogue == "qkv_norm_rope":
                e = synth.qkv_epilogue_inputs(cfg.M, seed=0)
                L["qk_norm_w"], L["rope"], L["eps"] = t(e["qk_norm_w"]), t(e["rope"]), e["eps"]
            layers.append(L)
        if chain:
            # the fused chain writes the down-projection's codes, scales and lora_act
            # directly; its fp32 partials live in a caller-owned workspace
            Lu, Ld = layers
            wsb = P.lib().svdq_gemm_w4a4_mlp_workspace(Lu["cfg"].M, Lu["cfg"].N, Ld["r"])
            Lu["workspace"] = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev)
        G = {"x": t(gp["x"]), "codes": t(gp["codes"]), "scales": t(gp["scales"]),
             "zeros": t(gp["zeros"]), "y": torch.empty((1, gcfg.N), dtype=torch.float16, device=dev)}
        sets.append((layers, G))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    nk = 4 if chain else sum(2 for _ in cfgs) + 1   # timed calls per step

    def step_chain(layers, G, events):
        Lu, Ld = layers
        ev = (lambda k: events[k].record(stream)) if events is not None else (lambda k: None)
        ev(0)
        P.svdq_quantize_act(Lu["X"], Lu["smooth_inv"], Lu["lora_down"], "int4_g64",
                            Lu["codes"], Lu["scales"], Lu["lora_act"])
        ev(1)
        P.svdq_gemm_w4a4_mlp(Lu["codes"], Lu["scales"], Lu["lora_act"], Lu["w_codes"], Lu["w_scales"],
                             Lu["lora_up"], Lu["bias"], Ld["smooth_inv"], Ld["lora_down"], "int4_g64",
                             Ld["codes"], Ld["scales"], Ld["lora_act"], Lu["workspace"])
        ev(2)
        P.svdq_gemm_w4a4(Ld["codes"], Ld["scales"], Ld["lora_act"], Ld["w_codes"], Ld["w_scales"],
                         Ld["lora_up"], Ld["bias"], "int4_g64", "none", out=Ld["Y"])
        ev(3)
        P.awq_gemv_w4a16(G["x"], G["codes"], G["scales"], G["zeros"], out=G["y"])
        ev(4)

    def step(i, events=None):
        layers, G = sets[i % nsets]
        if chain:
            step_chain(layers, G, events)
            return
        j = 0
        for L in layers:
            cfg = L["cfg"]
            if events is not None:
                events[j].record(stream)
            if cfg.fmt == "nvfp4_g16":
                P.svdq_quantize_act_nvfp4(L["X"], L["smooth_inv"], L["lora_down"], L["act_gscale"],
                                          L["codes"], L["scales"], L["lora_act"])
            else:
                P.svdq_quantize_act(L["X"], L["smooth_inv"], L["lora_down"], cfg.fmt,
                                    L["codes"], L["scales"], L["lora_act"])
            if events is not None:
                events[j + 1].record(stream)
            if cfg.fmt == "nvfp4_g16":
                P.svdq_gemm_nvfp4(L["codes"], L["scales"], L["lora_act"], L["w_codes"], L["w_scales"],
                                  L["lora_up"], L["bias"], L["alpha"], cfg.epilogue, out=L["Y"])
            elif cfg.epilogue == "qkv_norm_rope":
                P.svdq_gemm_w4a4_qkv(L["codes"], L["scales"], L["lora_act"], L["w_codes"], L["w_scales"],
                                     L["lora_up"], L["bias"], L["qk_norm_w"], L["rope"], L["eps"],
                                     out=L["Y"])
            else:
                P.svdq_gemm_w4a4(L["codes"], L["scales"], L["lora_act"], L["w_codes"], L["w_scales"],
                                 L["lora_up"], L["bias"], cfg.fmt, cfg.epilogue, out=L["Y"])
            j += 2
        if events is not None:
            events[j].record(stream)
        P.awq_gemv_w4a16(G["x"], G["codes"], G["scales"], G["zeros"], out=G["y"])
        if events is not None:
            events[j + 1].record(stream)

    # clocks ramp for tens of ms under load after idle: run untimed steps for
    # --prewarm-ms of wall time (synchronizing every 8 steps so the host clock
    # follows the GPU), then the W warm-up steps
    t_end = time.perf_counter() + args.prewarm_ms * 1e-3
    i = 0
    while time.perf_counter() < t_end:
        step(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # event pairs per launch: quantize_l, gemm_l ..., gemv
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)     # writes n bytes
        torch.cuda.synchronize()
        dst = torch.add(src, 1)                                 # reads n, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    # per-launch durations (ms): launch k spans events[k] -> events[k+1]
    durs = np.zeros((args.steps, nk))
    for s in range(args.steps):
        e = evs[s]
        for k in range(nk):
            durs[s, k] = e[k].elapsed_time(e[k + 1])
    mean_ms = durs.mean(axis=0)
    med_ms = np.median(durs, axis=0)
    p10_ms = np.percentile(durs, 10, axis=0)
    p90_ms = np.percentile(durs, 90, axis=0)

    def spread(k):
        return {"p10_us": round(p10_ms[k] * 1e3, 2), "p90_us": round(p90_ms[k] * 1e3, 2)}
    ms_per_step = wall * 1e3 / args.steps

    total_ops = sum(2.0 * c.M * c.N * c.K for c in cfgs)
    value = total_ops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    gemm_ms_sum = 0.0
    dominant = None
    if chain:
        (cu, ru, _), (cd, rd, _) = host_sets
        qb, _ = layer_bytes(cu, ru)
        kernels[f"{cu.name}.svdq_quantize_act"] = {
            "avg_us": round(mean_ms[0] * 1e3, 2), "median_us": round(med_ms[0] * 1e3, 2), **spread(0),
            "alg_bytes": qb, "GB/s": round(qb / (mean_ms[0] * 1e-3) / 1e9, 1)}
        for k, (cfg, r, name) in ((1, (cu, ru, "svdq_gemm_w4a4_mlp")), (2, (cd, rd, "svdq_gemm_w4a4"))):
            ops = 2.0 * cfg.M * cfg.N * cfg.K
            tops = ops / (mean_ms[k] * 1e-3) / 1e12
            kernels[f"{cfg.name}.{name}"] = {
                "avg_us": round(mean_ms[k] * 1e3, 2), "median_us": round(med_ms[k] * 1e3, 2), **spread(k),
                "alg_ops": ops, "TOPS": round(tops, 1), "frac_peak": round(tops / PEAK_TOPS[cfg.fmt], 4),
                "format": cfg.fmt, "rank": r,
                "note": "GEMM + GELU + the next layer's quantizer, then the fixed-order sum of the "
                        "low-rank partials (two launches)" if k == 1 else "reads the chain's codes"}
            gemm_ms_sum += mean_ms[k]
            if dominant is None or mean_ms[k] > dominant[1]:
                dominant = (cfg, mean_ms[k], ops, r)
    for li, (cfg, r, _) in enumerate([] if chain else host_sets):
        qb, gb = layer_bytes(cfg, r)
        qms, gms = mean_ms[2 * li], mean_ms[2 * li + 1]
        gemm_ms_sum += gms
        ops = 2.0 * cfg.M * cfg.N * cfg.K
        kernels[f"{cfg.name}.svdq_quantize_act"] = {
            "avg_us": round(qms * 1e3, 2), "median_us": round(med_ms[2 * li] * 1e3, 2), **spread(2 * li),
            "alg_bytes": qb, "GB/s": round(qb / (qms * 1e-3) / 1e9, 1),
            "frac_hbm": round(qb / (qms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        tops = ops / (gms * 1e-3) / 1e12
        gname = gemm_name(cfg)
        kernels[f"{cfg.name}.{gname}"] = {
            "avg_us": round(gms * 1e3, 2), "median_us": round(med_ms[2 * li + 1] * 1e3, 2), **spread(2 * li + 1),
            "alg_ops": ops, "lowrank_ops": 2.0 * cfg.M * cfg.N * r + 2.0 * cfg.M * cfg.K * r,
            "TOPS": round(tops, 1), "frac_peak": round(tops / PEAK_TOPS[cfg.fmt], 4),
            "format": cfg.fmt, "epilogue": cfg.epilogue, "rank": r}
        if dominant is None or gms > dominant[1]:
            dominant = (cfg, gms, ops, r)
    gvb = gemv_bytes(gcfg)
    gvms = mean_ms[-1]
    kernels["gemv.awq_gemv_w4a16"] = {
        "avg_us": round(gvms * 1e3, 2), "median_us": round(med_ms[-1] * 1e3, 2), **spread(nk - 1),
        "alg_bytes": gvb, "GB/s": round(gvb / (gvms * 1e-3) / 1e9, 1),
        "frac_hbm": round(gvb / (gvms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    dcfg, dms, dops, dr = dominant
    achieved = dops / (dms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": gemm_name(dcfg), "workload": dcfg.name,
                "achieved": round(achieved, 1), "peak": PEAK_TOPS[dcfg.fmt], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TOPS[dcfg.fmt], 4),
                "traffic": stored_traffic(dcfg.name),
                "ops_per_launch": dops,
                "note": PEAK_NOTE[dcfg.fmt]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfgs[0], gcfg, host_sets[0][2], gp, host_sets[0][1])

    wl = ("DiT block linear stream (QKV, out-proj, MLP-up GELU, MLP-down; all W4A4 INT4 g64 r32)"
          if args.workload == "block" else
          "DiT MLP (M4096: up K3072 N12288 + GELU, down K12288 N3072; INT4 g64 r32)"
          + (", fused chain: the up-projection's epilogue quantizes for the down-projection"
             if chain else ", unfused")
          if args.workload in ("mlp_pair", "mlp_chain") else
          f"SVDQ W4A4 {cfgs[0].name} M={cfgs[0].M} K={cfgs[0].K} N={cfgs[0].N} r={host_sets[0][1]} "
          f"{cfgs[0].fmt} epilogue={cfgs[0].epilogue}")
    wl += f" + AWQ W4A16 modulation GEMV M=1 K={gcfg.K} N={gcfg.N} g{gcfg.group}"
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "+".join(sorted({MFMA_DTYPE[c.fmt] for c in cfgs})),
        "data": "synthetic",
        "config": {"workload": wl, "layers": names, "rotating_sets": nsets,
                   "cache": "warm" if args.warm else "cold (rotated > Infinity Cache)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "gemm_TOPS": round(sum(2.0 * c.M * c.N * c.K for c in cfgs) / (gemm_ms_sum * 1e-3) / 1e12, 1),
        "gemv_GBps": kernels["gemv.awq_gemv_w4a16"]["GB/s"],
        "device": torch.cuda.get_device_properties(dev).gcnArchName,
    }
    print(json.dumps(out), flush=True)


MFMA_DTYPE = {"int4_g64": "int8", "fp4_b32": "fp4", "nvfp4_g16": "f16"}


def gemm_name(cfg):
    if cfg.fmt == "nvfp4_g16":
        return "svdq_gemm_nvfp4"
    return "svdq_gemm_w4a4_qkv" if cfg.epilogue == "qkv_norm_rope" else "svdq_gemm_w4a4"


def cpu_baseline(cfg, gcfg, p, gp, r, min_seconds=10.0, max_passes=200):
    """The oracle's run-time steps, as they stand, on the same workload:
    quantizer + fp64 group-scaled GEMM + low-rank + bias over all tokens,
    repeated until at least min_seconds of host time (a bounded sample), and
    the fp64 AWQ GEMV. Scaled to TOPS over the passes' own 2*M*N*K."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    X = p["X"]
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(cfg.fmt == "int4_g64"))
    t0 = time.perf_counter()
    passes = 0
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        codes_u, _, scales = oracle.quantize_act_ref(X, p["smooth_inv"], cfg.fmt, p.get("act_gscale"))
        la = oracle.lora_act_ref(X, p["lora_down"][:r])
        oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"][:, :r], p["bias"], cfg.fmt,
                        cfg.epilogue, act_gscale=p.get("act_gscale"), w_gscale=p.get("w_gscale"))
        passes += 1
    t_layer = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.gemv_ref(gp["x"], gp["codes"], gp["scales"], gp["zeros"], gcfg.group)
    t_gemv = time.perf_counter() - t1
    ops = 2.0 * cfg.M * cfg.N * cfg.K * passes
    return {"value": round(ops / t_layer / 1e12, 5), "unit": "TOPS", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{passes} passes over all {cfg.M} tokens of the {cfg.name} layer (quantizer + "
                      f"fp64 forward), {t_layer:.1f} s; full AWQ GEMV fp64 {t_gemv * 1e3:.0f} ms "
                      f"({gemv_bytes(gcfg) / t_gemv / 1e9:.2f} GB/s)"}


if __name__ == "__main__":
    main()
