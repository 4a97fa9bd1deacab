#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 + low-rank linear layers and the AWQ W4A16
GEMV on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input.
The default workload is one DiT block's linear stream at 4096 tokens, hidden
3072: for each of QKV (3072 -> 9216), out-projection (3072 -> 3072), MLP-up
(3072 -> 12288, GELU) and MLP-down (12288 -> 3072), all W4A4 INT4 group 64
rank 32, the fused quantizer (svdq_quantize_act: smoothing + low-rank down +
4-bit activation codes) then the fused GEMM (svdq_gemm_w4a4: 4-bit GEMM +
low-rank up + scales + bias [+ GELU]); then the AWQ W4A16 modulation GEMV
(M 1, K 3072, N 18432, group 64). `--workload` selects a single layer or the
MLP pair / fused chain instead. Inputs are resident in HBM before the timed
region; R sets of inputs and outputs rotate so the working set (> 600 MB)
cannot live in the 256 MB Infinity Cache.

Prints ONE JSON line. `value` is the stream's effective throughput
sum(2 M N K) / step time in TOPS (the quantizers' and the GEMV's time is
inside the step). The timed steps are eager launches with HIP events recorded
on the launch stream around every launch, which give the per-launch
durations (mean, median, p10, p90 over the steps); --graph times HIP graph
replays instead (one graph per rotating input set, captured after the warm-up
and checked bit for bit against an eager step), with the per-launch durations
from an eager pass. The low-rank overhead t(rank r) / t(rank 0) - 1 is measured by a
second timed pass with the low-rank branch off. The shader clock is measured
on the GPU just before and just after the timed steps (cycles against the
real-time counter), and amdsmi's reported clock is sampled during them.

Options: --gpus N (only 1: one GPU), --steps K (default 100), --warmup W
(default 20), --workload NAME, --graph, --no-cpu-baseline, --no-lowrank-overhead,
--warm (no buffer rotation), --rank R, --prewarm-ms T (untimed steps for T ms
before the warm-up steps, default 150: after idle the clocks need tens of ms
of load to settle), --calib-copy-mib N (a plain fill and add of N MiB after
the timed region: the reference kernels for scaling HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import threading
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
             "nvfp4_g16": "NVFP4 operands dequantized exactly to fp16 (bf16 inputs and outputs, the pages' "
                          "compute dtype): against the 2.5 PFLOP/s fp16 peak"}
MFMA_DTYPE = {"int4_g64": "int8", "fp4_b32": "fp4", "nvfp4_g16": "f16"}
SCALE_BYTES_PER_ROW = {"int4_g64": lambda K: (K // 64) * 2, "fp4_b32": lambda K: K // 32,
                       "nvfp4_g16": lambda K: K // 16}
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 600 << 20

# workloads of several layers, in stream order; CHAINS names the layers whose
# output feeds the next layer through the fused MLP chain (the next layer's
# quantizer runs in their epilogue)
BLOCK_INT4 = ("qkv", "attn_out", "mlp_up_int4", "mlp_down")
BLOCK_FP4 = ("qkv", "attn_out", "mlp_up", "mlp_down")   # MLP-up in FP4 E2M1, as its own workload has it
WORKLOADS = {
    "block": BLOCK_INT4,
    "block_chain": BLOCK_INT4,
    "block_fp4": BLOCK_FP4,
    "block_fp4_chain": BLOCK_FP4,
    "mlp_pair": ("mlp_up_int4", "mlp_down"),
    "mlp_chain": ("mlp_up_int4", "mlp_down"),
    "mlp_pair_fp4": ("mlp_up", "mlp_down"),
    "mlp_chain_fp4": ("mlp_up", "mlp_down"),
}
CHAINS = {"block_chain": ("mlp_up_int4",), "block_fp4_chain": ("mlp_up",), "mlp_chain": ("mlp_up_int4",),
          "mlp_chain_fp4": ("mlp_up",)}
SINGLE = ("qkv", "qkv_normrope", "mlp_up", "mlp_up_nvfp4", "mlp_down", "mlp_down_m1024", "attn_out",
          "mlp_up_int4")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="block", choices=list(WORKLOADS) + list(SINGLE))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lowrank-overhead", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP graph replays: each rotating input set's step captured "
                         "once (checked bit for bit against an eager step) and replayed (default: eager "
                         "launches; the two measured within 0.1 %% of each other on the block stream)")
    ap.add_argument("--warm", action="store_true", help="no buffer rotation (cache-warm)")
    ap.add_argument("--rank", type=int, default=None, help="override the low-rank width")
    ap.add_argument("--prewarm-ms", type=float, default=150.0,
                    help="untimed steps for this long before the warm-up steps: the GPU's clocks "
                         "take tens of ms of sustained load to settle after idle")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device fill and add of this many MiB "
                         "(the reference kernels for scaling HBM byte counters)")
    return ap.parse_args(argv)


def layer_bytes(cfg, r):
    """Algorithmic HBM bytes of the quantizer and of the GEMM of one layer."""
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


def stored_traffic(workload, layer=None):
    """HBM bytes per launch of a GEMM from committed rocprofv3 --pmc counters,
    only if the kernel's source file is unchanged since they were taken. A
    record holds one GEMM (top-level fields) or, for a stream of layers, one
    entry per layer under "layers"."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        if layer is not None and "layers" in d:
            d = d["layers"][layer]
        if d.get("source_sha") != kernel_source_hash(d["source"]):
            return None
    except (OSError, ValueError, KeyError, TypeError):
        return None
    return d.get("hbm_bytes_per_launch")


def splitk_bytes(cfg):
    """Workspace of the split-K GEMM for this layer (0: it runs unsplit): INT4
    layers with too few 128 x 128 output tiles to fill the GPU."""
    if cfg.fmt != "int4_g64" or cfg.epilogue not in ("none", "gelu_tanh"):
        return 0
    import bit_diffusion_transformer_act_amd as P
    return P.svdq_gemm_w4a4_splitk_workspace(cfg.M, cfg.N, cfg.K, cfg.fmt)


def gemm_name(cfg):
    if cfg.fmt == "nvfp4_g16":
        return "svdq_gemm_nvfp4"
    if cfg.epilogue == "qkv_norm_rope":
        return "svdq_gemm_w4a4_qkv"
    return "svdq_gemm_w4a4_splitk" if splitk_bytes(cfg) else "svdq_gemm_w4a4"


class ClockSampler:
    """The graphics clock that amdsmi reports (amdsmi_get_clock_info), sampled
    on a host thread every `period` seconds between start() and stop(). On the
    MI355X boxes measured this reading does not follow the shader clock (it
    read 157 to 1719 MHz while svdq_clock_probe measured 2.38 to 2.43 GHz on
    the CUs over the same steps), so it is recorded only as the driver's own
    report; the clock of the run is the one measured on the GPU."""

    def __init__(self, pci_bus=None, period=0.005):
        self.period, self.samples, self.err, self.h, self.max_gfx = period, [], None, None, None
        try:
            import amdsmi
            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            h = handles[0]
            if pci_bus is not None and len(handles) > 1:
                for c in handles:
                    if int(amdsmi.amdsmi_get_gpu_device_bdf(c).split(":")[1], 16) == pci_bus:
                        h = c
            self.h = h
            self.max_gfx = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("max_clk")
        except Exception as e:  # no amdsmi, no permission: report why
            self.err = f"{type(e).__name__}: {e}"
        self._stop = threading.Event()
        self._t = None

    def _run(self):
        a = self.amdsmi
        while not self._stop.is_set():
            try:
                self.samples.append(float(a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.GFX)["clk"]))
            except Exception as e:
                self.err = f"{type(e).__name__}: {e}"
                return
            time.sleep(self.period)

    def start(self):
        if self.h is not None:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()

    def stop(self):
        if self._t is not None:
            self._stop.set()
            self._t.join()

    def summary(self):
        if not self.samples:
            return {"amdsmi_error": self.err or "no samples"}
        import numpy as np
        g = np.array(self.samples, float)
        return {"amdsmi_reported_gfx_mhz_median": float(np.median(g)), "amdsmi_samples": len(g),
                "gfx_mhz_limit": self.max_gfx}


def probe_clock(P):
    """Median over ~one workgroup per CU of the shader clock (MHz) measured on
    the GPU over 2 ms: shader cycles against the real-time counter."""
    import numpy as np
    return round(float(np.median(P.svdq_clock_probe(0, workgroups=256, ticks=200_000))), 1)


def main(argv=None):
    args = parse(argv)
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

    chained = CHAINS.get(args.workload, ())
    names = list(WORKLOADS.get(args.workload, (args.workload,)))
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

    per_set = gemv_bytes(gcfg) + sum(sum(layer_bytes(cfg, r)) for cfg, r, _ in host_sets)
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
            if splitk_bytes(cfg):
                L["splitk_ws"] = torch.empty((splitk_bytes(cfg),), dtype=torch.uint8, device=dev)
            if cfg.epilogue == "qkv_norm_rope":
                e = synth.qkv_epilogue_inputs(cfg.M, seed=0)
                L["qk_norm_w"], L["rope"], L["eps"] = t(e["qk_norm_w"]), t(e["rope"]), e["eps"]
            layers.append(L)
        for li, L in enumerate(layers):
            if L["cfg"].name in chained:
                # the fused chain writes the next layer's codes, scales and lora_act
                # directly; its fp32 partials live in a caller-owned workspace
                wsb = P.lib().svdq_gemm_w4a4_mlp_workspace(L["cfg"].M, L["cfg"].N, layers[li + 1]["r"])
                L["workspace"] = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev)
        G = {"x": t(gp["x"]), "codes": t(gp["codes"]), "scales": t(gp["scales"]),
             "zeros": t(gp["zeros"]), "y": torch.empty((1, gcfg.N), dtype=torch.float16, device=dev)}
        sets.append((layers, G))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    # ---- the launches of one step, in order: (label, kind, cfg, rank, fn(layers, G, lowrank))
    def quant(L, lr):
        cfg = L["cfg"]
        ld, la = (L["lora_down"], L["lora_act"]) if lr else (None, None)
        if cfg.fmt == "nvfp4_g16":
            P.svdq_quantize_act_nvfp4(L["X"], L["smooth_inv"], ld, L["act_gscale"], L["codes"], L["scales"], la)
        else:
            P.svdq_quantize_act(L["X"], L["smooth_inv"], ld, cfg.fmt, L["codes"], L["scales"], la)

    def gemm(L, lr):
        cfg = L["cfg"]
        la, lu = (L["lora_act"], L["lora_up"]) if lr else (None, None)
        h = IO_DTYPE[cfg.fmt]
        if cfg.fmt == "nvfp4_g16":
            P.svdq_gemm_nvfp4(L["codes"], L["scales"], la, L["w_codes"], L["w_scales"], lu, L["bias"],
                              L["alpha"], cfg.epilogue, out=L["Y"], dtype=h)
        elif cfg.epilogue == "qkv_norm_rope":
            P.svdq_gemm_w4a4_qkv(L["codes"], L["scales"], la, L["w_codes"], L["w_scales"], lu, L["bias"],
                                 L["qk_norm_w"], L["rope"], L["eps"], out=L["Y"], dtype=h)
        elif "splitk_ws" in L:
            P.svdq_gemm_w4a4_splitk(L["codes"], L["scales"], la, L["w_codes"], L["w_scales"], lu, L["bias"],
                                    cfg.fmt, cfg.epilogue, out=L["Y"], dtype=h, workspace=L["splitk_ws"])
        else:
            P.svdq_gemm_w4a4(L["codes"], L["scales"], la, L["w_codes"], L["w_scales"], lu, L["bias"],
                             cfg.fmt, cfg.epilogue, out=L["Y"], dtype=h)

    def fused_chain(Lu, Ld, lr):
        la, lu = (Lu["lora_act"], Lu["lora_up"]) if lr else (None, None)
        ld2, la2 = (Ld["lora_down"], Ld["lora_act"]) if lr else (None, None)
        P.svdq_gemm_w4a4_mlp(Lu["codes"], Lu["scales"], la, Lu["w_codes"], Lu["w_scales"], lu, Lu["bias"],
                             Ld["smooth_inv"], ld2, Lu["cfg"].fmt, Ld["codes"], Ld["scales"], la2,
                             Lu["workspace"] if lr else None, dtype=torch.float16)

    def gemv(G):
        P.awq_gemv_w4a16(G["x"], G["codes"], G["scales"], G["zeros"], out=G["y"])

    plan = []
    for li, (cfg, r, _) in enumerate(host_sets):
        if li == 0 or host_sets[li - 1][0].name not in chained:   # else the chain quantized for it
            plan.append((f"{cfg.name}.svdq_quantize_act", "quantize", cfg, r,
                         lambda Ls, G, lr, li=li: quant(Ls[li], lr)))
        if cfg.name in chained:
            plan.append((f"{cfg.name}.svdq_gemm_w4a4_mlp", "chain", cfg, r,
                         lambda Ls, G, lr, li=li: fused_chain(Ls[li], Ls[li + 1], lr)))
        else:
            plan.append((f"{cfg.name}.{gemm_name(cfg)}", "gemm", cfg, r,
                         lambda Ls, G, lr, li=li: gemm(Ls[li], lr)))
    plan.append(("gemv.awq_gemv_w4a16", "gemv", gcfg, 0, lambda Ls, G, lr: gemv(G)))
    nk = len(plan)

    def step(i, events=None, lowrank=True):
        layers, G = sets[i % nsets]
        for k, (_, _, _, _, fn) in enumerate(plan):
            if events is not None:
                events[k].record(stream)
            fn(layers, G, lowrank)
        if events is not None:
            events[nk].record(stream)

    clock = {}

    def settle(run):
        # clocks ramp for tens of ms under load after idle: untimed steps for
        # --prewarm-ms of wall time (synchronizing every 8 steps so the host
        # clock follows the GPU), then the W warm-up steps
        t_end = time.perf_counter() + args.prewarm_ms * 1e-3
        i = 0
        while time.perf_counter() < t_end:
            run(i)
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()

    def timed(lowrank, sampler=None):
        """Eager launches with HIP events around every launch: per-launch
        durations (and the eager step time)."""
        settle(lambda i: step(i, lowrank=lowrank))
        if sampler is not None:
            clock["gfx_mhz_before"] = probe_clock(P)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        if sampler is not None:
            sampler.start()
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(args.warmup + s, evs[s], lowrank=lowrank)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if sampler is not None:
            clock["gfx_mhz_after"] = probe_clock(P)
            sampler.stop()
        # launch k spans events[k] -> events[k + 1] (ms)
        durs = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(nk)] for e in evs])
        return wall * 1e3 / args.steps, durs

    def capture(lowrank):
        """One HIP graph per rotating input set holding that set's whole step
        (the same launches, on torch's capture stream); checked against an
        eager step on the same set, output for output, bit for bit."""
        graphs = []
        for i in range(nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i, lowrank=lowrank)
            graphs.append(g)
        torch.cuda.synchronize()
        layers, G = sets[0]
        outs = [L[k] for L in layers for k in ("Y", "codes", "scales") if L.get(k) is not None] + [G["y"]]
        step(0, lowrank=lowrank)
        torch.cuda.synchronize()
        ref = [o.clone() for o in outs]
        for o in outs:
            o.fill_(0)
        graphs[0].replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            if not torch.equal(o.view(torch.uint8), r.view(torch.uint8)):
                raise RuntimeError("a graph replay differs from the eager step")
        return graphs

    def timed_graph(graphs, sampler=None):
        """The steps as graph replays: the step time without per-launch events
        or per-launch host overhead."""
        settle(lambda i: graphs[i % nsets].replay())
        if sampler is not None:
            clock["gfx_mhz_before"] = probe_clock(P)
            sampler.start()
        t0 = time.perf_counter()
        for s in range(args.steps):
            graphs[(args.warmup + s) % nsets].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if sampler is not None:
            clock["gfx_mhz_after"] = probe_clock(P)
            sampler.stop()
        return wall * 1e3 / args.steps

    props = torch.cuda.get_device_properties(dev)
    sampler = ClockSampler(getattr(props, "pci_bus_id", None))
    if not args.graph:
        ms_per_step, durs = timed(True, sampler)
        ms_eager = ms_per_step
    else:
        ms_eager, durs = timed(True)
        ms_per_step = timed_graph(capture(True), sampler)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)     # writes n bytes
        torch.cuda.synchronize()
        dst = torch.add(src, 1)                                 # reads n, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    any_rank = any(r > 0 for _, _, _, r, _ in plan)
    lr_over = None
    if any_rank and not args.no_lowrank_overhead:
        ms0, durs0 = timed(False)
        if args.graph:
            ms0 = timed_graph(capture(False))
        mean0 = durs0.mean(axis=0)
        lr_over = {"step": round(ms_per_step / ms0 - 1, 4), "rank": max(r for _, _, _, r, _ in plan),
                   "ms_per_step_rank0": round(ms0, 4),
                   "per_launch": {plan[k][0]: round(float(durs[:, k].mean() / mean0[k] - 1), 4)
                                  for k in range(nk) if plan[k][1] != "gemv"},
                   "note": "t(rank r) / t(rank 0) - 1, same inputs with the low-rank branch off "
                           "(second timed pass; the step in the timed mode, per launch from events)"}

    mean_ms = durs.mean(axis=0)
    med_ms = np.median(durs, axis=0)
    p10_ms = np.percentile(durs, 10, axis=0)
    p90_ms = np.percentile(durs, 90, axis=0)

    total_ops = sum(2.0 * c.M * c.N * c.K for c in cfgs)
    value = total_ops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    gemm_ms_sum = 0.0
    dominant = None
    for k, (label, kind, cfg, r, _) in enumerate(plan):
        base = {"avg_us": round(mean_ms[k] * 1e3, 2), "median_us": round(med_ms[k] * 1e3, 2),
                "p10_us": round(p10_ms[k] * 1e3, 2), "p90_us": round(p90_ms[k] * 1e3, 2)}
        if kind in ("quantize", "gemv"):
            b = layer_bytes(cfg, r)[0] if kind == "quantize" else gemv_bytes(cfg)
            gbs = b / (mean_ms[k] * 1e-3) / 1e9
            kernels[label] = {**base, "alg_bytes": b, "GB/s": round(gbs, 1),
                              "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
            continue
        ops = 2.0 * cfg.M * cfg.N * cfg.K
        tops = ops / (mean_ms[k] * 1e-3) / 1e12
        gemm_ms_sum += mean_ms[k]
        kernels[label] = {**base, "alg_ops": ops,
                          "lowrank_ops": 2.0 * cfg.M * cfg.N * r + 2.0 * cfg.M * cfg.K * r,
                          "TOPS": round(tops, 1), "frac_peak": round(tops / PEAK_TOPS[cfg.fmt], 4),
                          "format": cfg.fmt, "epilogue": cfg.epilogue, "rank": r}
        if kind == "chain":
            kernels[label]["note"] = ("GEMM + GELU + the next layer's quantizer, then the fixed-order sum "
                                      "of the low-rank partials (two launches)")
        if dominant is None or mean_ms[k] > dominant[1]:
            dominant = (label, mean_ms[k], ops, cfg, kind)

    dlabel, dms, dops, dcfg, dkind = dominant
    achieved = dops / (dms * 1e-3) / 1e12
    multi = len(names) > 1
    roofline = {"bound": "mfma", "kernel": dlabel.split(".", 1)[1], "layer": dcfg.name,
                "achieved": round(achieved, 1), "peak": PEAK_TOPS[dcfg.fmt], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TOPS[dcfg.fmt], 4),
                "traffic": stored_traffic(args.workload, dcfg.name if multi else None),
                "ops_per_launch": dops,
                "note": PEAK_NOTE[dcfg.fmt] + "; the dominant kernel is the launch with the longest "
                        "mean event time, its algorithmic ops 2 M N K per launch"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline([(c, r, p) for c, r, p in host_sets], gcfg, gp)

    fused = (", fused chain: the MLP up-projection's epilogue quantizes for the down-projection"
             if chained else "")
    up_fmt = "FP4 E2M1 b32" if "mlp_up" in names else "INT4 g64"
    if args.workload.startswith("block"):
        wl = ("DiT block linear stream at M=4096, hidden 3072 (QKV 3072->9216, out-proj 3072->3072, "
              "MLP-up 3072->12288 GELU, MLP-down 12288->3072; W4A4 r32, "
              + ("all INT4 g64)" if up_fmt == "INT4 g64" else f"INT4 g64 except MLP-up {up_fmt})")
              + fused)
    elif args.workload in WORKLOADS:
        wl = (f"DiT MLP at M=4096 (up K3072 N12288 + GELU in {up_fmt}, down K12288 N3072 INT4 g64; r32)"
              + (fused or ", unfused"))
    else:
        c = cfgs[0]
        wl = f"SVDQ W4A4 {c.name} M={c.M} K={c.K} N={c.N} r={host_sets[0][1]} {c.fmt} epilogue={c.epilogue}"
    wl += f" + AWQ W4A16 modulation GEMV M=1 K={gcfg.K} N={gcfg.N} g{gcfg.group}"
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "+".join(sorted({MFMA_DTYPE[c.fmt] for c in cfgs})),
        "data": "synthetic",
        "config": {"workload": wl, "name": args.workload, "layers": names, "rotating_sets": nsets,
                   "cache": "warm" if args.warm else "cold (rotated > Infinity Cache)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "lowrank_overhead": lr_over,
        "launch": {"mode": "hip graph per rotating input set, replayed" if args.graph else "eager",
                   "ms_per_step_eager_with_events": round(ms_eager, 4),
                   "note": "kernels and roofline come from the eager pass (HIP events around every "
                           "launch); ms_per_step and value from the timed steps of this mode"},
        "clocks": {"source": "shader cycles (s_memtime) over the real-time counter (s_memrealtime), "
                             "2 ms on ~every CU just before and just after the timed steps; amdsmi's "
                             "reported clock sampled every 5 ms during them",
                   **clock, **sampler.summary()},
        "gemm_TOPS": round(total_ops / (gemm_ms_sum * 1e-3) / 1e12, 1),
        "gemv_GBps": kernels["gemv.awq_gemv_w4a16"]["GB/s"],
        "device": props.gcnArchName,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(layers, gcfg, gp, min_seconds=10.0, max_passes=50):
    """The oracle's run-time steps, as they stand, on the same workload: per
    layer of the stream, the quantizer (fp32 emulation) and the fp64 forward
    (group-scaled GEMM + low-rank + bias [+ GELU]) over all of the layer's
    tokens; whole passes over the stream until at least min_seconds of host
    time (a bounded sample), then the fp64 AWQ GEMV once. Scaled to TOPS over
    the passes' own 2 M N K."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    unpacked = [oracle.unpack_nibbles(p["w_codes"], signed=(cfg.fmt == "int4_g64")) for cfg, _, p in layers]
    t0 = time.perf_counter()
    passes = 0
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        for (cfg, r, p), wu in zip(layers, unpacked):
            codes_u, _, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], cfg.fmt, p.get("act_gscale"))
            la = oracle.lora_act_ref(p["X"], p["lora_down"][:r])
            oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"][:, :r], p["bias"], cfg.fmt,
                            "gelu_tanh" if cfg.epilogue == "gelu_tanh" else "none",
                            act_gscale=p.get("act_gscale"), w_gscale=p.get("w_gscale"))
        passes += 1
    t_layers = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.gemv_ref(gp["x"], gp["codes"], gp["scales"], gp["zeros"], gcfg.group)
    t_gemv = time.perf_counter() - t1
    ops = sum(2.0 * cfg.M * cfg.N * cfg.K for cfg, _, _ in layers) * passes
    names = ", ".join(cfg.name for cfg, _, _ in layers)
    return {"value": round(ops / t_layers / 1e12, 5), "unit": "TOPS", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{passes} pass(es) over all tokens of every layer ({names}): quantizer + fp64 "
                      f"forward, {t_layers:.1f} s; the fp64 AWQ GEMV once, {t_gemv * 1e3:.0f} ms "
                      f"({gemv_bytes(gcfg) / t_gemv / 1e9:.2f} GB/s)"
                      + ("; the QKV epilogue's norm and rotation are not in the sample"
                         if any(cfg.epilogue == "qkv_norm_rope" for cfg, _, _ in layers) else "")}


if __name__ == "__main__":
    main()
