"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph on
the capture stream) and replayed: every entry point the benchmark replays,
on small shapes, with every output preallocated. Each replay is compared bit
for bit with the eager result, three replays in a row with the program's own
eager work (other launches on the same buffers' neighbours, fills of the
outputs) and synchronizations between them. The library records no memset and
allocates nothing, so a graph holds kernel nodes only."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def layer(name, M, K, N, r, fmt, epi, seed):
    cfg = synth.LayerConfig(name, 80, M, K, N, r, fmt, epi, "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=seed)
    L = {k: dev(p[k]) for k in ("X", "smooth_inv", "w_codes", "w_scales", "lora_up", "bias")}
    L["lora_down"] = dev(p["lora_down"])
    sc = (M, K // 64) if fmt == "int4_g64" else (M, K // 32)
    L["codes"] = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    L["scales"] = torch.empty(sc, dtype=torch.float16 if fmt == "int4_g64" else torch.uint8, device=DEV)
    L["lora_act"] = torch.empty((M, r), dtype=torch.float32, device=DEV)
    L["Y"] = torch.empty((M, N), dtype=torch.float16, device=DEV)
    L["fmt"], L["epi"] = fmt, epi
    return L


def test_graph_replays_equal_eager(P):
    a = layer("graph_int4", 200, 512, 512, 16, "int4_g64", "gelu_tanh", 1)
    b = layer("graph_fp4", 300, 1024, 1024, 32, "fp4_b32", "none", 2)
    s = layer("graph_splitk", 200, 4096, 512, 16, "int4_g64", "none", 3)
    c = layer("graph_chain", 256, 512, 1024, 16, "int4_g64", "gelu_tanh", 4)
    g = np.random.default_rng(5)
    si2 = dev(np.exp(g.normal(0.0, 0.3, 1024)).astype(np.float32))
    ld2 = dev((g.standard_normal((16, 1024)) * 0.02).astype(np.float16))
    c2 = torch.empty((256, 512), dtype=torch.uint8, device=DEV)
    s2 = torch.empty((256, 16), dtype=torch.float16, device=DEV)
    la2 = torch.empty((256, 16), dtype=torch.float32, device=DEV)
    ws = torch.empty((P.lib().svdq_gemm_w4a4_mlp_workspace(256, 1024, 16),), dtype=torch.uint8, device=DEV)
    sws = torch.empty((P.svdq_gemm_w4a4_splitk_workspace(200, 512, 4096),), dtype=torch.uint8, device=DEV)
    gc = synth.GemvConfig("graph_gemv", 81, 1, 1024, 777, 64)
    gp = synth.random_awq_layer(gc, seed=6)
    gx, gq, gs_, gz = dev(gp["x"]), dev(gp["codes"]), dev(gp["scales"]), dev(gp["zeros"])
    gy = torch.empty((1, 777), dtype=torch.float16, device=DEV)

    def quant(L):
        P.svdq_quantize_act(L["X"], L["smooth_inv"], L["lora_down"], L["fmt"], L["codes"], L["scales"],
                            L["lora_act"])

    def gemm(L):
        P.svdq_gemm_w4a4(L["codes"], L["scales"], L["lora_act"], L["w_codes"], L["w_scales"], L["lora_up"],
                         L["bias"], L["fmt"], L["epi"], out=L["Y"])

    def work():
        quant(a)
        gemm(a)
        quant(b)
        gemm(b)
        quant(s)
        P.svdq_gemm_w4a4_splitk(s["codes"], s["scales"], s["lora_act"], s["w_codes"], s["w_scales"],
                                s["lora_up"], s["bias"], out=s["Y"], workspace=sws)
        quant(c)
        P.svdq_gemm_w4a4_mlp(c["codes"], c["scales"], c["lora_act"], c["w_codes"], c["w_scales"], c["lora_up"],
                             c["bias"], si2, ld2, "int4_g64", c2, s2, la2, ws)
        P.awq_gemv_w4a16(gx, gq, gs_, gz, out=gy)

    outs = [t for L in (a, b, s, c) for t in (L["codes"], L["scales"], L["lora_act"])] + \
           [a["Y"], b["Y"], s["Y"], c2, s2, la2, gy]
    work()                       # eager, also the warm-up before capture
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(0)
        gemm(b)                  # eager work between replays (rewrites b's Y, which the replay rewrites again)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), (rep, i)
