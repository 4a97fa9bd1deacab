"""The torch modules on the GPU against the oracle: one SVDQLinear /
AWQLinear at a time, and the synthetic DiT block with every linear patched
to the 4-bit kernels.

Bars. A module: the layer bar (relative L2 2e-3 against the oracle's float64
layer on the module's own fp16 input). The block, in three parts, with values
flowing only from the oracle to the GPU, never back:
  - each 4-bit GPU layer on the oracle block's own input to that layer
    (rounded to the layer's 16-bit type), against the oracle's output of that
    layer: the layer bar;
  - the composition: the GPU block with every layer's output replaced by the
    oracle's output of that layer, so that only the block's arithmetic around
    the layers (modulation, LayerNorm, Q/K norm and rotation when unfused,
    attention, residuals) differs; the layer inputs it forms (16-bit on both
    sides) and its output must match the oracle block's within GLUE_TOL (the
    GPU's fp32 arithmetic and the rare last-bit rounding differences it causes);
  - free running, GPU block against oracle block from the same x, c, rope:
    4-bit activation quantization is not continuous at fp16 resolution (a
    last-bit change of a layer input moves a code by a whole step), so the
    two drift apart by as much as the oracle drifts from itself when its
    layer outputs carry relative noise of 1e-5; that drift, measured here,
    bounds the GPU's (times 2, plus 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.block
import synth
from bit_diffusion_transformer_act_amd.dit import DiTBlock
from bit_diffusion_transformer_act_amd.modules import (AWQLinear, SVDQLinear, SVDQLinearQKV,
                                                       fuse_qkv_norm_rope, quantize_model)
from oracle.block import linear as oracle_linear
from tests.dit_support import dense_params, quant_config, quantized_params, to_torch
from tests.parity import Y_TOL, assert_close, rel_l2

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GLUE_TOL = 1e-3
H16 = {"float16": torch.float16, "bfloat16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("fmt,epi", [("int4_g64", "none"), ("fp4_b32", "gelu_tanh"), ("int4_g64", "gelu_tanh")])
def test_svdq_linear_module(fmt, epi):
    cfg = synth.CONFIGS["tiny"]
    d = synth.make_layer_inputs(cfg, seed=0)
    si = oracle.smoothing_factors(d["X_cal"], d["W"], cfg.alpha)
    layer = oracle.prep_svdq_layer(d["W"], si, cfg.rank, fmt)
    m = SVDQLinear(cfg.K, cfg.N, cfg.rank, fmt, bias=True, epilogue=epi, device=DEV)
    m.load_state_dict(to_torch({"smooth_inv": si, "lora_down": layer["lora_down"], "lora_up": layer["lora_up"],
                                "w_codes": layer["w_codes"], "w_scales": layer["w_scales"], "bias": d["bias"]}, DEV))
    X = d["X"][:150]
    y = m(torch.from_numpy(X.reshape(3, 50, cfg.K)).to(DEV))
    assert tuple(y.shape) == (3, 50, cfg.N) and y.dtype == torch.float16
    ref = oracle_linear(X, {"kind": "svdq", "layer": layer, "b": d["bias"], "epilogue": epi})
    assert_close(host(y).reshape(150, cfg.N), ref)


@pytest.mark.parametrize("M", [1, 11])
def test_awq_linear_module(M):
    g = synth.GemvConfig("gemv_mod", 43, 1, 1024, 768, 64)
    x = synth.make_gemv_inputs(g, seed=8, M=M)["x"]
    W = synth.make_gemv_inputs(g, seed=8, M=1)["W"]
    b = (np.random.default_rng(3).standard_normal(g.N) * 0.5).astype(np.float16)
    a = oracle.awq_prep(W)
    m = AWQLinear(g.K, g.N, device=DEV)
    m.load_state_dict(to_torch({"w_codes": a["codes"], "scales": a["scales"], "zeros": a["zeros"], "bias": b}, DEV))
    y = m(torch.from_numpy(x).to(DEV))
    ref = oracle.gemv_ref(x, a["codes"], a["scales"], a["zeros"], bias=b)
    assert_close(host(y), ref)


def _block(fmt, fuse, D=1024, C=768, B=2, T=200, rank=32, dtype="float16"):
    w = synth.dit_block_params(D, C, seed=11)
    cal = synth.dit_block_inputs(2, 256, D, C, seed=12)
    inp = synth.dit_block_inputs(B, T, D, C, seed=13)
    P, sd = quantized_params(w, cal, fmt=fmt, rank=rank, fuse_qkv=fuse, dtype=dtype)
    blk = DiTBlock(D, C)
    quantize_model(blk, quant_config(fmt, rank, dtype), device=DEV)
    if fuse:
        assert fuse_qkv_norm_rope(blk) == ["self_attention"]
    blk.load_state_dict(to_torch(sd, DEV), strict=True)
    blk.to(DEV)
    return w, inp, P, blk


def _layers(blk):
    return {n: m for n, m in blk.named_modules() if isinstance(m, (SVDQLinear, SVDQLinearQKV, AWQLinear))}


def _run(blk, inp, forced=None):
    """The GPU block on (x, c, rope). Returns its output and, per 4-bit layer,
    the 16-bit input the block fed it (rows). With forced (name -> the
    oracle's output rows of that layer), each layer's output is replaced by
    the oracle's before the block goes on: the block's own arithmetic then
    runs on the oracle's layer values."""
    seen, hooks = {}, []

    def hook(name):
        def f(mod, args, out):
            seen[name] = host(args[0].float()).reshape(-1, args[0].shape[-1])
            if forced is None:
                return None
            like = out[0] if isinstance(out, tuple) else out
            y = torch.from_numpy(np.asarray(forced[name], np.float32)).to(DEV, like.dtype)
            if isinstance(out, tuple):
                return y.reshape(*args[0].shape[:-1], -1).split(like.shape[-1], dim=-1)
            return y.reshape(out.shape)
        return f
    for name, mod in _layers(blk).items():
        hooks.append(mod.register_forward_hook(hook(name)))
    try:
        with torch.no_grad():
            out = blk(torch.from_numpy(inp["x"]).to(DEV), torch.from_numpy(inp["c"]).to(DEV),
                      torch.from_numpy(inp["rope"]).to(DEV))
    finally:
        for h in hooks:
            h.remove()
    return host(out), seen


@pytest.mark.parametrize("fmt,fuse,dtype", [("int4_g64", True, "float16"), ("fp4_b32", False, "float16"),
                                            ("nvfp4_g16", False, "bfloat16"),     # the pages' own config
                                            ("int4_g64", True, "bfloat16")])
def test_dit_block_end_to_end(fmt, fuse, dtype, monkeypatch):
    w, inp, P, blk = _block(fmt, fuse, dtype=dtype)
    expect = {"adaLN_modulation.1", "self_attention.to_out", "mlp.0", "mlp.2"} | (
        {"self_attention.to_qkv"} if fuse else {f"self_attention.to_{p}" for p in "qkv"})
    layers = _layers(blk)
    assert set(layers) == expect
    # the oracle block, free running; cap holds each layer's input and output rows
    cap = {}
    ref = oracle.dit_block_ref(inp["x"], inp["c"], inp["rope"], P, capture=cap)
    assert set(cap) == expect

    # each 4-bit layer on the GPU, fed the oracle's own input to that layer
    for name, mod in layers.items():
        dt = P[name].get("dtype", "float16")
        xin = torch.from_numpy(np.asarray(oracle.block._r16(cap[name][0], dt), np.float32)).to(DEV, H16[dt])
        with torch.no_grad():
            y = mod(xin, torch.from_numpy(inp["rope"]).to(DEV)) if name.endswith("to_qkv") else mod(xin)
        y = torch.cat(y, -1) if isinstance(y, tuple) else y
        err = assert_close(host(y.float()), cap[name][1], Y_TOL, kind=dt, what=name)
        print(f"{fmt} {name}: rows {xin.shape[0]} rel_l2 {err:.2e}")

    # the composition: the GPU block with every layer output replaced by the
    # oracle's; the inputs it then feeds the layers, and its output, against the oracle's
    out_f, seen_f = _run(blk, inp, forced={n: cap[n][1] for n in expect})
    for name in expect:
        err = rel_l2(seen_f[name], oracle.block._r16(cap[name][0], P[name].get("dtype", "float16")))
        print(f"{fmt} input of {name}, oracle layer outputs forced: rel_l2 {err:.2e}")
        assert err <= GLUE_TOL, name
    err = rel_l2(out_f, ref)
    print(f"{fmt} {dtype} block output, oracle layer outputs forced: rel_l2 {err:.2e}")
    assert np.isfinite(out_f).all() and err <= GLUE_TOL

    # free running, against the oracle's own sensitivity
    out, _ = _run(blk, inp)
    x64 = inp["x"].astype(np.float64)
    err = rel_l2(out - x64, ref - x64)
    rng = np.random.default_rng(17)

    # up to one ulp of the layer's 16-bit type (2^-10 fp16, 2^-7 bf16, relative),
    # then its rounding: last-bit changes in a share of the outputs comparable
    # to the GPU's (whose per-layer difference is about a quarter ulp RMS)
    def noisy(xr, e, rope=None):
        dt = e.get("dtype", "float16")
        y = oracle_linear(xr, e, rope).astype(np.float64)
        eps = 2.0 ** -10 if dt == "float16" else 2.0 ** -7
        return oracle.block._r16(y * (1 + eps * rng.uniform(-1, 1, y.shape)), dt)
    monkeypatch.setattr(oracle.block, "linear", noisy)
    floor = rel_l2(oracle.dit_block_ref(inp["x"], inp["c"], inp["rope"], P) - x64, ref - x64)
    monkeypatch.undo()
    dense = oracle.dit_block_ref(inp["x"], inp["c"], inp["rope"], dense_params(w))
    qerr = rel_l2(ref - x64, dense - x64)
    print(f"{fmt} {dtype} block increment: GPU vs oracle {err:.2e}, oracle vs itself under 1-ulp noise "
          f"{floor:.2e}, 4-bit vs dense {qerr:.2e} (T={inp['x'].shape[1]})")
    assert err <= 2 * floor + 1e-3
