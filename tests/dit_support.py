"""Builds the synthetic DiT block's quantized parameters for the tests: the
dense weights come from the seeded generators, the calibration inputs of
each linear from the oracle's dense block, and the 4-bit parameters from the
oracle's offline preparation. Returns both the oracle's parameter entries and
the state dict the patched torch block loads."""
import numpy as np
import torch

import oracle

SVDQ_TARGETS = ["self_attention.to_q", "self_attention.to_k", "self_attention.to_v",
                "self_attention.to_out", "mlp.0", "mlp.2"]
AWQ_TARGETS = ["adaLN_modulation.1"]
ALPHA = 0.5


def quant_config(fmt="int4_g64", rank=32, dtype="float16"):
    prec, gs = {"int4_g64": ("int4", 64), "fp4_b32": ("mxfp4", 32), "nvfp4_g16": ("nvfp4", 16)}[fmt]
    return {"quantization_config": {
        "quant_method": "nunchaku_lite", "compute_dtype": dtype,
        "svdq_w4a4": {"precision": prec, "group_size": gs, "rank": rank, "targets": SVDQ_TARGETS},
        "awq_w4a16": {"precision": "int4", "group_size": 64, "targets": AWQ_TARGETS}}}


def dense_params(w: dict) -> dict:
    P = {}
    for name in SVDQ_TARGETS + AWQ_TARGETS:
        P[name] = {"kind": "dense", "W": w[name + ".weight"], "b": w[name + ".bias"]}
    P["self_attention.norm_q"] = w["self_attention.norm_q.weight"]
    P["self_attention.norm_k"] = w["self_attention.norm_k.weight"]
    return P


def _svdq_sd(prefix, layer, b):
    sd = {prefix + ".smooth_inv": layer["smooth_inv"], prefix + ".lora_down": layer["lora_down"],
          prefix + ".lora_up": layer["lora_up"], prefix + ".w_codes": layer["w_codes"],
          prefix + ".w_scales": layer["w_scales"], prefix + ".bias": b}
    if layer["fmt"] == "nvfp4_g16":
        sd[prefix + ".act_gscale"] = np.float32(layer["act_gscale"])
        sd[prefix + ".w_gscale"] = np.float32(layer["w_gscale"])
    return sd


def _h16(a, dtype):
    """A 16-bit parameter or input in the layer's type (bf16 values as float32)."""
    a = np.asarray(a)
    return oracle.bf16_round(a.astype(np.float32)) if dtype == "bfloat16" else a.astype(np.float16)


def _prep(W, X_cal, fmt, rank, dtype):
    si = oracle.smoothing_factors(X_cal, W, ALPHA)
    ga = oracle.nvfp4_act_global_scale(_h16(X_cal, dtype), si) if fmt == "nvfp4_g16" else None
    return oracle.prep_svdq_layer(W, si, rank, fmt, act_gscale=ga, dtype=dtype)


def quantized_params(w: dict, cal: dict, fmt="int4_g64", rank=32, fuse_qkv=True, dtype="float16"):
    """(oracle params, numpy state dict) for the block with its linears
    quantized; cal holds x, c, rope of the calibration batch; dtype is the
    layers' 16-bit compute type ("float16" or "bfloat16")."""
    cap = {}
    oracle.dit_block_ref(cal["x"], cal["c"], cal["rope"], dense_params(w), capture=cap)
    P, sd = {}, {}
    names = [n for n in SVDQ_TARGETS if not (fuse_qkv and n.split(".")[-1] in ("to_q", "to_k", "to_v"))]
    for name in names:
        W, b = w[name + ".weight"], _h16(w[name + ".bias"], dtype)
        layer = _prep(W, cap[name][0], fmt, rank, dtype)
        P[name] = {"kind": "svdq", "layer": layer, "b": b, "dtype": dtype,
                   "epilogue": "gelu_tanh" if name == "mlp.0" else "none"}
        sd.update(_svdq_sd(name, layer, b))
    nq, nk = w["self_attention.norm_q.weight"], w["self_attention.norm_k.weight"]
    if fuse_qkv:
        nq, nk = _h16(nq, dtype), _h16(nk, dtype)
        W = np.concatenate([w[f"self_attention.to_{p}.weight"] for p in "qkv"])
        b = _h16(np.concatenate([w[f"self_attention.to_{p}.bias"] for p in "qkv"]), dtype)
        layer = _prep(W, cap["self_attention.to_q"][0], fmt, rank, dtype)
        P["self_attention.to_qkv"] = {"kind": "svdq_qkv", "layer": layer, "b": b, "dtype": dtype,
                                      "qk_norm_w": np.stack([nq, nk]), "eps": 1e-6}
        sd.update(_svdq_sd("self_attention.to_qkv", layer, b))
    else:
        P["self_attention.norm_q"], P["self_attention.norm_k"] = nq, nk
    sd["self_attention.norm_q.weight"], sd["self_attention.norm_k.weight"] = nq, nk
    W, b = w["adaLN_modulation.1.weight"], _h16(w["adaLN_modulation.1.bias"], dtype)
    a = oracle.awq_prep(W)
    P["adaLN_modulation.1"] = {"kind": "awq", "awq": a, "b": b, "dtype": dtype}
    sd.update({"adaLN_modulation.1.w_codes": a["codes"], "adaLN_modulation.1.scales": a["scales"],
               "adaLN_modulation.1.zeros": a["zeros"], "adaLN_modulation.1.bias": b})
    return P, sd


def to_torch(sd: dict, device="cpu") -> dict:
    out = {}
    for k, v in sd.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k.endswith("norm_q.weight") or k.endswith("norm_k.weight"):
            t = t.to(torch.float32)
        out[k] = t.to(device)
    return out


def dense_state_dict(w: dict, dtype=torch.float64) -> dict:
    return {k: torch.from_numpy(np.asarray(v, np.float64)).to(dtype) for k, v in w.items()}
