"""quantization_config parsing and the nn.Linear patching, on the CPU (no
kernel is called: a 4-bit module's forward on a CPU tensor must raise)."""
import copy
import json

import numpy as np
import pytest
import torch

import synth
from bit_diffusion_transformer_act_amd.config import (UnsupportedQuantConfig,
                                                      parse_quantization_config)
from bit_diffusion_transformer_act_amd.dit import DiTBlock, DiTStack
from bit_diffusion_transformer_act_amd.modules import (AWQLinear, SVDQLinear, SVDQLinearQKV,
                                                       fuse_qkv_norm_rope, quantize_model)
from tests.dit_support import quant_config, quantized_params, to_torch

# the block as printed on the pages (nvfp4, group 16, bfloat16 compute)
PAGES_EXAMPLE = {
    "quant_method": "nunchaku_lite",
    "compute_dtype": "bfloat16",
    "svdq_w4a4": {"precision": "nvfp4", "group_size": 16, "rank": 32,
                  "targets": ["layers.0.self_attention.to_q", "layers.0.self_attention.to_k", "..."]},
    "awq_w4a16": {"precision": "int4", "group_size": 64, "targets": ["adaLN_modulation.1", "..."]},
}


def test_pages_example_parses():
    q = parse_quantization_config({"quantization_config": PAGES_EXAMPLE})
    assert q.compute_dtype == "bfloat16"
    assert q.svdq.fmt == "nvfp4_g16" and q.svdq.rank == 32
    q = parse_quantization_config(dict(PAGES_EXAMPLE, compute_dtype="float16"))
    assert q.compute_dtype == "float16"


def test_bf16_patching_makes_bf16_buffers():
    blk = DiTBlock(256)
    cfg = dict(PAGES_EXAMPLE, svdq_w4a4=dict(PAGES_EXAMPLE["svdq_w4a4"], targets=["self_attention.*", "mlp.*"]))
    quantize_model(blk, cfg)
    m = blk.self_attention.to_q
    assert m.fmt == "nvfp4_g16" and m.io_dtype == torch.bfloat16
    assert m.lora_down.dtype == torch.bfloat16 and m.bias.dtype == torch.bfloat16
    assert blk.adaLN_modulation[1].bias.dtype == torch.bfloat16
    assert fuse_qkv_norm_rope(blk) == []      # the fused QKV epilogue is INT4 only


@pytest.mark.parametrize("prec,gs,fmt", [("int4", 64, "int4_g64"), ("mxfp4", 32, "fp4_b32"),
                                         ("nvfp4", 16, "nvfp4_g16")])
def test_supported_precisions(prec, gs, fmt):
    cfg = copy.deepcopy(dict(PAGES_EXAMPLE, compute_dtype="float16"))
    cfg["svdq_w4a4"].update(precision=prec, group_size=gs)
    q = parse_quantization_config(json.dumps({"quantization_config": cfg}))
    assert q.svdq.fmt == fmt and q.svdq.rank == 32
    assert q.svdq.targets == ("layers.0.self_attention.to_q", "layers.0.self_attention.to_k")
    assert q.awq.targets == ("adaLN_modulation.1",)
    assert q.method_for("layers.0.self_attention.to_k") == "svdq"
    assert q.method_for("adaLN_modulation.1") == "awq"
    assert q.method_for("layers.0.self_attention.to_v") is None


def test_config_errors_and_wildcards():
    base = {"quant_method": "nunchaku_lite", "compute_dtype": "float16",
            "svdq_w4a4": {"precision": "int4", "group_size": 64, "rank": 32, "targets": ["layers.*.mlp.0"]}}
    q = parse_quantization_config(base)
    assert q.method_for("layers.17.mlp.0") == "svdq" and q.awq is None
    for bad, exc in [({"quant_method": "gptq"}, ValueError),
                     ({"compute_dtype": "float32"}, ValueError),
                     ({"compute_dtype": "float8"}, ValueError),
                     ({"svdq_w4a4": {"precision": "int4", "group_size": 128, "rank": 32}}, UnsupportedQuantConfig),
                     ({"svdq_w4a4": {"precision": "nvfp4", "group_size": 32, "rank": 32}}, UnsupportedQuantConfig),
                     ({"svdq_w4a4": {"precision": "int4", "group_size": 64, "rank": 20}}, UnsupportedQuantConfig),
                     ({"svdq_w4a4": {"precision": "int4", "group_size": 64, "rank": 256}}, UnsupportedQuantConfig),
                     ({"svdq_w4a4": {"precision": "int4", "group_size": 64, "targets": "mlp.0"}}, ValueError)]:
        with pytest.raises(exc):
            parse_quantization_config(dict(base, **bad))
    with pytest.raises(UnsupportedQuantConfig):
        parse_quantization_config({"quant_method": "nunchaku_lite",
                                   "awq_w4a16": {"precision": "int4", "group_size": 32}})
    with pytest.raises(ValueError):
        parse_quantization_config({"quant_method": "nunchaku_lite"})


def test_patch_stack_by_name():
    model = DiTStack(2, 256)
    cfg = {"quant_method": "nunchaku_lite", "compute_dtype": "float16",
           "svdq_w4a4": {"precision": "int4", "group_size": 64, "rank": 16,
                         "targets": ["layers.0.self_attention.to_q", "layers.1.mlp.*"]},
           "awq_w4a16": {"precision": "int4", "group_size": 64, "targets": ["layers.*.adaLN_modulation.1"]}}
    done = quantize_model(model, cfg)
    assert sorted(done) == ["layers.0.adaLN_modulation.1", "layers.0.self_attention.to_q",
                            "layers.1.adaLN_modulation.1", "layers.1.mlp.0", "layers.1.mlp.2"]
    assert isinstance(model.layers[0].self_attention.to_q, SVDQLinear)
    assert isinstance(model.layers[0].self_attention.to_k, torch.nn.Linear)
    assert isinstance(model.layers[1].adaLN_modulation[1], AWQLinear)
    # GELU(tanh) after a patched mlp.0 moves into its epilogue
    assert model.layers[1].mlp[0].epilogue == "gelu_tanh"
    assert isinstance(model.layers[1].mlp[1], torch.nn.Identity)
    assert isinstance(model.layers[0].mlp[1], torch.nn.GELU)
    # only layer 0's to_q is quantized: no fusion there
    assert fuse_qkv_norm_rope(model) == []


def test_patch_fuse_and_load_block():
    D = 256
    w = synth.dit_block_params(D, seed=5)
    cal = synth.dit_block_inputs(2, 16, D, seed=6)
    _, sd = quantized_params(w, cal, rank=16)
    blk = DiTBlock(D)
    quantize_model(blk, quant_config(rank=16))
    assert fuse_qkv_norm_rope(blk) == ["self_attention"]
    att = blk.self_attention
    assert isinstance(att.to_qkv, SVDQLinearQKV) and att.to_qkv.out_features == 3 * D
    assert not hasattr(att, "to_q") and not hasattr(att, "norm_q")
    blk.load_state_dict(to_torch(sd), strict=True)
    assert np.array_equal(att.to_qkv.w_codes.numpy(), sd["self_attention.to_qkv.w_codes"])
    qk = np.stack([w["self_attention.norm_q.weight"], w["self_attention.norm_k.weight"]])
    assert np.array_equal(att.to_qkv.qk_norm_w.numpy().view(np.uint16), qk.view(np.uint16))
    assert np.array_equal(blk.adaLN_modulation[1].zeros.numpy(), sd["adaLN_modulation.1.zeros"])
    with pytest.raises(RuntimeError, match="HIP device"):
        blk(torch.zeros(1, 4, D, dtype=torch.float16), torch.zeros(1, D, dtype=torch.float16),
            torch.zeros(4, 64, 2))


def test_module_shape_checks():
    with pytest.raises(ValueError):
        SVDQLinear(200, 256)
    with pytest.raises(ValueError):
        SVDQLinear(256, 256, rank=24)
    with pytest.raises(ValueError):
        SVDQLinearQKV(256, fmt="fp4_b32")
    with pytest.raises(ValueError):
        AWQLinear(100, 64)
    m = SVDQLinear(256, 384, rank=32, fmt="fp4_b32")
    assert m.w_scales.dtype == torch.uint8 and tuple(m.w_scales.shape) == (384, 8)
    with pytest.raises(RuntimeError):
        m(torch.zeros(3, 256, dtype=torch.float16))
    with pytest.raises(ValueError):
        SVDQLinear(384, 256, fmt="nvfp4_g16")
    n = SVDQLinear(512, 256, rank=16, fmt="nvfp4_g16")
    assert tuple(n.w_scales.shape) == (256, 32)
    sd = n.state_dict()
    sd["act_gscale"] = torch.tensor(0.25)
    sd["w_gscale"] = torch.tensor(3.0)
    n.load_state_dict(sd)
    assert n._gs == (0.25, 3.0) and n._alpha == 0.75
    assert n.act_gscale.device.type == "cpu"
