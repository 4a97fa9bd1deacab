"""Host logic of bench.py, on the CPU: the one-GPU guard, the algorithmic
bytes that the HBM fractions divide by, and the rule that stored traffic
counters are used only while the kernel's source is the one they were taken
with."""
import json
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_layer_bytes_qkv():
    """The DiT QKV layer (M4096 K3072 N9216 r32, INT4 g64), term by term."""
    cfg = synth.CONFIGS["qkv"]
    q, g = bench.layer_bytes(cfg, 32)
    x_read = 4096 * 3072 * 2                # fp16 activations
    smooth = 3072 * 4                       # fp32 smooth_inv, once
    lora_down = 32 * 3072 * 2               # fp16, once
    codes = 4096 * 3072 // 2                # two codes per byte
    scales = 4096 * (3072 // 64) * 2        # one fp16 scale per 64
    lora_act = 4096 * 32 * 4                # fp32
    assert q == x_read + smooth + lora_down + codes + scales + lora_act == 32_583_680
    w = 9216 * 3072 // 2 + 9216 * (3072 // 64) * 2 + 9216 * 32 * 2 + 9216 * 2
    assert g == codes + scales + lora_act + w + 4096 * 9216 * 2


def test_layer_bytes_scale_formats():
    """FP4 keeps one E8M0 byte per 32, NVFP4 one E4M3 byte per 16."""
    for name, per_row in (("mlp_up", 3072 // 32), ("mlp_up_nvfp4", 3072 // 16)):
        cfg = synth.CONFIGS[name]
        q, _ = bench.layer_bytes(cfg, 0)
        assert q == 4096 * 3072 * 2 + 3072 * 4 + 4096 * 3072 // 2 + 4096 * per_row


def test_gemv_bytes():
    g = synth.CONFIGS["gemv"]   # M1 K3072 N18432, group 64
    codes = 18432 * 3072 // 2
    scales_zeros = 2 * 18432 * (3072 // 64) * 2
    assert bench.gemv_bytes(g) == codes + scales_zeros + 3072 * 2 + 18432 * 2 == 31_893_504
    assert bench.gemv_bytes(g, M=8) == codes + scales_zeros + 8 * 3072 * 2 + 8 * 18432 * 2


def test_stored_traffic_follows_the_source(tmp_path, monkeypatch):
    csrc = tmp_path / "bit_diffusion_transformer_act_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = csrc / "k.hip"
    src.write_text("// kernel as profiled\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_hash("k.hip")
    rec = {"source": "k.hip", "source_sha": sha, "hbm_bytes_per_launch": 123456}
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("w") == 123456
    assert bench.stored_traffic("absent") is None
    src.write_text("// kernel changed since\n")
    assert bench.stored_traffic("w") is None
    (tmp_path / "profiles" / "traffic_w.json").write_text("{ not json")
    assert bench.stored_traffic("w") is None


@pytest.mark.parametrize("w", ["qkv", "mlp_up", "mlp_down", "mlp_up_nvfp4", "qkv_normrope"])
def test_committed_traffic_records_are_well_formed(w):
    """Each committed record names an existing kernel source, a 16-hex-digit hash
    and a per-launch byte count per kernel (bench.py reports the GEMM's only while
    that hash matches, else null)."""
    d = json.load(open(os.path.join(ROOT, "profiles", f"traffic_{w}.json")))
    assert os.path.exists(os.path.join(ROOT, "bit_diffusion_transformer_act_amd", "csrc", d["source"]))
    assert len(d["source_sha"]) == 16 and int(d["source_sha"], 16) >= 0
    assert d["hbm_bytes_per_launch"] > 0
    for k in d["kernels"].values():
        # each of the three is rounded to whole bytes on its own
        assert abs(k["hbm_bytes_per_launch"] - k["hbm_read_bytes"] - k["hbm_write_bytes"]) <= 1
