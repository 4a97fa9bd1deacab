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


def test_stored_traffic_per_layer(tmp_path, monkeypatch):
    """A stream's record holds one GEMM per layer; each is used only while its
    source is unchanged."""
    csrc = tmp_path / "bit_diffusion_transformer_act_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text("// kernel as profiled\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_hash("k.hip")
    rec = {"layers": {"a": {"source": "k.hip", "source_sha": sha, "hbm_bytes_per_launch": 11},
                      "b": {"source": "k.hip", "source_sha": "0" * 16, "hbm_bytes_per_launch": 22}}}
    (tmp_path / "profiles" / "traffic_s.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("s", "a") == 11
    assert bench.stored_traffic("s", "b") is None      # taken with another source
    assert bench.stored_traffic("s", "c") is None      # no such layer


def test_default_workload_is_the_block_stream():
    """The default run is the DiT block's linear stream (QKV, out-projection,
    MLP-up, MLP-down) with at least 100 timed and 20 warm-up steps."""
    a = bench.parse([])
    assert a.workload == "block" and a.steps >= 100 and a.warmup >= 20
    assert bench.WORKLOADS["block"] == ("qkv", "attn_out", "mlp_up_int4", "mlp_down")
    cfgs = [synth.CONFIGS[n] for n in bench.WORKLOADS["block"]]
    assert [(c.K, c.N) for c in cfgs] == [(3072, 9216), (3072, 3072), (3072, 12288), (12288, 3072)]
    assert all(c.M == 4096 and c.rank == 32 and c.fmt == "int4_g64" for c in cfgs)


def test_step_pattern_labels_the_block():
    """bench_counters labels every library dispatch by its slot in the step and
    keeps a multi-dispatch launch (the quantizer's K split) together."""
    import bench_counters as bc
    pat = bc.step_pattern("block")
    assert [p[0] for p in pat] == ["qkv", "qkv", "attn_out", "attn_out", "mlp_up_int4", "mlp_up_int4",
                                   "mlp_down", "mlp_down", "gemv"]
    names = ["quantize_act_kernel<0>", "gemm_w4a4_kernel<0>"] * 4 + ["awq_gemv_kernel<0>"]
    rows = [{"Kernel_Name": "void svdq::" + n} for n in names * 3]
    lab = bc.label(rows, pat)
    assert len(lab) == 27 and [l[0] for l, _ in lab[:9]] == [p[0] for p in pat]
    # M 1024: the quantizer splits K (two dispatches, one launch), the GEMM splits
    # K (its kernel, then the reduce of the partials as a slot of its own)
    split = [{"Kernel_Name": "svdq::" + n} for n in ["quantize_act_kernel<a>", "quantize_act_kernel<b>",
                                                     "gemm_w4a4_kernel<0>", "splitk_reduce_kernel<0>",
                                                     "awq_gemv_kernel<0>"]]
    lab = bc.label(split * 2, bc.step_pattern("mlp_down_m1024"))
    assert [len(rs) for _, rs in lab] == [2, 1, 1, 1, 2, 1, 1, 1]
    assert [l[1] for l, _ in lab[:4]] == ["svdq_quantize_act", "svdq_gemm_w4a4_splitk",
                                          "svdq_gemm_w4a4_splitk.reduce", "awq_gemv_w4a16"]
    with pytest.raises(SystemExit):
        bc.label([{"Kernel_Name": "svdq::awq_gemv_kernel<0>"}], pat)


def _traffic_records():
    d = os.path.join(ROOT, "profiles")
    return sorted(f for f in os.listdir(d) if f.startswith("traffic_") and f.endswith(".json"))


@pytest.mark.parametrize("fname", _traffic_records())
def test_committed_traffic_records_are_well_formed(fname):
    """Each committed record names an existing kernel source, a 16-hex-digit hash
    and a per-launch byte count per kernel (bench.py reports the GEMM's only while
    that hash matches, else null); a stream's record does so per layer."""
    d = json.load(open(os.path.join(ROOT, "profiles", fname)))
    entries = list(d["layers"].values()) if "layers" in d else [d]
    assert any("source" in e for e in entries)
    for e in entries:
        if "source" in e:   # a layer with a GEMM (the GEMV's entry has its kernel record only)
            assert os.path.exists(os.path.join(ROOT, "bit_diffusion_transformer_act_amd", "csrc", e["source"]))
            assert len(e["source_sha"]) == 16 and int(e["source_sha"], 16) >= 0
            assert e["hbm_bytes_per_launch"] > 0
        for k in e["kernels"].values():
            # each of the three is rounded to whole bytes on its own
            assert abs(k["hbm_bytes_per_launch"] - k["hbm_read_bytes"] - k["hbm_write_bytes"]) <= 1
