"""The fused MLP chain (svdq_gemm_w4a4_mlp): the up-projection with GELU whose
16-bit output goes straight into the down-projection's INT4 quantizer.

Two bars. (1) It equals the unfused path on the GPU (svdq_gemm_w4a4 with
GELU, then svdq_quantize_act on its output): codes and scales bit for bit,
lora_act2 within the lora_act bar (a different fp32 summation order).
(2) Against the oracle chain (oracle.mlp_chain_ref), on every row at a small
size and on one row from every band of 64 at the DiT MLP size: U is a float
result and the oracle's differs from the GPU's in the last bit now and then,
so the 4-bit codes may differ where a value sits at a rounding edge. Fewer
than 1 in 1000 code bytes and scales may differ, a differing scale is one
fp16 ulp from the oracle's, every code dequantizes to within half a step
(plus that one-ulp slack) of the oracle's smoothed U, and lora_act2 meets the
lora_act bar. The down-projection then runs on the oracle chain's codes and
meets the layer bar against the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import LORA_TOL, Y_TOL, assert_close, band_rows, rel_l2  # noqa: F401

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def chain_inputs(M, K, N, r, r2, seed=0, fmt="int4_g64"):
    """Up-projection in storage format (INT4, or FP4 E2M1 with E8M0 block-32
    scales), and the down-projection's smoothing vector and low-rank down
    factor (fp16)."""
    cfg = synth.LayerConfig(f"chain_{M}_{K}_{N}", 70, M, K, N, r, fmt, "gelu_tanh", "normal", 0.005, 30.0)
    up = synth.random_quantized_layer(cfg, seed=seed)
    g = synth.rng_for(seed, 71, 7)
    si2 = np.exp(g.normal(0.0, 0.3, N)).astype(np.float32)
    ld2 = (g.standard_normal((r2, N)) * 0.02).astype(np.float16)
    return up, si2, ld2


def run_unfused(P, codes, scales, la, up, si2, ld2, h, fmt="int4_g64"):
    y = P.svdq_gemm_w4a4(codes, scales, la, dev(up["w_codes"]), dev(up["w_scales"]),
                         dev(up["lora_up"], h) if la is not None else None, dev(up["bias"], h), fmt,
                         "gelu_tanh", dtype=h)
    return P.svdq_quantize_act(y, dev(si2), dev(ld2, h) if ld2.shape[0] else None, "int4_g64")


def run_fused(P, codes, scales, la, up, si2, ld2, h, fmt="int4_g64"):
    return P.svdq_gemm_w4a4_mlp(codes, scales, la, dev(up["w_codes"]), dev(up["w_scales"]),
                                dev(up["lora_up"], h) if la is not None else None, dev(up["bias"], h), dev(si2),
                                dev(ld2, h) if ld2.shape[0] else None, fmt=fmt, dtype=h)


def _equals_unfused(P, M, K, N, r, r2, h, fmt, seed=0):
    up, si2, ld2 = chain_inputs(M, K, N, r, r2, seed=seed, fmt=fmt)
    X = dev(up["X"], h)
    codes, scales, la = P.svdq_quantize_act(X, dev(up["smooth_inv"]), dev(up["lora_down"][:r], h) if r else None,
                                            fmt)
    c1, s1, l1 = run_unfused(P, codes, scales, la, up, si2, ld2, h, fmt)
    c2, s2, l2 = run_fused(P, codes, scales, la, up, si2, ld2, h, fmt)
    assert np.array_equal(host(c2), host(c1))
    assert np.array_equal(host(s2).view(np.uint16), host(s1).view(np.uint16))
    if r2:
        assert l2.dtype == torch.float32
        assert_close(host(l2), host(l1), LORA_TOL)
    else:
        assert l2 is None


@pytest.mark.parametrize("M,K,N,r,r2,h", [(200, 512, 1024, 16, 16, torch.float16),
                                          (37, 256, 384, 16, 32, torch.float16),
                                          (256, 512, 512, 0, 0, torch.float16),
                                          (130, 512, 768, 32, 16, torch.bfloat16),
                                          (4096, 3072, 12288, 32, 32, torch.float16),
                                          (200, 512, 1024, 16, 48, torch.bfloat16),   # ranks past the prefetched 32
                                          (130, 128, 65536, 16, 128, torch.float16)])  # the largest N and rank
def test_chain_equals_unfused(P, M, K, N, r, r2, h):
    _equals_unfused(P, M, K, N, r, r2, h, "int4_g64")


@pytest.mark.parametrize("M,K,N,r,r2,h", [
    (4096, 3072, 12288, 32, 32, torch.float16),   # the DiT MLP: the 256 x 256 FP4 kernel
    (2000, 1024, 8192, 16, 128, torch.float16),   # 256 x 256 tiles, ragged M, the largest rank
    (2048, 512, 8192, 0, 0, torch.bfloat16),      # 256 x 256 tiles without low-rank branches
    (200, 512, 1024, 16, 16, torch.float16),      # too few tiles: the 128 x 128 FP4 path
    (130, 384, 768, 32, 48, torch.bfloat16),      # 128 x 128, ragged M, K not a multiple of 512
])
def test_fp4_chain_equals_unfused(P, M, K, N, r, r2, h):
    """The chain on an FP4 E2M1 up-projection (its GELU output quantized to the
    down-projection's INT4 in the epilogue of either FP4 kernel) equals the
    unfused FP4 GEMM followed by the quantizer."""
    _equals_unfused(P, M, K, N, r, r2, h, "fp4_b32", seed=7)


def test_chain_is_deterministic(P):
    up, si2, ld2 = chain_inputs(200, 512, 1024, 16, 32, seed=2)
    X = dev(up["X"])
    codes, scales, la = P.svdq_quantize_act(X, dev(up["smooth_inv"]), dev(up["lora_down"][:16]), "int4_g64")
    a = [host(t) for t in run_fused(P, codes, scales, la, up, si2, ld2, torch.float16)]
    b = [host(t) for t in run_fused(P, codes, scales, la, up, si2, ld2, torch.float16)]
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def _check_chain_codes(cg, sg, c2p_ref, s2_ref, U16, si2):
    """The chain's codes and scales against the oracle's: U is a float result,
    so where the GPU's U and the oracle's differ in the last bit a group's scale
    or a code may differ. Fewer than 1 in 1000 code bytes and scales may, a
    differing scale is one fp16 ulp from the oracle's, and every GPU code
    dequantizes to within half a step (plus the one-ulp slack of U) of the
    oracle's smoothed value."""
    code_diff = np.mean(cg != c2p_ref)
    sc_diff = np.mean(sg.view(np.uint16) != s2_ref.view(np.uint16))
    print(f"chain codes differing from the oracle's: bytes {code_diff:.2e}, scales {sc_diff:.2e}")
    assert code_diff < 1e-3 and sc_diff < 1e-3
    ulp_gap = np.abs(sg.view(np.uint16).astype(np.int32) - s2_ref.view(np.uint16).astype(np.int32))
    assert ulp_gap.max() <= 1
    qg = oracle.unpack_nibbles(cg, signed=True).astype(np.float64)
    sgx = np.repeat(sg.astype(np.float64), 64, axis=1)
    xhat = oracle.smooth_act(U16, si2).astype(np.float64)
    err = np.abs(qg * sgx - xhat)
    assert (err <= 0.5 * sgx + 2.0 ** -8 * sgx + 2.0 ** -9 * np.abs(xhat) + 1e-30).all()


def test_mlp_against_oracle_chain(P):
    """The whole MLP at a small size: the chain's outputs against the oracle
    chain, then the GPU down-projection on the oracle chain's codes against the
    oracle's down-projection (values flow from the oracle to the GPU only)."""
    M, K, N, N2, r, r2 = 200, 512, 1024, 384, 16, 16
    up, si2, ld2 = chain_inputs(M, K, N, r, r2, seed=3)
    cfg2 = synth.LayerConfig("chain_down", 72, M, N, N2, r2, "int4_g64", "none", "gelu_normal", 0.005, 30.0)
    down = synth.random_quantized_layer(cfg2, seed=3)
    # the oracle: quantize X, the up-projection with GELU, the chain's quantizer, the down-projection
    cu, packed, scales = oracle.quantize_act_ref(up["X"], up["smooth_inv"], "int4_g64")
    la = oracle.lora_act_ref(up["X"], up["lora_down"][:r]).astype(np.float32)
    wu = oracle.unpack_nibbles(up["w_codes"], signed=True)
    U16, c2u, c2p, s2, la2 = oracle.mlp_chain_ref(cu, scales, la, wu, up["w_scales"], up["lora_up"][:, :r],
                                                 up["bias"], "int4_g64", si2, ld2)
    w2u = oracle.unpack_nibbles(down["w_codes"], signed=True)
    la2_32 = la2.astype(np.float32)
    y_ref = oracle.gemm_ref(c2u, s2, la2_32, w2u, down["w_scales"], down["lora_up"][:, :r2], down["bias"],
                            "int4_g64")
    # the GPU: the same quantized X (bit-exact, checked), then the fused chain
    codes, sc, la_g = P.svdq_quantize_act(dev(up["X"]), dev(up["smooth_inv"]), dev(up["lora_down"][:r]), "int4_g64")
    assert np.array_equal(host(codes), packed)
    c2, sc2, l2 = P.svdq_gemm_w4a4_mlp(codes, sc, dev(la), dev(up["w_codes"]), dev(up["w_scales"]),
                                       dev(up["lora_up"][:, :r]), dev(up["bias"]), dev(si2), dev(ld2))
    assert_close(host(l2), la2, LORA_TOL, what="lora_act2")
    _check_chain_codes(host(c2), host(sc2), c2p, s2, U16, si2)
    y = P.svdq_gemm_w4a4(dev(c2p), dev(s2), dev(la2_32), dev(down["w_codes"]), dev(down["w_scales"]),
                         dev(down["lora_up"][:, :r2]), dev(down["bias"]), "int4_g64")
    assert_close(host(y), y_ref, what="down-projection")


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
def test_chain_full_size_against_oracle(P, fmt):
    """The DiT MLP up-projection (M 4096, K 3072, N 12288, rank 32; INT4, or
    FP4 E2M1 as in the MLP-up workload) through the fused chain, against the
    oracle chain on one row from every band of 64 (all 12288 columns): codes
    and scales as _check_chain_codes states, lora_act2 against the oracle's."""
    M, K, N, r, r2 = 4096, 3072, 12288, 32, 32
    up, si2, ld2 = chain_inputs(M, K, N, r, r2, seed=5, fmt=fmt)
    cu, packed, scales = oracle.quantize_act_ref(up["X"], up["smooth_inv"], fmt)
    la = oracle.lora_act_ref(up["X"], up["lora_down"][:r]).astype(np.float32)
    c2, s2, l2 = P.svdq_gemm_w4a4_mlp(dev(packed), dev(scales), dev(la), dev(up["w_codes"]), dev(up["w_scales"]),
                                      dev(up["lora_up"][:, :r]), dev(up["bias"]), dev(si2), dev(ld2), fmt=fmt)
    rows = band_rows(M, seed=14)
    wu = oracle.unpack_nibbles(up["w_codes"], signed=(fmt == "int4_g64"))
    U16, c2u_ref, c2p_ref, s2_ref, la2_ref = oracle.mlp_chain_ref(
        cu, scales, la, wu, up["w_scales"], up["lora_up"][:, :r], up["bias"], fmt, si2, ld2, rows=rows)
    _check_chain_codes(host(c2)[rows], host(s2)[rows], c2p_ref, s2_ref, U16, si2)
    assert_close(host(l2)[rows], la2_ref, LORA_TOL, what="lora_act2")
