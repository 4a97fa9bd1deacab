"""The C ABI library on the CPU: it loads, exports every symbol include/svdq.h
declares, and rejects bad arguments with the documented status before it
touches a device. No kernel is launched here (there is no GPU in this test;
the device check itself reports SVDQ_ERR_UNSUPPORTED_DEVICE).
"""
import ctypes
import os
import re
import subprocess

import pytest

import bit_diffusion_transformer_act_amd as P
from bit_diffusion_transformer_act_amd import ops
from bit_diffusion_transformer_act_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

A = 4096  # a 16-byte aligned, never dereferenced fake device address
U = 4099  # unaligned fake address


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(ops.EXPORTED_SYMBOLS)
    lib = P.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings_and_version():
    for st in (0, -1, -2, -3, -4, -5):
        assert P.svdq_status_str(st)
    assert "unknown" in P.svdq_status_str(17)
    assert P.svdq_version() == 200


def q(fmt=0, M=4, K=128, r=16, X=A, si=A, ld=A, codes=A, scales=A, la=A, dt=0):
    return P.lib().svdq_quantize_act(fmt, dt, M, K, r, X, si, ld, codes, scales, la, None)


def g(fmt=0, M=4, N=128, K=128, r=16, ac=A, sa=A, la=A, wc=A, ws=A, lu=A, b=None, epi=0, Y=A, dt=0):
    return P.lib().svdq_gemm_w4a4(fmt, dt, M, N, K, r, ac, sa, la, wc, ws, lu, b, epi, Y, None)


def v(M=1, N=64, K=128, G=64, x=A, c=A, s=A, z=A, b=None, y=A, dt=0):
    return P.lib().awq_gemv_w4a16(dt, M, N, K, G, x, c, s, z, b, y, None)


def test_dtype_argument():
    for f in (q, g, v, qn, gn):
        assert f(dt=2) == ops.SVDQ_ERR_INVALID_ARG
        assert f(dt=-1) == ops.SVDQ_ERR_INVALID_ARG
        assert f(dt=1) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE   # bf16 is accepted


def test_quantize_act_argument_errors():
    assert q(fmt=2) == ops.SVDQ_ERR_INVALID_ARG
    assert q(K=64) == ops.SVDQ_ERR_SHAPE
    assert q(K=192) == ops.SVDQ_ERR_SHAPE
    assert q(r=8) == ops.SVDQ_ERR_SHAPE
    assert q(r=144) == ops.SVDQ_ERR_SHAPE
    assert q(M=-1) == ops.SVDQ_ERR_SHAPE
    assert q(M=(1 << 23) + 1) == ops.SVDQ_ERR_SHAPE
    assert q(M=1 << 23) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE   # the largest M is accepted
    assert q(M=0, X=None, si=None, ld=None, codes=None, scales=None, la=None) == ops.SVDQ_OK
    assert q(X=None) == ops.SVDQ_ERR_INVALID_ARG
    assert q(la=None) == ops.SVDQ_ERR_INVALID_ARG
    assert q(r=0, ld=None, la=None) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert q(codes=U) == ops.SVDQ_ERR_ALIGN
    assert q(si=U) == ops.SVDQ_ERR_ALIGN
    # valid arguments reach the device check, which fails without a gfx950
    assert q() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_gemm_argument_errors():
    assert g(fmt=5) == ops.SVDQ_ERR_INVALID_ARG
    assert g(epi=3) == ops.SVDQ_ERR_INVALID_ARG
    assert g(N=192) == ops.SVDQ_ERR_SHAPE
    assert g(N=0) == ops.SVDQ_ERR_SHAPE
    assert g(K=320) == ops.SVDQ_ERR_SHAPE
    assert g(r=40) == ops.SVDQ_ERR_SHAPE
    assert g(M=(1 << 23) + 1) == ops.SVDQ_ERR_SHAPE
    assert g(N=65536 + 128) == ops.SVDQ_ERR_SHAPE
    assert g(K=65536 + 128) == ops.SVDQ_ERR_SHAPE
    assert g(M=1 << 23, N=65536, K=65536, r=128) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert g(M=0, ac=None, sa=None, la=None, wc=None, ws=None, lu=None, Y=None) == ops.SVDQ_OK
    assert g(wc=None) == ops.SVDQ_ERR_INVALID_ARG
    assert g(lu=None) == ops.SVDQ_ERR_INVALID_ARG
    assert g(r=0, la=None, lu=None) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert g(Y=U) == ops.SVDQ_ERR_ALIGN
    assert g(b=U) == ops.SVDQ_ERR_ALIGN
    assert g() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_gemv_argument_errors():
    assert v(G=32) == ops.SVDQ_ERR_SHAPE
    assert v(M=9) == ops.SVDQ_ERR_SHAPE
    assert v(K=96) == ops.SVDQ_ERR_SHAPE
    assert v(M=2, K=32768) == ops.SVDQ_ERR_SHAPE
    assert v(N=0) == ops.SVDQ_ERR_SHAPE
    assert v(N=(1 << 20) + 1) == ops.SVDQ_ERR_SHAPE
    assert v(M=8, K=4096, N=1 << 20) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE   # the limits themselves pass
    assert v(M=0, x=None, c=None, s=None, z=None, y=None) == ops.SVDQ_OK
    assert v(z=None) == ops.SVDQ_ERR_INVALID_ARG
    assert v(y=U) == ops.SVDQ_ERR_ALIGN
    assert v(b=U) == ops.SVDQ_ERR_ALIGN
    assert v() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert v(b=A) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def qn(M=4, K=256, r=16, X=A, si=A, ld=A, g=0.5, codes=A, scales=A, la=A, dt=0):
    return P.lib().svdq_quantize_act_nvfp4(dt, M, K, r, X, si, ld, ctypes.c_float(g), codes, scales, la, None)


def gn(M=4, N=128, K=256, r=16, ac=A, sa=A, la=A, wc=A, ws=A, lu=A, b=None, alpha=1.0, epi=0, Y=A, dt=0):
    return P.lib().svdq_gemm_nvfp4(dt, M, N, K, r, ac, sa, la, wc, ws, lu, b, ctypes.c_float(alpha), epi, Y,
                                   None)


def test_nvfp4_argument_errors():
    assert qn(K=128) == ops.SVDQ_ERR_SHAPE          # K % 256
    assert qn(K=384) == ops.SVDQ_ERR_SHAPE
    assert qn(r=8) == ops.SVDQ_ERR_SHAPE
    assert qn(M=(1 << 23) + 1) == ops.SVDQ_ERR_SHAPE
    assert qn(g=0.0) == ops.SVDQ_ERR_INVALID_ARG
    assert qn(g=-1.0) == ops.SVDQ_ERR_INVALID_ARG
    assert qn(g=float("inf")) == ops.SVDQ_ERR_INVALID_ARG
    assert qn(g=1e38) == ops.SVDQ_ERR_INVALID_ARG     # 6 g overflows fp32
    assert qn(M=0, X=None, si=None, ld=None, codes=None, scales=None, la=None) == ops.SVDQ_OK
    assert qn(X=None) == ops.SVDQ_ERR_INVALID_ARG
    assert qn(scales=U) == ops.SVDQ_ERR_ALIGN
    assert qn() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert gn(epi=2) == ops.SVDQ_ERR_INVALID_ARG
    assert gn(alpha=float("nan")) == ops.SVDQ_ERR_INVALID_ARG
    assert gn(K=128) == ops.SVDQ_ERR_SHAPE
    assert gn(N=64) == ops.SVDQ_ERR_SHAPE
    assert gn(N=200) == ops.SVDQ_ERR_SHAPE
    assert gn(r=144) == ops.SVDQ_ERR_SHAPE
    assert gn(M=(1 << 23) + 1) == ops.SVDQ_ERR_SHAPE
    assert gn(N=65536 + 128) == ops.SVDQ_ERR_SHAPE
    assert gn(K=65536 + 256) == ops.SVDQ_ERR_SHAPE
    assert gn(M=0, ac=None, sa=None, la=None, wc=None, ws=None, lu=None, Y=None) == ops.SVDQ_OK
    assert gn(ws=None) == ops.SVDQ_ERR_INVALID_ARG
    assert gn(lu=None) == ops.SVDQ_ERR_INVALID_ARG
    assert gn(Y=U) == ops.SVDQ_ERR_ALIGN
    assert gn(b=U) == ops.SVDQ_ERR_ALIGN
    assert gn() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def gm(M=4, N=128, K=128, r=16, r2=16, ac=A, sa=A, la=A, wc=A, ws=A, lu=A, b=None, si2=A, ld2=A,
       c2=A, s2=A, la2=A, wk=A, wkb=1 << 20, dt=0, fmt=0):
    return P.lib().svdq_gemm_w4a4_mlp(fmt, dt, M, N, K, r, ac, sa, la, wc, ws, lu, b, si2, ld2, r2, c2, s2, la2,
                                      wk, wkb, None)


def test_mlp_chain_argument_errors():
    assert P.lib().svdq_gemm_w4a4_mlp_workspace(4096, 12288, 32) == 96 * 4096 * 32 * 4
    assert gm(fmt=2) == ops.SVDQ_ERR_INVALID_ARG          # INT4 or FP4 up-projections only
    assert gm(fmt=1, sa=A) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert gm(dt=3) == ops.SVDQ_ERR_INVALID_ARG
    assert gm(N=192) == ops.SVDQ_ERR_SHAPE
    assert gm(r2=24) == ops.SVDQ_ERR_SHAPE
    assert gm(wkb=4 * 16 * 4 - 1) == ops.SVDQ_ERR_SHAPE   # one tile x 4 rows x 16 ranks x 4 bytes needed
    assert gm(wk=None) == ops.SVDQ_ERR_INVALID_ARG
    assert gm(r2=0, ld2=None, la2=None, wk=None, wkb=0) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert gm(c2=U) == ops.SVDQ_ERR_ALIGN
    assert gm(M=0, ac=None, sa=None, la=None, wc=None, ws=None, lu=None, si2=None, ld2=None, c2=None,
              s2=None, la2=None, wk=None) == ops.SVDQ_OK
    assert gm() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def gz(M=4, N=128, K=128, r=16, r2=16, ac=A, sa=A, la=A, wc=A, ws=A, lu=A, b=None, si2=A, ld2=A,
       c2=A, s2=A, la2=A, dt=0, fmt=0):
    return P.lib().svdq_gemm_w4a4_mlp_noalloc(fmt, dt, M, N, K, r, ac, sa, la, wc, ws, lu, b, si2, ld2, r2, c2, s2,
                                              la2, None)


def test_mlp_chain_noalloc_argument_errors():
    """The allocation-free chain: the chain's checks, no workspace, and the
    64 MiB limit of the library's device scratch (partials M (N/128) r2 fp32)."""
    assert gz(fmt=2) == ops.SVDQ_ERR_INVALID_ARG
    assert gz(N=192) == ops.SVDQ_ERR_SHAPE
    assert gz(c2=U) == ops.SVDQ_ERR_ALIGN
    assert gz(la2=None) == ops.SVDQ_ERR_INVALID_ARG
    assert gz() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    # the DiT MLP (M 4096, N 12288, rank 32: 50331648 bytes) fits; exactly 64 MiB fits; more does not
    assert gz(M=4096, N=12288, K=3072, r2=32) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert gz(M=4096, N=16384, K=3072, r2=32) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert gz(M=4096, N=16384, K=3072, r2=48) == ops.SVDQ_ERR_SHAPE
    assert gz(M=8192, N=12288, K=3072, r2=32) == ops.SVDQ_ERR_SHAPE
    assert gz(M=8192, N=12288, K=3072, r2=0, ld2=None, la2=None) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert ops.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_splitk_workspace_and_argument_errors():
    """The split rule through its workspace size: K is split only for INT4 and
    fewer than 256 output tiles of 128 x 128, into the largest power of two S
    with S tiles' workgroups within 768 and at least 8 K steps per split."""
    ws = P.lib().svdq_gemm_w4a4_splitk_workspace
    assert ws(0, 1024, 3072, 12288) == 4 * 1024 * 3072 * 4     # 192 tiles, 96 steps: S 4
    assert ws(0, 256, 3072, 12288) == 8 * 256 * 3072 * 4       # 48 tiles: S 8 (12 steps each)
    assert ws(0, 200, 512, 4096) == 4 * 200 * 512 * 4          # 8 tiles, 32 steps: S 4 (8 each)
    assert ws(0, 64, 1024, 2048) == 2 * 64 * 1024 * 4          # 16 steps: S 2
    assert ws(0, 2048, 3072, 12288) == 0                        # 384 tiles: no split
    assert ws(0, 1024, 3072, 1024) == 0                         # 8 steps: too short to split
    assert ws(1, 1024, 3072, 12288) == 0                        # FP4 does not split
    assert ws(0, 1024, 3000, 12288) == 0 and ws(0, 0, 3072, 12288) == 0 and ws(2, 1024, 3072, 12288) == 0

    def sk(fmt=0, M=4, N=128, K=128, r=16, epi=0, w=A, n=1 << 20, Y=A, dt=0):
        return P.lib().svdq_gemm_w4a4_splitk(fmt, dt, M, N, K, r, A, A, A, A, A, A, None, epi, Y, w, n, None)
    assert sk(fmt=2) == ops.SVDQ_ERR_INVALID_ARG
    assert sk(epi=2) == ops.SVDQ_ERR_INVALID_ARG
    assert sk(N=192) == ops.SVDQ_ERR_SHAPE
    assert sk(w=U) == ops.SVDQ_ERR_ALIGN
    assert sk(Y=None) == ops.SVDQ_ERR_INVALID_ARG
    assert sk(M=0, Y=None) == ops.SVDQ_OK
    assert sk() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert sk(w=None, n=0) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE   # no workspace: the unsplit kernel


def test_clock_probe_argument_errors():
    khz = ctypes.c_int(0)
    probe = lambda wg=4, ticks=1000, out=A, k=ctypes.byref(khz): P.lib().svdq_clock_probe(wg, ticks, out, k, None)
    assert probe(wg=0) == ops.SVDQ_ERR_SHAPE
    assert probe(wg=4097) == ops.SVDQ_ERR_SHAPE
    assert probe(ticks=0) == ops.SVDQ_ERR_SHAPE
    assert probe(ticks=100_000_001) == ops.SVDQ_ERR_SHAPE
    assert probe(out=None) == ops.SVDQ_ERR_INVALID_ARG
    assert probe(k=None) == ops.SVDQ_ERR_INVALID_ARG
    assert probe(out=U) == ops.SVDQ_ERR_ALIGN
    assert probe() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_device_check_without_gpu():
    assert P.svdq_device_check(0) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert P.svdq_device_check(-1) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_forced_arch_override(monkeypatch):
    monkeypatch.setenv("SVDQ_FORCE_ARCH", "gfx942")
    assert q() == ops.SVDQ_ERR_UNSUPPORTED_DEVICE
    assert P.svdq_device_check(0) == ops.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_binding_rejects_cpu_tensors():
    import torch
    X = torch.zeros((4, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        P.svdq_quantize_act(X, torch.ones(128), None)


def test_product_path_does_not_import_the_oracle():
    pkg_dir = os.path.join(ROOT, "bit_diffusion_transformer_act_amd")
    for dirpath, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle/" not in text, f
