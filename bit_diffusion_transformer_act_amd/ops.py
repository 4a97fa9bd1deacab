"""Python binding of the C ABI in include/svdq.h (ctypes).

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), outputs are allocated with torch on the input's device, and the
call goes to the HIP library on torch's current stream. Every step of the
layer runs in the library's kernels; there is no fallback of any kind, and a
missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import LIB_PATH

INT4_G64 = 0
FP4_E2M1_B32 = 1
NVFP4_G16 = 2
# formats of svdq_quantize_act / svdq_gemm_w4a4; NVFP4 has entry points of its own
FORMATS = {"int4_g64": INT4_G64, "fp4_b32": FP4_E2M1_B32}
ALL_FORMATS = ("int4_g64", "fp4_b32", "nvfp4_g16")
EPI_NONE = 0
EPI_GELU_TANH = 1
EPILOGUES = {"none": EPI_NONE, "gelu_tanh": EPI_GELU_TANH}

# the layer's 16-bit compute type (activations, low-rank branch, biases, outputs)
DTYPES = {torch.float16: 0, torch.bfloat16: 1}

SVDQ_OK = 0
SVDQ_ERR_INVALID_ARG = -1
SVDQ_ERR_SHAPE = -2
SVDQ_ERR_ALIGN = -3
SVDQ_ERR_UNSUPPORTED_DEVICE = -4
SVDQ_ERR_HIP = -5

EXPORTED_SYMBOLS = ("svdq_device_check", "svdq_status_str", "svdq_version",
                    "svdq_quantize_act", "svdq_gemm_w4a4", "svdq_gemm_w4a4_qkv",
                    "svdq_quantize_act_nvfp4", "svdq_gemm_nvfp4", "awq_gemv_w4a16",
                    "svdq_gemm_w4a4_mlp", "svdq_gemm_w4a4_mlp_workspace", "svdq_gemm_w4a4_mlp_noalloc",
                    "svdq_clock_probe", "svdq_gemm_w4a4_splitk", "svdq_gemm_w4a4_splitk_workspace")

_lock = threading.Lock()
_handle = None


class SvdqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {svdq_status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libsvdq_mi355x.so (after torch, so both share one HIP runtime)."""
    global _handle
    with _lock:
        if _handle is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library {LIB_PATH} is not built; run "
                    "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
            h = ctypes.CDLL(LIB_PATH)
            vp, i32 = ctypes.c_void_p, ctypes.c_int
            h.svdq_device_check.argtypes = [i32]
            h.svdq_device_check.restype = i32
            h.svdq_status_str.argtypes = [i32]
            h.svdq_status_str.restype = ctypes.c_char_p
            h.svdq_version.argtypes = []
            h.svdq_version.restype = i32
            h.svdq_quantize_act.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
            h.svdq_quantize_act.restype = i32
            h.svdq_gemm_w4a4.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
            h.svdq_gemm_w4a4.restype = i32
            h.svdq_gemm_w4a4_qkv.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_float, vp, vp]
            h.svdq_gemm_w4a4_qkv.restype = i32
            f32 = ctypes.c_float
            h.svdq_quantize_act_nvfp4.argtypes = [i32, i32, i32, i32, vp, vp, vp, f32, vp, vp, vp, vp]
            h.svdq_quantize_act_nvfp4.restype = i32
            h.svdq_gemm_nvfp4.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, f32, i32, vp, vp]
            h.svdq_gemm_nvfp4.restype = i32
            sz = ctypes.c_size_t
            h.svdq_gemm_w4a4_mlp_workspace.argtypes = [i32, i32, i32]
            h.svdq_gemm_w4a4_mlp_workspace.restype = sz
            h.svdq_gemm_w4a4_mlp.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp, i32, vp, vp, vp, vp, sz, vp]
            h.svdq_gemm_w4a4_mlp.restype = i32
            h.svdq_gemm_w4a4_mlp_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                     vp, vp, i32, vp, vp, vp, vp]
            h.svdq_gemm_w4a4_mlp_noalloc.restype = i32
            h.awq_gemv_w4a16.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
            h.awq_gemv_w4a16.restype = i32
            h.svdq_gemm_w4a4_splitk.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                vp, sz, vp]
            h.svdq_gemm_w4a4_splitk.restype = i32
            h.svdq_gemm_w4a4_splitk_workspace.argtypes = [i32, i32, i32, i32]
            h.svdq_gemm_w4a4_splitk_workspace.restype = sz
            h.svdq_clock_probe.argtypes = [i32, ctypes.c_ulonglong, vp, ctypes.POINTER(i32), vp]
            h.svdq_clock_probe.restype = i32
            _handle = h
        return _handle


def svdq_status_str(status: int) -> str:
    return lib().svdq_status_str(int(status)).decode()


def svdq_version() -> int:
    return lib().svdq_version()


def svdq_device_check(device: int = 0) -> int:
    return lib().svdq_device_check(int(device))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, shape, dev):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _io(t: torch.Tensor, name: str) -> int:
    if t.dtype not in DTYPES:
        raise TypeError(f"{name} has dtype {t.dtype}; the layer's 16-bit type is float16 or bfloat16")
    return DTYPES[t.dtype]


def _pick_dtype(dtype, *tensors):
    """The GEMM's 16-bit type: given, else that of the first 16-bit tensor passed, else fp16."""
    if dtype is not None:
        return dtype
    for t in tensors:
        if t is not None:
            return t.dtype
    return torch.float16


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}")
        return FORMATS[fmt]
    return int(fmt)


def _scale_spec(fmt: int, rows: int, K: int):
    if fmt == INT4_G64:
        return torch.float16, (rows, K // 64)
    return torch.uint8, (rows, K // 32)


def svdq_quantize_act(X: torch.Tensor, smooth_inv: torch.Tensor, lora_down, fmt="int4_g64",
                      act_codes=None, act_scales=None, lora_act=None):
    """Smoothing + low-rank down-projection + 4-bit activation quantization.

    X [M][K] in the layer's 16-bit type (float16 or bfloat16); smooth_inv fp32
    [K]; lora_down [r][K] (same 16-bit type) or None. Returns (act_codes u8
    [M][K/2], act_scales fp16 [M][K/64] | u8 [M][K/32], lora_act fp32 [M][r] or
    None). Output tensors may be passed in.
    """
    f = _fmt(fmt)
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("X must be a HIP device tensor")
    M, K = X.shape
    io = _io(X, "X")
    h = X.dtype
    r = 0 if lora_down is None else lora_down.shape[0]
    _check(X, "X", h, (M, K), dev)
    _check(smooth_inv, "smooth_inv", torch.float32, (K,), dev)
    if lora_down is not None:
        _check(lora_down, "lora_down", h, (r, K), dev)
    sdt, sshape = _scale_spec(f, M, K)
    if act_codes is None:
        act_codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if act_scales is None:
        act_scales = torch.empty(sshape, dtype=sdt, device=dev)
    if r > 0 and lora_act is None:
        lora_act = torch.empty((M, r), dtype=torch.float32, device=dev)
    _check(act_codes, "act_codes", torch.uint8, (M, K // 2), dev)
    _check(act_scales, "act_scales", sdt, sshape, dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
    with torch.cuda.device(dev):
        st = lib().svdq_quantize_act(f, io, M, K, r, _ptr(X), _ptr(smooth_inv), _ptr(lora_down),
                                     _ptr(act_codes), _ptr(act_scales),
                                     _ptr(lora_act) if r > 0 else None, _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "svdq_quantize_act")
    return act_codes, act_scales, (lora_act if r > 0 else None)


def _gemm_call(name, act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias, fmt, epilogue, out,
               dtype, extra):
    f = _fmt(fmt)
    h = _pick_dtype(dtype, lora_up, bias, out)
    io = DTYPES[h]
    e = EPILOGUES[epilogue] if isinstance(epilogue, str) else int(epilogue)
    dev = act_codes.device
    if dev.type != "cuda":
        raise ValueError("act_codes must be a HIP device tensor")
    M, KB = act_codes.shape
    K = 2 * KB
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    sdt, sa_shape = _scale_spec(f, M, K)
    _, sw_shape = _scale_spec(f, N, K)
    _check(act_codes, "act_codes", torch.uint8, (M, KB), dev)
    _check(act_scales, "act_scales", sdt, sa_shape, dev)
    _check(w_codes, "w_codes", torch.uint8, (N, KB), dev)
    _check(w_scales, "w_scales", sdt, sw_shape, dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
        _check(lora_up, "lora_up", h, (N, r), dev)
    if bias is not None:
        _check(bias, "bias", h, (N,), dev)
    if out is None:
        out = torch.empty((M, N), dtype=h, device=dev)
    _check(out, "out", h, (M, N), dev)
    with torch.cuda.device(dev):
        st = getattr(lib(), name)(f, io, M, N, K, r, _ptr(act_codes), _ptr(act_scales),
                                  _ptr(lora_act) if r > 0 else None, _ptr(w_codes), _ptr(w_scales),
                                  _ptr(lora_up) if r > 0 else None, _ptr(bias), e, _ptr(out),
                                  *extra(f, M, N, K, dev), _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, name)
    return out


def svdq_gemm_w4a4(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                   fmt="int4_g64", epilogue="none", out=None, dtype=None):
    """Fused 4-bit GEMM + low-rank up-projection + bias (+ GELU) -> Y [M][N] in
    the layer's 16-bit type (dtype, else that of lora_up / bias / out, else
    float16); lora_act is fp32 [M][r]."""
    return _gemm_call("svdq_gemm_w4a4", act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias, fmt,
                      epilogue, out, dtype, lambda f, M, N, K, dev: ())


def svdq_gemm_w4a4_splitk_workspace(M: int, N: int, K: int, fmt="int4_g64") -> int:
    """Bytes of workspace svdq_gemm_w4a4_splitk splits K with (0: no split)."""
    return int(lib().svdq_gemm_w4a4_splitk_workspace(_fmt(fmt), int(M), int(N), int(K)))


def svdq_gemm_w4a4_splitk(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                          fmt="int4_g64", epilogue="none", out=None, dtype=None, workspace=None):
    """svdq_gemm_w4a4 with K split across workgroups for shapes with few output
    tiles; `workspace` is a device uint8 tensor of at least
    svdq_gemm_w4a4_splitk_workspace(M, N, K) bytes (allocated here when None;
    a smaller one runs the unsplit kernel)."""
    def extra(f, M, N, K, dev):
        nonlocal workspace
        if workspace is None:
            n = int(lib().svdq_gemm_w4a4_splitk_workspace(f, M, N, K))
            workspace = torch.empty((max(n, 16),), dtype=torch.uint8, device=dev)
        _check(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
        return (_ptr(workspace), ctypes.c_size_t(workspace.numel()))
    return _gemm_call("svdq_gemm_w4a4_splitk", act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                      fmt, epilogue, out, dtype, extra)


def svdq_gemm_w4a4_qkv(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                       qk_norm_w, rope, eps: float = 1e-6, fmt="int4_g64", out=None, dtype=None):
    """Fused Q|K|V projection: the 4-bit GEMM, then per-head (128-channel)
    RMSNorm of the Q and K thirds and the rotation of channel pairs by rope
    (fp32 [M][64][2] cos, sin); V unchanged -> Y [M][N], N % 384 == 0, in the
    layer's 16-bit type (that of qk_norm_w)."""
    f = _fmt(fmt)
    h = _pick_dtype(dtype, qk_norm_w)
    io = DTYPES[h]
    dev = act_codes.device
    if dev.type != "cuda":
        raise ValueError("act_codes must be a HIP device tensor")
    M, KB = act_codes.shape
    K = 2 * KB
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    sdt, sa_shape = _scale_spec(f, M, K)
    _, sw_shape = _scale_spec(f, N, K)
    _check(act_codes, "act_codes", torch.uint8, (M, KB), dev)
    _check(act_scales, "act_scales", sdt, sa_shape, dev)
    _check(w_codes, "w_codes", torch.uint8, (N, KB), dev)
    _check(w_scales, "w_scales", sdt, sw_shape, dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
        _check(lora_up, "lora_up", h, (N, r), dev)
    if bias is not None:
        _check(bias, "bias", h, (N,), dev)
    _check(qk_norm_w, "qk_norm_w", h, (2, 128), dev)
    _check(rope, "rope", torch.float32, (M, 64, 2), dev)
    if out is None:
        out = torch.empty((M, N), dtype=h, device=dev)
    _check(out, "out", h, (M, N), dev)
    with torch.cuda.device(dev):
        st = lib().svdq_gemm_w4a4_qkv(f, io, M, N, K, r, _ptr(act_codes), _ptr(act_scales),
                                      _ptr(lora_act) if r > 0 else None, _ptr(w_codes), _ptr(w_scales),
                                      _ptr(lora_up) if r > 0 else None, _ptr(bias), _ptr(qk_norm_w),
                                      _ptr(rope), ctypes.c_float(eps), _ptr(out), _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "svdq_gemm_w4a4_qkv")
    return out


def svdq_gemm_w4a4_mlp(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                       smooth_inv2, lora_down2, fmt="int4_g64", act_codes2=None, act_scales2=None,
                       lora_act2=None, workspace=None, dtype=None):
    """The fused MLP chain: the up-projection with GELU, straight into the
    down-projection's INT4 quantizer. Returns (act_codes2 u8 [M][N/2],
    act_scales2 fp16 [M][N/64], lora_act2 fp32 [M][r2] or None), what
    svdq_quantize_act would give on the up-projection's output. workspace:
    fp32 device memory of svdq_gemm_w4a4_mlp_workspace(M, N, r2) bytes (taken
    from torch's allocator when not given)."""
    f = _fmt(fmt)
    h = _pick_dtype(dtype, lora_up, bias, lora_down2)
    io = DTYPES[h]
    dev = act_codes.device
    if dev.type != "cuda":
        raise ValueError("act_codes must be a HIP device tensor")
    M, KB = act_codes.shape
    K = 2 * KB
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    r2 = 0 if lora_down2 is None else lora_down2.shape[0]
    sdt, sa_shape = _scale_spec(f, M, K)
    _, sw_shape = _scale_spec(f, N, K)
    _check(act_codes, "act_codes", torch.uint8, (M, KB), dev)
    _check(act_scales, "act_scales", sdt, sa_shape, dev)
    _check(w_codes, "w_codes", torch.uint8, (N, KB), dev)
    _check(w_scales, "w_scales", sdt, sw_shape, dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
        _check(lora_up, "lora_up", h, (N, r), dev)
    if bias is not None:
        _check(bias, "bias", h, (N,), dev)
    _check(smooth_inv2, "smooth_inv2", torch.float32, (N,), dev)
    if r2 > 0:
        _check(lora_down2, "lora_down2", h, (r2, N), dev)
    if act_codes2 is None:
        act_codes2 = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    if act_scales2 is None:
        act_scales2 = torch.empty((M, N // 64), dtype=torch.float16, device=dev)
    if r2 > 0 and lora_act2 is None:
        lora_act2 = torch.empty((M, r2), dtype=torch.float32, device=dev)
    _check(act_codes2, "act_codes2", torch.uint8, (M, N // 2), dev)
    _check(act_scales2, "act_scales2", torch.float16, (M, N // 64), dev)
    if r2 > 0:
        _check(lora_act2, "lora_act2", torch.float32, (M, r2), dev)
    need = lib().svdq_gemm_w4a4_mlp_workspace(M, N, r2)
    if r2 > 0 and workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = lib().svdq_gemm_w4a4_mlp(f, io, M, N, K, r, _ptr(act_codes), _ptr(act_scales),
                                      _ptr(lora_act) if r > 0 else None, _ptr(w_codes), _ptr(w_scales),
                                      _ptr(lora_up) if r > 0 else None, _ptr(bias), _ptr(smooth_inv2),
                                      _ptr(lora_down2) if r2 > 0 else None, r2, _ptr(act_codes2),
                                      _ptr(act_scales2), _ptr(lora_act2) if r2 > 0 else None,
                                      _ptr(workspace) if r2 > 0 else None, wbytes, _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "svdq_gemm_w4a4_mlp")
    return act_codes2, act_scales2, (lora_act2 if r2 > 0 else None)


NOALLOC_SCRATCH_BYTES = 64 << 20   # the library's device scratch of the allocation-free chain


def svdq_gemm_w4a4_mlp_noalloc(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                               smooth_inv2, lora_down2, act_codes2, act_scales2, lora_act2, fmt="int4_g64",
                               dtype=None):
    """svdq_gemm_w4a4_mlp without a workspace and without any allocation: the
    fp32 partials live in the library's per-GPU device scratch (64 MiB; calls
    that overlap on one GPU race). The outputs act_codes2 u8 [M][N/2],
    act_scales2 fp16 [M][N/64] and lora_act2 fp32 [M][r2] (None when r2 == 0)
    must be passed; nothing is allocated here either. Returns them."""
    f = _fmt(fmt)
    h = _pick_dtype(dtype, lora_up, bias, lora_down2)
    io = DTYPES[h]
    dev = act_codes.device
    if dev.type != "cuda":
        raise ValueError("act_codes must be a HIP device tensor")
    M, KB = act_codes.shape
    K = 2 * KB
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    r2 = 0 if lora_down2 is None else lora_down2.shape[0]
    sdt, sa_shape = _scale_spec(f, M, K)
    _, sw_shape = _scale_spec(f, N, K)
    _check(act_codes, "act_codes", torch.uint8, (M, KB), dev)
    _check(act_scales, "act_scales", sdt, sa_shape, dev)
    _check(w_codes, "w_codes", torch.uint8, (N, KB), dev)
    _check(w_scales, "w_scales", sdt, sw_shape, dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
        _check(lora_up, "lora_up", h, (N, r), dev)
    if bias is not None:
        _check(bias, "bias", h, (N,), dev)
    _check(smooth_inv2, "smooth_inv2", torch.float32, (N,), dev)
    _check(act_codes2, "act_codes2", torch.uint8, (M, N // 2), dev)
    _check(act_scales2, "act_scales2", torch.float16, (M, N // 64), dev)
    if r2 > 0:
        _check(lora_down2, "lora_down2", h, (r2, N), dev)
        _check(lora_act2, "lora_act2", torch.float32, (M, r2), dev)
    with torch.cuda.device(dev):
        st = lib().svdq_gemm_w4a4_mlp_noalloc(f, io, M, N, K, r, _ptr(act_codes), _ptr(act_scales),
                                              _ptr(lora_act) if r > 0 else None, _ptr(w_codes),
                                              _ptr(w_scales), _ptr(lora_up) if r > 0 else None, _ptr(bias),
                                              _ptr(smooth_inv2), _ptr(lora_down2) if r2 > 0 else None, r2,
                                              _ptr(act_codes2), _ptr(act_scales2),
                                              _ptr(lora_act2) if r2 > 0 else None, _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "svdq_gemm_w4a4_mlp_noalloc")
    return act_codes2, act_scales2, (lora_act2 if r2 > 0 else None)


def svdq_quantize_act_nvfp4(X: torch.Tensor, smooth_inv: torch.Tensor, lora_down, act_gscale: float,
                            act_codes=None, act_scales=None, lora_act=None):
    """NVFP4 activation quantizer (E2M1 codes, E4M3 scale per 16, per-tensor
    scale act_gscale) + smoothing + low-rank down-projection.
    Returns (act_codes u8 [M][K/2], act_scales u8 [M][K/16], lora_act fp32
    [M][r] or None); X and lora_down share the layer's 16-bit type."""
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("X must be a HIP device tensor")
    M, K = X.shape
    io = _io(X, "X")
    h = X.dtype
    r = 0 if lora_down is None else lora_down.shape[0]
    _check(X, "X", h, (M, K), dev)
    _check(smooth_inv, "smooth_inv", torch.float32, (K,), dev)
    if lora_down is not None:
        _check(lora_down, "lora_down", h, (r, K), dev)
    if act_codes is None:
        act_codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if act_scales is None:
        act_scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    if r > 0 and lora_act is None:
        lora_act = torch.empty((M, r), dtype=torch.float32, device=dev)
    _check(act_codes, "act_codes", torch.uint8, (M, K // 2), dev)
    _check(act_scales, "act_scales", torch.uint8, (M, K // 16), dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
    with torch.cuda.device(dev):
        st = lib().svdq_quantize_act_nvfp4(io, M, K, r, _ptr(X), _ptr(smooth_inv), _ptr(lora_down),
                                           ctypes.c_float(act_gscale), _ptr(act_codes), _ptr(act_scales),
                                           _ptr(lora_act) if r > 0 else None, _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "svdq_quantize_act_nvfp4")
    return act_codes, act_scales, (lora_act if r > 0 else None)


def svdq_gemm_nvfp4(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias, alpha: float,
                    epilogue="none", out=None, dtype=None):
    """NVFP4 GEMM + low-rank up-projection + bias (+ GELU) -> Y [M][N] in the
    layer's 16-bit type; alpha = act_gscale * w_gscale scales the 4-bit sum;
    lora_act is fp32 [M][r]."""
    e = EPILOGUES[epilogue] if isinstance(epilogue, str) else int(epilogue)
    h = _pick_dtype(dtype, lora_up, bias, out)
    io = DTYPES[h]
    dev = act_codes.device
    if dev.type != "cuda":
        raise ValueError("act_codes must be a HIP device tensor")
    M, KB = act_codes.shape
    K = 2 * KB
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    _check(act_codes, "act_codes", torch.uint8, (M, KB), dev)
    _check(act_scales, "act_scales", torch.uint8, (M, K // 16), dev)
    _check(w_codes, "w_codes", torch.uint8, (N, KB), dev)
    _check(w_scales, "w_scales", torch.uint8, (N, K // 16), dev)
    if r > 0:
        _check(lora_act, "lora_act", torch.float32, (M, r), dev)
        _check(lora_up, "lora_up", h, (N, r), dev)
    if bias is not None:
        _check(bias, "bias", h, (N,), dev)
    if out is None:
        out = torch.empty((M, N), dtype=h, device=dev)
    _check(out, "out", h, (M, N), dev)
    with torch.cuda.device(dev):
        st = lib().svdq_gemm_nvfp4(io, M, N, K, r, _ptr(act_codes), _ptr(act_scales),
                                   _ptr(lora_act) if r > 0 else None, _ptr(w_codes), _ptr(w_scales),
                                   _ptr(lora_up) if r > 0 else None, _ptr(bias), ctypes.c_float(alpha), e,
                                   _ptr(out), _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "svdq_gemm_nvfp4")
    return out


def awq_gemv_w4a16(x, w_codes, scales, zeros, group: int = 64, out=None, bias=None):
    """AWQ W4A16 GEMV: y[m,n] = sum_k x[m,k] (q[n,k] - z) s + bias[n] -> y [M][N];
    x, bias and y share the layer's 16-bit type, scales and zeros are fp16."""
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a HIP device tensor")
    M, K = x.shape
    N = w_codes.shape[0]
    io = _io(x, "x")
    h = x.dtype
    _check(x, "x", h, (M, K), dev)
    _check(w_codes, "w_codes", torch.uint8, (N, K // 2), dev)
    _check(scales, "scales", torch.float16, (N, K // group), dev)
    _check(zeros, "zeros", torch.float16, (N, K // group), dev)
    if bias is not None:
        _check(bias, "bias", h, (N,), dev)
    if out is None:
        out = torch.empty((M, N), dtype=h, device=dev)
    _check(out, "out", h, (M, N), dev)
    with torch.cuda.device(dev):
        st = lib().awq_gemv_w4a16(io, M, N, K, group, _ptr(x), _ptr(w_codes), _ptr(scales),
                                  _ptr(zeros), _ptr(bias), _ptr(out), _stream(dev))
    if st != SVDQ_OK:
        raise SvdqError(st, "awq_gemv_w4a16")
    return out


def svdq_linear(X, layer: dict, bias=None, epilogue: str = "none"):
    """One SVDQ W4A4 linear layer: the two fused calls back to back.
    layer holds device tensors smooth_inv, lora_down, w_codes, w_scales,
    lora_up and the format name under "fmt"."""
    codes, scales, la = svdq_quantize_act(X, layer["smooth_inv"], layer.get("lora_down"), layer["fmt"])
    return svdq_gemm_w4a4(codes, scales, la, layer["w_codes"], layer["w_scales"],
                          layer.get("lora_up"), bias, layer["fmt"], epilogue)


def svdq_clock_probe(device=0, workgroups=256, ticks=200_000):
    """The shader clock in MHz, one value per workgroup (numpy float64): each
    workgroup counts shader cycles while the real-time counter advances by
    `ticks`. Synchronizes the device's current stream."""
    dev = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
    with torch.cuda.device(dev):
        out = torch.empty((workgroups, 2), dtype=torch.int64, device=dev)
        khz = ctypes.c_int(0)
        st = lib().svdq_clock_probe(int(workgroups), int(ticks), _ptr(out), ctypes.byref(khz), _stream(dev))
        if st != 0:
            raise SvdqError(st, "svdq_clock_probe")
        cyc = out.cpu().numpy().astype("float64")
    return cyc[:, 0] / cyc[:, 1] * khz.value / 1000.0
