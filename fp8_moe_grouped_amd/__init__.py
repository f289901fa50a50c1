"""Python binding of libfp8_moe_grouped.so, the MI355X (gfx950) routed-expert
FP8 grouped-matmul library.

Argument marshalling only: each function checks dtypes, shapes, devices and
contiguity of torch tensors, allocates outputs and the device workspace with
torch (torch is used for device memory and streams), and calls the C entry
point of the same name on the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
shared library is missing the first call raises.

The C contract of every call is documented in include/fp8_moe_grouped.h.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8_moe_grouped.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fp8_moe_grouped.h")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = -1, -2, -3, -4, -5, -6
DEV_SUM_CLAMPED, DEV_NEGATIVE_SIZE = 1, 2
E4M3, E5M2 = 0, 1
OP_FWD, OP_SILU, OP_DLHS, OP_TGMM, OP_BF16_FWD, OP_BF16_DLHS = 0, 1, 2, 3, 4, 5
GRAD_DTYPES = {"e4m3": E4M3, "e5m2": E5M2}


class Fp8GmmError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "gmm_fp8_fwd": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "gmm_silu_fp8": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "gmm_dlhs_fp8": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _SZ, _P, _P],
    "tgmm_quant": [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "dequantize_fp8_codes": [_P, _P, _I32, _I64, _I64, _P, _P],
    "quantize_rows_fp8": [_P, _P, _I64, _I64, _I32, _P, _P, _P],
    "gmm_fp8_fwd_q": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "gmm_silu_fp8_q": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "gmm_bf16_fwd": [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "gmm_bf16_dlhs": [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m fp8_moe_grouped_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.fp8gmm_workspace_bytes.argtypes = [_I32, _I64, _I64, _I64, _I32, _I32]
        L.fp8gmm_workspace_bytes.restype = ctypes.c_size_t
        L.fp8gmm_status_string.argtypes = [_I32]
        L.fp8gmm_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/fp8_moe_grouped.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return lib().fp8gmm_status_string(int(status)).decode()


def workspace_bytes(op: int, M: int, K: int, N: int, G: int, tile_m: int = 512) -> int:
    return int(lib().fp8gmm_workspace_bytes(op, M, K, N, G, tile_m))


# --------------------------------------------------------------------------- marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _req(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    return devs.pop()


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != OK:
        raise Fp8GmmError(name, st)


def _workspace(op, M, K, N, G, dev, tile_m=512, workspace=None):
    need = workspace_bytes(op, M, K, N, G, tile_m)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    return workspace, need


def _fwd(name, op, lhs, codes, scale, group_sizes, out, debug, dev_status, workspace, swiglu):
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, codes, scale, group_sizes)
    M, K = lhs.shape
    G, K2, N = codes.shape
    if K2 != K or tuple(scale.shape) != (G, N) or group_sizes.shape[0] != G:
        raise ValueError(f"shape mismatch: lhs {tuple(lhs.shape)} codes {tuple(codes.shape)} "
                         f"scale {tuple(scale.shape)} group_sizes {tuple(group_sizes.shape)}")
    ncol = N // 2 if swiglu else N
    if out is None:
        out = torch.empty((M, ncol), dtype=torch.bfloat16, device=dev)
    _req(out, "out", torch.bfloat16, 2)
    dbg_codes = torch.empty((M, K), dtype=torch.uint8, device=dev) if debug else None
    dbg_scale = torch.empty((M,), dtype=torch.float32, device=dev) if debug else None
    ws, need = _workspace(op, M, K, N, G, dev, workspace=workspace)
    with torch.cuda.device(dev):
        _call(name, _ptr(lhs), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
              _ptr(dbg_codes), _ptr(dbg_scale), _ptr(ws), need, _ptr(dev_status), _stream(dev))
    return (out, dbg_codes, dbg_scale) if debug else out


def gmm_fp8_fwd(lhs, codes, scale, group_sizes, *, out=None, debug=False, dev_status=None, workspace=None):
    """Native FP8 forward GMM; returns bf16 [M, N] (and, with debug, the
    activation codes [M, K] and row scales [M] the GEMM consumed)."""
    return _fwd("gmm_fp8_fwd", OP_FWD, lhs, codes, scale, group_sizes, out, debug, dev_status, workspace, False)


def gmm_silu_fp8(lhs, codes, scale, group_sizes, *, out=None, debug=False, dev_status=None, workspace=None):
    """Native FP8 forward GMM with fused SwiGLU over [gate | up]; bf16 [M, N/2]."""
    return _fwd("gmm_silu_fp8", OP_SILU, lhs, codes, scale, group_sizes, out, debug, dev_status, workspace, True)


def quantize_rows_fp8(lhs, group_sizes, *, codes=None, scales=None):
    """e4m3 codes [M, K] and f32 row scales [M] of the valid rows (the first
    half of gmm_fp8_fwd); rows past the valid prefix are left untouched."""
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, group_sizes)
    M, K = lhs.shape
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=dev)
    _req(codes, "codes", torch.uint8, 2)
    _req(scales, "scales", torch.float32, 1)
    with torch.cuda.device(dev):
        _call("quantize_rows_fp8", _ptr(lhs), _ptr(group_sizes), M, K, group_sizes.shape[0], _ptr(codes),
              _ptr(scales), _stream(dev))
    return codes, scales


def _fwd_q(name, aq, ascale, codes, scale, group_sizes, out, dev_status, swiglu):
    _req(aq, "aq", torch.uint8, 2)
    _req(ascale, "ascale", torch.float32, 1)
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(aq, ascale, codes, scale, group_sizes)
    M, K = aq.shape
    G, K2, N = codes.shape
    if K2 != K or tuple(scale.shape) != (G, N) or group_sizes.shape[0] != G or ascale.shape[0] != M:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, N // 2 if swiglu else N), dtype=torch.bfloat16, device=dev)
    _req(out, "out", torch.bfloat16, 2)
    with torch.cuda.device(dev):
        _call(name, _ptr(aq), _ptr(ascale), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
              _ptr(dev_status), _stream(dev))
    return out


def gmm_fp8_fwd_q(aq, ascale, codes, scale, group_sizes, *, out=None, dev_status=None):
    """FP8 forward GEMM on already quantized activations (codes + row scales)."""
    return _fwd_q("gmm_fp8_fwd_q", aq, ascale, codes, scale, group_sizes, out, dev_status, False)


def gmm_silu_fp8_q(aq, ascale, codes, scale, group_sizes, *, out=None, dev_status=None):
    """FP8 forward GEMM + SwiGLU on already quantized activations."""
    return _fwd_q("gmm_silu_fp8_q", aq, ascale, codes, scale, group_sizes, out, dev_status, True)


def gmm_dlhs_fp8(dout, codes, scale, group_sizes, *, out=None, dev_status=None, workspace=None):
    """Backward dLHS from FP8 codes; returns bf16 [M, K]."""
    _req(dout, "dout", torch.bfloat16, 2)
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(dout, codes, scale, group_sizes)
    M, N = dout.shape
    G, K, N2 = codes.shape
    if N2 != N or tuple(scale.shape) != (G, N) or group_sizes.shape[0] != G:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    _req(out, "out", torch.bfloat16, 2)
    ws, need = _workspace(OP_DLHS, M, K, N, G, dev, workspace=workspace)
    with torch.cuda.device(dev):
        _call("gmm_dlhs_fp8", _ptr(dout), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
              _ptr(ws), need, _ptr(dev_status), _stream(dev))
    return out


def tgmm_quant(lhs, dout, group_sizes, grad_dtype="e5m2", tile_m=512, *, out=None, debug=False,
               dev_status=None, workspace=None):
    """Weight-gradient tgmm with in-kernel per-(tile, channel) operand
    quantization; returns f32 [G, K, N] (and, with debug, the scales sL
    [Tmax, K] and sD [Tmax, N] of the non-empty (expert, tile) pairs)."""
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(dout, "dout", torch.bfloat16, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, dout, group_sizes)
    M, K = lhs.shape
    M2, N = dout.shape
    G = group_sizes.shape[0]
    if M2 != M:
        raise ValueError("lhs and dout must have the same number of rows")
    gd = GRAD_DTYPES[grad_dtype] if isinstance(grad_dtype, str) else int(grad_dtype)
    if out is None:
        out = torch.empty((G, K, N), dtype=torch.float32, device=dev)
    _req(out, "out", torch.float32, 3)
    tmax = -(-M // tile_m) + G - 1 if tile_m > 0 else 0
    dbg_sL = torch.empty((max(tmax, 1), K), dtype=torch.float32, device=dev) if debug else None
    dbg_sD = torch.empty((max(tmax, 1), N), dtype=torch.float32, device=dev) if debug else None
    ws, need = _workspace(OP_TGMM, M, K, N, G, dev, tile_m=tile_m, workspace=workspace)
    with torch.cuda.device(dev):
        _call("tgmm_quant", _ptr(lhs), _ptr(dout), _ptr(group_sizes), M, K, N, G, gd, tile_m, _ptr(out),
              _ptr(dbg_sL), _ptr(dbg_sD), _ptr(ws), need, _ptr(dev_status), _stream(dev))
    return (out, dbg_sL, dbg_sD) if debug else out


def dequantize_fp8_codes(codes, scale, *, out=None):
    """bf16 [G, K, N] = bf16(f32(dec(codes) * scale))."""
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    dev = _same_device(codes, scale)
    G, K, N = codes.shape
    if tuple(scale.shape) != (G, N):
        raise ValueError("scale must be [G, N]")
    if out is None:
        out = torch.empty((G, K, N), dtype=torch.bfloat16, device=dev)
    _req(out, "out", torch.bfloat16, 3)
    with torch.cuda.device(dev):
        _call("dequantize_fp8_codes", _ptr(codes), _ptr(scale), G, K, N, _ptr(out), _stream(dev))
    return out


def gmm_bf16_fwd(lhs, w, group_sizes, *, out=None, workspace=None):
    """bf16 x bf16 grouped GEMM (the bf16 measurement arm); bf16 [M, N]."""
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(w, "w", torch.bfloat16, 3)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, w, group_sizes)
    M, K = lhs.shape
    G, K2, N = w.shape
    if K2 != K or group_sizes.shape[0] != G:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    with torch.cuda.device(dev):
        _call("gmm_bf16_fwd", _ptr(lhs), _ptr(w), _ptr(group_sizes), M, K, N, G, _ptr(out), None, _stream(dev))
    return out


def gmm_bf16_dlhs(dout, w, group_sizes, *, out=None):
    """bf16 dLHS with bf16 weights w [G, K, N] (the bf16 measurement arm and
    the bit-identity reference of gmm_dlhs_fp8); bf16 [M, K]."""
    _req(dout, "dout", torch.bfloat16, 2)
    _req(w, "w", torch.bfloat16, 3)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(dout, w, group_sizes)
    M, N = dout.shape
    G, K, N2 = w.shape
    if N2 != N or group_sizes.shape[0] != G:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    with torch.cuda.device(dev):
        _call("gmm_bf16_dlhs", _ptr(dout), _ptr(w), _ptr(group_sizes), M, K, N, G, _ptr(out), None, _stream(dev))
    return out
