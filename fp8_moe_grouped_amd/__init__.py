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
ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 32 << 20
DEV_SUM_CLAMPED, DEV_NEGATIVE_SIZE = 1, 2
E4M3, E5M2 = 0, 1
(OP_FWD, OP_SILU, OP_DLHS, OP_TGMM, OP_BF16_FWD, OP_BF16_DLHS, OP_FFN_FWD, OP_FFN_BWD, OP_FWD_VARIANT,
 OP_TGMM_DENSE) = range(10)
LHS_SCALE_BF16, ACC_BF16, RHS_SCALE_FIRST = 1, 2, 4
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
    "gmm_fp8_fwd_noalloc": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "gmm_silu_fp8": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _SZ, _P, _P],
    "gmm_dlhs_fp8": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _SZ, _P, _P],
    "tgmm_quant": [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "dequantize_fp8_codes": [_P, _P, _I32, _I64, _I64, _P, _P],
    "tgmm_dense_quant": [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "quantize_rows_fp8": [_P, _P, _I64, _I64, _I32, _P, _P, _P],
    "gmm_fp8_fwd_q": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "gmm_silu_fp8_q": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P],
    "gmm_fp8_fwd_variant": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "gmm_dswiglu_fp8": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "moe_ffn_fp8_fwd": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _SZ, _P, _P],
    "moe_ffn_fp8_bwd": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _P,
                        _SZ, _P, _P],
    "gmm_bf16_fwd": [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
    "gmm_bf16_silu": [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _P, _P],
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


def _fwd(name, op, lhs, codes, scale, group_sizes, out, debug, dev_status, workspace, swiglu, preact=None):
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
    if preact is True:
        preact = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if preact is not None:
        _req(preact, "preact", torch.bfloat16, 2)
        if tuple(preact.shape) != (M, N):
            raise ValueError(f"preact must be [{M}, {N}], got {tuple(preact.shape)}")
    dbg_codes = torch.empty((M, K), dtype=torch.uint8, device=dev) if debug else None
    dbg_scale = torch.empty((M,), dtype=torch.float32, device=dev) if debug else None
    ws, need = _workspace(op, M, K, N, G, dev, workspace=workspace)
    extra = (_ptr(preact),) if swiglu else ()
    with torch.cuda.device(dev):
        _call(name, _ptr(lhs), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G, _ptr(out), *extra,
              _ptr(dbg_codes), _ptr(dbg_scale), _ptr(ws), need, _ptr(dev_status), _stream(dev))
    res = (out,) + ((preact,) if preact is not None else ()) + ((dbg_codes, dbg_scale) if debug else ())
    return res if len(res) > 1 else out


def gmm_fp8_fwd(lhs, codes, scale, group_sizes, *, out=None, debug=False, dev_status=None, workspace=None):
    """Native FP8 forward GMM; returns bf16 [M, N] (and, with debug, the
    activation codes [M, K] and row scales [M] the GEMM consumed)."""
    return _fwd("gmm_fp8_fwd", OP_FWD, lhs, codes, scale, group_sizes, out, debug, dev_status, workspace, False)


def gmm_fp8_fwd_noalloc(lhs, codes, scale, group_sizes, *, out=None, dev_status=None):
    """gmm_fp8_fwd through the allocation-free entry point: the library keeps
    the quantized activations in its fixed per-GPU scratch (the call itself
    allocates nothing; only ``out``, if not given, is allocated here).
    Returns bf16 [M, N]."""
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, codes, scale, group_sizes)
    M, K = lhs.shape
    G, K2, N = codes.shape
    if K2 != K or tuple(scale.shape) != (G, N) or group_sizes.shape[0] != G:
        raise ValueError("shape mismatch")
    out = _out(out, (M, N), torch.bfloat16, dev, "out")
    with torch.cuda.device(dev):
        _call("gmm_fp8_fwd_noalloc", _ptr(lhs), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
              _ptr(dev_status), _stream(dev))
    return out


def gmm_silu_fp8(lhs, codes, scale, group_sizes, *, out=None, preact=None, debug=False, dev_status=None,
                 workspace=None):
    """Native FP8 forward GMM with fused SwiGLU over [gate | up]; bf16 [M, N/2].
    ``preact`` (a bf16 [M, N] tensor, or True to allocate one) also receives
    the pre-activation; the result is then ``(out, preact)`` (followed by the
    debug outputs when asked)."""
    return _fwd("gmm_silu_fp8", OP_SILU, lhs, codes, scale, group_sizes, out, debug, dev_status, workspace, True,
                preact)


def gmm_fp8_fwd_variant(lhs, codes, scale, group_sizes, *, lhs_block=0, scale_bf16=False, acc_bf16=False,
                        rhs_scale_first=False, out=None, debug=False, dev_status=None, workspace=None):
    """The FP8 forward with the ops-level LHS-quantization options: one scale
    per row (lhs_block=0) or per 512 columns, optionally rounded to bf16, a
    bf16 accumulator across the 512-column blocks, and the weight scale
    applied first.  Returns bf16 [M, N] (with debug also the codes [M, K] and
    the scales [M, nb])."""
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, codes, scale, group_sizes)
    M, K = lhs.shape
    G, K2, N = codes.shape
    if K2 != K or tuple(scale.shape) != (G, N) or group_sizes.shape[0] != G:
        raise ValueError("shape mismatch")
    flags = (LHS_SCALE_BF16 if scale_bf16 else 0) | (ACC_BF16 if acc_bf16 else 0) | \
        (RHS_SCALE_FIRST if rhs_scale_first else 0)
    nb = -(-K // 512) if lhs_block == 512 else 1
    out = _out(out, (M, N), torch.bfloat16, dev, "out")
    dbg_codes = torch.empty((M, K), dtype=torch.uint8, device=dev) if debug else None
    dbg_scale = torch.empty((M, nb), dtype=torch.float32, device=dev) if debug else None
    ws, need = _workspace(OP_FWD_VARIANT, M, K, N, G, dev, tile_m=lhs_block, workspace=workspace)
    with torch.cuda.device(dev):
        _call("gmm_fp8_fwd_variant", _ptr(lhs), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G,
              int(lhs_block), flags, _ptr(out), _ptr(dbg_codes), _ptr(dbg_scale), _ptr(ws), need, _ptr(dev_status),
              _stream(dev))
    return (out, dbg_codes, dbg_scale) if debug else out


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


def _fwd_q(name, aq, ascale, codes, scale, group_sizes, out, dev_status, swiglu, preact=None):
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
    if preact is not None:
        _req(preact, "preact", torch.bfloat16, 2)
        if tuple(preact.shape) != (M, N):
            raise ValueError(f"preact must be [{M}, {N}], got {tuple(preact.shape)}")
    extra = (_ptr(preact),) if swiglu else ()
    with torch.cuda.device(dev):
        _call(name, _ptr(aq), _ptr(ascale), _ptr(codes), _ptr(scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
              *extra, _ptr(dev_status), _stream(dev))
    return out


def gmm_fp8_fwd_q(aq, ascale, codes, scale, group_sizes, *, out=None, dev_status=None):
    """FP8 forward GEMM on already quantized activations (codes + row scales)."""
    return _fwd_q("gmm_fp8_fwd_q", aq, ascale, codes, scale, group_sizes, out, dev_status, False)


def gmm_silu_fp8_q(aq, ascale, codes, scale, group_sizes, *, out=None, preact=None, dev_status=None):
    """FP8 forward GEMM + SwiGLU on already quantized activations; a bf16
    [M, N] ``preact`` tensor, if given, receives the pre-activation."""
    return _fwd_q("gmm_silu_fp8_q", aq, ascale, codes, scale, group_sizes, out, dev_status, True, preact)


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


def gmm_dswiglu_fp8(dout, codes, scale, group_sizes, preact, *, out=None, dev_status=None):
    """wo backward dLHS fused with the SwiGLU derivative: from the wo output
    gradient dout [M, H], the wo codes [G, I, H] and the wi pre-activation
    preact [M, 2I], returns the pre-activation gradient bf16 [M, 2I]."""
    _req(dout, "dout", torch.bfloat16, 2)
    _req(codes, "codes", torch.uint8, 3)
    _req(scale, "scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    _req(preact, "preact", torch.bfloat16, 2)
    dev = _same_device(dout, codes, scale, group_sizes, preact)
    M, N = dout.shape
    G, K, N2 = codes.shape
    if N2 != N or tuple(scale.shape) != (G, N) or group_sizes.shape[0] != G or tuple(preact.shape) != (M, 2 * K):
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, 2 * K), dtype=torch.bfloat16, device=dev)
    _req(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, 2 * K):
        raise ValueError("out must be [M, 2K]")
    with torch.cuda.device(dev):
        _call("gmm_dswiglu_fp8", _ptr(dout), _ptr(codes), _ptr(scale), _ptr(group_sizes), _ptr(preact), M, K, N, G,
              _ptr(out), _ptr(dev_status), _stream(dev))
    return out


def _ffn_shapes(x, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes):
    _req(x, "x", torch.bfloat16, 2)
    _req(wi_codes, "wi_codes", torch.uint8, 3)
    _req(wi_scale, "wi_scale", torch.float32, 2)
    _req(wo_codes, "wo_codes", torch.uint8, 3)
    _req(wo_scale, "wo_scale", torch.float32, 2)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(x, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes)
    M, H = x.shape
    G, H2, I2 = wi_codes.shape
    I = I2 // 2
    if (H2 != H or I2 != 2 * I or tuple(wi_scale.shape) != (G, I2) or tuple(wo_codes.shape) != (G, I, H)
            or tuple(wo_scale.shape) != (G, H) or group_sizes.shape[0] != G):
        raise ValueError(f"FFN shape mismatch: x {tuple(x.shape)} wi {tuple(wi_codes.shape)} "
                         f"wo {tuple(wo_codes.shape)}")
    return dev, M, H, I, G


def _out(t, shape, dtype, dev, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _req(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    return t


def moe_ffn_fp8_fwd(x, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes, *, keep_preact=True, h=None,
                    preact=None, y=None, dev_status=None, workspace=None):
    """Forward of one routed-expert FFN: h = SwiGLU FP8 GMM of x with wi,
    y = FP8 GMM of h with wo.  Returns (y [M, H], h [M, I], preact [M, 2I] or
    None)."""
    dev, M, H, I, G = _ffn_shapes(x, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes)
    h = _out(h, (M, I), torch.bfloat16, dev, "h")
    y = _out(y, (M, H), torch.bfloat16, dev, "y")
    preact = _out(preact, (M, 2 * I), torch.bfloat16, dev, "preact") if (keep_preact or preact is not None) else None
    ws, need = _workspace(OP_FFN_FWD, M, H, I, G, dev, tile_m=0, workspace=workspace)
    with torch.cuda.device(dev):
        _call("moe_ffn_fp8_fwd", _ptr(x), _ptr(wi_codes), _ptr(wi_scale), _ptr(wo_codes), _ptr(wo_scale),
              _ptr(group_sizes), M, H, I, G, _ptr(h), _ptr(preact), _ptr(y), _ptr(ws), need, _ptr(dev_status),
              _stream(dev))
    return y, h, preact


def moe_ffn_fp8_bwd(x, h, preact, dy, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes, grad_dtype="e5m2", *,
                    need_dx=True, d_preact=None, dx=None, dwi=None, dwo=None, dev_status=None, workspace=None):
    """Backward of one routed-expert FFN from the forward's x, h, preact and
    the output gradient dy [M, H].  Returns (dx [M, H] or None, dwi
    [G, H, 2I] f32, dwo [G, I, H] f32, d_preact [M, 2I])."""
    dev, M, H, I, G = _ffn_shapes(x, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes)
    for t, name, shape in ((h, "h", (M, I)), (preact, "preact", (M, 2 * I)), (dy, "dy", (M, H))):
        _req(t, name, torch.bfloat16, 2)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
    _same_device(x, h, preact, dy)
    gd = GRAD_DTYPES[grad_dtype] if isinstance(grad_dtype, str) else int(grad_dtype)
    d_preact = _out(d_preact, (M, 2 * I), torch.bfloat16, dev, "d_preact")
    dx = _out(dx, (M, H), torch.bfloat16, dev, "dx") if (need_dx or dx is not None) else None
    dwi = _out(dwi, (G, H, 2 * I), torch.float32, dev, "dwi")
    dwo = _out(dwo, (G, I, H), torch.float32, dev, "dwo")
    ws, need = _workspace(OP_FFN_BWD, M, H, I, G, dev, tile_m=512, workspace=workspace)
    with torch.cuda.device(dev):
        _call("moe_ffn_fp8_bwd", _ptr(x), _ptr(h), _ptr(preact), _ptr(dy), _ptr(wi_codes), _ptr(wi_scale),
              _ptr(wo_codes), _ptr(wo_scale), _ptr(group_sizes), M, H, I, G, gd, _ptr(d_preact), _ptr(dx),
              _ptr(dwi), _ptr(dwo), _ptr(ws), need, _ptr(dev_status), _stream(dev))
    return dx, dwi, dwo, d_preact


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


def tgmm_workspace_codes(workspace, M, K, N, G, tile_m=512):
    """Views of the operand codes a tgmm_quant call left in its workspace
    (the layout the header documents): qL uint8 [Tmax, tile_m, K] and qD
    uint8 [Tmax, tile_m, N], one slab per non-empty (expert, tile) pair in
    (expert, tile) order; slab p holds the pair's rows in order, then zero
    codes up to the next multiple of 32 rows."""
    tmax = -(-M // tile_m) + G - 1
    al = lambda x: (x + 255) // 256 * 256
    need = workspace_bytes(OP_TGMM, M, K, N, G, tile_m)
    if workspace.numel() < need or tmax <= 0:
        raise ValueError("workspace too small for these sizes")
    ql = workspace[: tmax * tile_m * K].view(tmax, tile_m, K)
    off = al(tmax * tile_m * K)
    qd = workspace[off: off + tmax * tile_m * N].view(tmax, tile_m, N)
    return ql, qd


def tgmm_workspace_deal(workspace, M, K, N, G, tile_m=512):
    """View of the GEMM's work-item deal a tgmm_quant call left in its
    workspace (the layout the header documents): int32 [G] block offsets."""
    tmax = -(-M // tile_m) + G - 1
    al = lambda x: (x + 255) // 256 * 256
    off = al(tmax * tile_m * K) + al(tmax * tile_m * N) + al(tmax * K * 4) + al(tmax * N * 4)
    if workspace.numel() < off + 4 * G or tmax <= 0:
        raise ValueError("workspace too small for these sizes")
    return workspace[off: off + 4 * G].view(torch.int32)


def tgmm_dense_quant(lhs, dout, group_sizes, grad_dtype="e5m2", *, out=None, debug=False, dev_status=None,
                     workspace=None):
    """The buffer-wide backward quantization baseline (every row of the
    buffer, stale rows included): per-row lhs scale folded into dout, one
    gradient scale per column; returns f32 [G, K, N] (with debug also the row
    scales [M] and the column scales [N])."""
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
    out = _out(out, (G, K, N), torch.float32, dev, "out")
    srow = torch.empty((max(M, 1),), dtype=torch.float32, device=dev) if debug else None
    scol = torch.empty((N,), dtype=torch.float32, device=dev) if debug else None
    ws, need = _workspace(OP_TGMM_DENSE, M, K, N, G, dev, tile_m=0, workspace=workspace)
    with torch.cuda.device(dev):
        _call("tgmm_dense_quant", _ptr(lhs), _ptr(dout), _ptr(group_sizes), M, K, N, G, gd, _ptr(out), _ptr(srow),
              _ptr(scol), _ptr(ws), need, _ptr(dev_status), _stream(dev))
    return (out, srow, scol) if debug else out


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


def _bf16_fwd(name, lhs, w, group_sizes, out, swiglu, dev_status):
    _req(lhs, "lhs", torch.bfloat16, 2)
    _req(w, "w", torch.bfloat16, 3)
    _req(group_sizes, "group_sizes", torch.int32, 1)
    dev = _same_device(lhs, w, group_sizes)
    M, K = lhs.shape
    G, K2, N = w.shape
    if K2 != K or group_sizes.shape[0] != G:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, N // 2 if swiglu else N), dtype=torch.bfloat16, device=dev)
    _req(out, "out", torch.bfloat16, 2)
    with torch.cuda.device(dev):
        _call(name, _ptr(lhs), _ptr(w), _ptr(group_sizes), M, K, N, G, _ptr(out), _ptr(dev_status), _stream(dev))
    return out


def gmm_bf16_fwd(lhs, w, group_sizes, *, out=None, dev_status=None):
    """bf16 x bf16 grouped GEMM (the bf16 measurement arm); bf16 [M, N]."""
    return _bf16_fwd("gmm_bf16_fwd", lhs, w, group_sizes, out, False, dev_status)


def gmm_bf16_silu(lhs, w, group_sizes, *, out=None, dev_status=None):
    """bf16 grouped GEMM with the SwiGLU epilogue over [gate | up] (the bf16
    arm of gmm_silu_fp8); bf16 [M, N/2]."""
    return _bf16_fwd("gmm_bf16_silu", lhs, w, group_sizes, out, True, dev_status)


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
