"""CPU tests of the C ABI boundary: the shared library loads, exports every
function include/fp8_moe_grouped.h declares, and rejects bad arguments on the
host before any HIP call (fake device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import fp8_moe_grouped_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(G.LIB_PATH):
        pytest.skip("library not built")
    return G.lib()


def test_exports_every_declared_function():
    L = _lib()
    names = G.header_functions()
    assert {"gmm_fp8_fwd", "gmm_silu_fp8", "gmm_dlhs_fp8", "tgmm_quant", "dequantize_fp8_codes"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    # the binding's marshalling table covers the same entry points
    for n in names:
        if not n.startswith("fp8gmm_"):
            assert n in G._SIGNATURES, n


def test_header_macros_match_binding():
    text = open(G.HEADER_PATH).read()
    vals = {m: int(v) for m, v in re.findall(r"#define (FP8GMM_\w+) \(?(-?\d+)\)?", text)}
    assert vals["FP8GMM_ERR_NULL"] == G.ERR_NULL and vals["FP8GMM_ERR_HIP"] == G.ERR_HIP
    assert vals["FP8GMM_E4M3"] == G.E4M3 and vals["FP8GMM_E5M2"] == G.E5M2
    assert vals["FP8GMM_OP_TGMM"] == G.OP_TGMM and vals["FP8GMM_DEV_NEGATIVE_SIZE"] == G.DEV_NEGATIVE_SIZE
    assert vals["FP8GMM_OP_FFN_FWD"] == G.OP_FFN_FWD and vals["FP8GMM_OP_FFN_BWD"] == G.OP_FFN_BWD
    assert vals["FP8GMM_OP_FWD_VARIANT"] == G.OP_FWD_VARIANT and vals["FP8GMM_ACC_BF16"] == G.ACC_BF16
    assert vals["FP8GMM_LHS_SCALE_BF16"] == G.LHS_SCALE_BF16 and vals["FP8GMM_RHS_SCALE_FIRST"] == G.RHS_SCALE_FIRST
    assert vals["FP8GMM_ERR_SCRATCH"] == G.ERR_SCRATCH
    assert "#define FP8GMM_NOALLOC_SCRATCH_BYTES (32u << 20)" in text and G.NOALLOC_SCRATCH_BYTES == 32 << 20


P = 0x10000          # fake, 16-byte aligned "device" address; never dereferenced
BAD = 0x10008        # misaligned


def _fwd(L, lhs=P, codes=P, scale=P, gs=P, M=256, K=128, N=256, Gn=4, out=P, ws=P, wsb=1 << 30, fn="gmm_fp8_fwd",
         preact=None):
    extra = (preact,) if fn == "gmm_silu_fp8" else ()
    return getattr(L, fn)(lhs, codes, scale, gs, M, K, N, Gn, out, *extra, None, None, ws, wsb, None, None)


def test_forward_validation():
    L = _lib()
    for fn in ("gmm_fp8_fwd", "gmm_silu_fp8"):
        assert _fwd(L, lhs=None, fn=fn) == G.ERR_NULL
        assert _fwd(L, out=None, fn=fn) == G.ERR_NULL
        assert _fwd(L, M=-1, fn=fn) == G.ERR_SHAPE
        assert _fwd(L, M=1 << 24, fn=fn) == G.ERR_SHAPE
        assert _fwd(L, K=0, fn=fn) == G.ERR_SHAPE
        assert _fwd(L, Gn=0, fn=fn) == G.ERR_SHAPE
        assert _fwd(L, K=100, fn=fn) == G.ERR_UNSUPPORTED
        assert _fwd(L, N=200, fn=fn) == G.ERR_UNSUPPORTED
        assert _fwd(L, K=16384 + 128, fn=fn) == G.ERR_UNSUPPORTED
        assert _fwd(L, Gn=1025, fn=fn) == G.ERR_UNSUPPORTED
        assert _fwd(L, lhs=BAD, fn=fn) == G.ERR_ALIGN
        assert _fwd(L, ws=None, fn=fn) == G.ERR_WORKSPACE
        need = L.fp8gmm_workspace_bytes(G.OP_FWD, 256, 128, 256, 4, 512)
        assert need >= 256 * 128 + 256 * 4
        assert _fwd(L, wsb=need - 1, fn=fn) == G.ERR_WORKSPACE
        assert _fwd(L, M=0, ws=None, wsb=0, fn=fn) == G.OK          # empty buffer: a no-op
    assert _fwd(L, N=384, fn="gmm_silu_fp8") == G.ERR_UNSUPPORTED   # I = 192 is not a multiple of 128
    assert _fwd(L, preact=BAD, fn="gmm_silu_fp8") == G.ERR_ALIGN


def test_dswiglu_and_ffn_validation():
    L = _lib()
    dsw = lambda **kw: L.gmm_dswiglu_fp8(kw.get("dout", P), P, P, P, kw.get("pre", P), kw.get("M", 64),
                                         kw.get("K", 256), 512, 2, kw.get("out", P), None, None)
    assert dsw(pre=None) == G.ERR_NULL
    assert dsw(out=None) == G.ERR_NULL
    assert dsw(M=0, pre=None, out=None, dout=None) == G.OK
    assert dsw(K=192) == G.ERR_UNSUPPORTED
    assert dsw(pre=BAD) == G.ERR_ALIGN
    assert dsw(M=-1) == G.ERR_SHAPE
    fwd = lambda **kw: L.moe_ffn_fp8_fwd(kw.get("x", P), P, P, P, P, P, kw.get("M", 64), kw.get("H", 512),
                                         kw.get("I", 256), 2, P, kw.get("pre", P), P, kw.get("ws", P),
                                         kw.get("wsb", 1 << 30), None, None)
    assert fwd(x=None) == G.ERR_NULL
    assert fwd(H=192) == G.ERR_UNSUPPORTED               # every size a multiple of 128
    assert fwd(I=64) == G.ERR_UNSUPPORTED
    assert fwd(pre=BAD) == G.ERR_ALIGN
    assert fwd(ws=None) == G.ERR_WORKSPACE
    need = L.fp8gmm_workspace_bytes(G.OP_FFN_FWD, 64, 512, 256, 2, 0)
    assert need >= 64 * 512 + 64 * 4
    assert fwd(wsb=need - 1) == G.ERR_WORKSPACE
    assert fwd(M=0, x=None, ws=None, wsb=0) == G.OK
    bwd = lambda **kw: L.moe_ffn_fp8_bwd(P, P, kw.get("pre", P), P, P, P, P, P, P, kw.get("M", 64), 512, 256, 2,
                                         kw.get("gd", G.E5M2), P, kw.get("dx", P), kw.get("dwi", P), P,
                                         kw.get("ws", P), kw.get("wsb", 1 << 30), None, None)
    assert bwd(pre=None) == G.ERR_NULL
    assert bwd(dwi=None) == G.ERR_NULL
    assert bwd(gd=3) == G.ERR_UNSUPPORTED
    assert bwd(dx=BAD) == G.ERR_ALIGN
    assert bwd(ws=None) == G.ERR_WORKSPACE
    need = L.fp8gmm_workspace_bytes(G.OP_FFN_BWD, 64, 512, 256, 2, 512)
    assert need >= L.fp8gmm_workspace_bytes(G.OP_TGMM, 64, 512, 512, 2, 512)
    assert bwd(wsb=need - 1) == G.ERR_WORKSPACE
    assert L.fp8gmm_workspace_bytes(G.OP_FFN_BWD, 64, 512, 256, 2, 256) == 0


def test_variant_validation():
    L = _lib()
    v = lambda **kw: L.gmm_fp8_fwd_variant(P, P, P, P, kw.get("M", 256), kw.get("K", 1024), 256, 4,
                                           kw.get("blk", 512), kw.get("flags", 3), kw.get("out", P), None, None,
                                           kw.get("ws", P), kw.get("wsb", 1 << 30), None, None)
    assert v(blk=256) == G.ERR_UNSUPPORTED
    assert v(flags=8) == G.ERR_UNSUPPORTED
    assert v(out=None) == G.ERR_NULL
    assert v(out=BAD) == G.ERR_ALIGN
    assert v(ws=None) == G.ERR_WORKSPACE
    need = L.fp8gmm_workspace_bytes(G.OP_FWD_VARIANT, 256, 1024, 256, 4, 512)
    assert need >= 256 * 1024 + 256 * 2 * 4
    assert v(wsb=need - 1) == G.ERR_WORKSPACE
    assert L.fp8gmm_workspace_bytes(G.OP_FWD_VARIANT, 256, 1024, 256, 4, 256) == 0


def test_dense_validation():
    L = _lib()
    dn = lambda **kw: L.tgmm_dense_quant(kw.get("lhs", P), P, P, kw.get("M", 1024), kw.get("K", 256), 128, 3,
                                         kw.get("gd", G.E5M2), kw.get("drhs", P), None, None, kw.get("ws", P),
                                         kw.get("wsb", 1 << 30), None, None)
    assert dn(lhs=None) == G.ERR_NULL
    assert dn(drhs=None) == G.ERR_NULL
    assert dn(gd=5) == G.ERR_UNSUPPORTED
    assert dn(K=192) == G.ERR_UNSUPPORTED
    assert dn(ws=None) == G.ERR_WORKSPACE
    need = L.fp8gmm_workspace_bytes(G.OP_TGMM_DENSE, 1024, 256, 128, 3, 0)
    assert need > L.fp8gmm_workspace_bytes(G.OP_TGMM, 1024, 256, 128, 3, 512) + 1024 * (256 + 128)
    assert dn(wsb=need - 1) == G.ERR_WORKSPACE


def test_dlhs_and_tgmm_validation():
    L = _lib()
    assert L.gmm_dlhs_fp8(None, P, P, P, 8, 128, 128, 2, P, P, 1 << 20, None, None) == G.ERR_NULL
    assert L.gmm_dlhs_fp8(P, P, P, P, -1, 128, 128, 2, P, P, 1 << 20, None, None) == G.ERR_SHAPE
    assert L.gmm_dlhs_fp8(P, P, P, P, 8, 100, 128, 2, P, P, 1 << 20, None, None) == G.ERR_UNSUPPORTED
    assert L.gmm_dlhs_fp8(P, P, P, P, 8, 128, 128, 2, BAD, P, 1 << 20, None, None) == G.ERR_ALIGN
    args = lambda **kw: [kw.get("lhs", P), kw.get("dout", P), P, kw.get("M", 1024), 256, 128, 3,
                         kw.get("gd", G.E5M2), kw.get("tm", 512), kw.get("drhs", P), None, None,
                         kw.get("ws", P), kw.get("wsb", 1 << 30), None, None]
    assert L.tgmm_quant(*args(lhs=None)) == G.ERR_NULL
    assert L.tgmm_quant(*args(drhs=None)) == G.ERR_NULL
    assert L.tgmm_quant(*args(gd=7)) == G.ERR_UNSUPPORTED
    assert L.tgmm_quant(*args(tm=256)) == G.ERR_UNSUPPORTED
    assert L.tgmm_quant(*args(M=-3)) == G.ERR_SHAPE
    assert L.tgmm_quant(*args(dout=BAD)) == G.ERR_ALIGN
    assert L.tgmm_quant(*args(ws=None)) == G.ERR_WORKSPACE


def test_dequant_validation():
    L = _lib()
    assert L.dequantize_fp8_codes(None, P, 2, 128, 128, P, None) == G.ERR_NULL
    assert L.dequantize_fp8_codes(P, P, 0, 128, 128, P, None) == G.ERR_SHAPE
    assert L.dequantize_fp8_codes(P, P, 2, 128, 24, P, None) == G.ERR_UNSUPPORTED
    assert L.dequantize_fp8_codes(P, P, 2, 128, 128, BAD, None) == G.ERR_ALIGN


def test_workspace_and_status_strings():
    L = _lib()
    assert L.fp8gmm_workspace_bytes(G.OP_FWD, 256, 100, 256, 4, 512) == 0      # rejected sizes
    assert L.fp8gmm_workspace_bytes(G.OP_SILU, 8192, 2048, 1536, 8, 512) >= 8192 * 2048
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert G.status_string(s) and G.status_string(s) != "unknown status"
    assert G.status_string(-99) == "unknown status"


def test_binding_rejects_cpu_tensors():
    import torch
    _lib()
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        G.gmm_fp8_fwd(x, torch.zeros((1, 128, 128), dtype=torch.uint8), torch.ones((1, 128)),
                      torch.tensor([4], dtype=torch.int32))


def test_product_path_does_not_import_oracle():
    for dirpath, _, files in os.walk(os.path.join(ROOT, "fp8_moe_grouped_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("no oracle", ""), os.path.join(dirpath, f)


def test_noalloc_validation():
    """The allocation-free forward rejects bad arguments, and inputs larger
    than its fixed scratch, on the host before any HIP call."""
    L = _lib()
    f = L.gmm_fp8_fwd_noalloc
    args = lambda **kw: [kw.get("lhs", P), kw.get("codes", P), P, P, kw.get("M", 4096), kw.get("K", 7168),
                         kw.get("N", 2048), 32, kw.get("out", P), None, None]
    assert f(*args(lhs=None)) == G.ERR_NULL
    assert f(*args(out=None)) == G.ERR_NULL
    assert f(*args(M=-1)) == G.ERR_SHAPE
    assert f(*args(K=100)) == G.ERR_UNSUPPORTED
    assert f(*args(codes=BAD)) == G.ERR_ALIGN
    # 4096 rows of K = 7168 fit the 32 MiB scratch (codes + row scales); 4682 rows do not
    assert 4096 * 7168 + 4096 * 4 <= G.NOALLOC_SCRATCH_BYTES < 4682 * 7168
    assert f(*args(M=4682)) == G.ERR_SCRATCH
    assert f(*args(M=1 << 20, K=128)) == G.ERR_SCRATCH
