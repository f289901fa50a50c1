"""GPU parity of the backward ops (gmm_dlhs_fp8, tgmm_quant) and of the bf16
measurement arm against the CPU oracle, through the C ABI."""
import functools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gmm as O
from tests.parity import bf16_np, check_bf16, check_f32

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA1


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def sentinel(rows, cols):
    return torch.full((rows, cols), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def run_dlhs(d, gs=None):
    import fp8_moe_grouped_amd as G
    gs = d["group_sizes"] if gs is None else gs
    M, K = d["dout"].shape[0], d["codes"].shape[1]
    out = sentinel(M, K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    G.gmm_dlhs_fp8(dev(d["dout"]), dev(d["codes"]), dev(d["scale"]), dev(np.asarray(gs, np.int32)), out=out,
                   dev_status=status)
    torch.cuda.synchronize()
    return out, int(status.item())


def check_dlhs(d, rows=None, gs=None):
    import fp8_moe_grouped_amd as G
    gs = d["group_sizes"] if gs is None else gs
    out, st = run_dlhs(d, gs)
    got = bf16_np(out)
    res = O.gmm_dlhs(d["dout"], d["codes"], d["scale"], gs, rows=rows)
    N = d["dout"].shape[1]
    err = check_bf16(got[res.rows], res.y, res.absum, res.group, N * 2.0 ** -24, "dlhs")
    mv = O.layout(gs, d["dout"].shape[0]).valid
    assert np.all(got[mv:] == SENTINEL), "rows past the valid prefix were written"
    # bit-identity with the bf16 main loop fed by the standalone dequantization
    w = G.dequantize_fp8_codes(dev(d["codes"]), dev(d["scale"]))
    ref = sentinel(*out.shape)
    G.gmm_bf16_dlhs(dev(d["dout"]), w, dev(np.asarray(gs, np.int32)), out=ref)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "dLHS tiles differ from dequantize_fp8_codes"
    return err, st


# ---------------------------------------------------------------- dLHS

def test_dlhs_config2():
    d = W.make(2, "dlhs_wo")
    err, st = check_dlhs(d)
    assert st == 0
    print(f"config2 dlhs: normwise {err[0]:.2e} ratio {err[1]:.3f}")


def test_dlhs_config0_shape():
    d = W.make(0, "dlhs")             # K = 128: the narrow-tile path
    err, _ = check_dlhs(d)
    print(f"config0 dlhs: normwise {err[0]:.2e}")


#: config-3 dLHS rows are checked in contiguous chunks (each a few tens of
#: seconds of oracle time)
CFG3_CHUNKS = {"dlhs_wi": 6, "dlhs_wo": 4}


@functools.lru_cache(maxsize=None)
def _cfg3_dlhs(op):
    """Inputs and the GPU's result of one config-3 dLHS, computed once per session."""
    d = W.make(3, op)
    out, st = run_dlhs(d)
    return d, out, st


@pytest.mark.parametrize("op,chunk", [(op, c) for op in ("dlhs_wi", "dlhs_wo") for c in range(CFG3_CHUNKS[op])])
def test_dlhs_config3_all_rows(op, chunk):
    """The dropless shape: every valid row against the oracle (bf16 rule)."""
    d, out, st = _cfg3_dlhs(op)
    assert st == 0
    got = bf16_np(out)
    lay = O.layout(d["group_sizes"], d["M"])
    rows = np.array_split(np.arange(lay.valid), CFG3_CHUNKS[op])[chunk]
    res = O.gmm_dlhs(d["dout"], d["codes"], d["scale"], d["group_sizes"], rows=rows)
    err = check_bf16(got[rows], res.y, res.absum, res.group, d["N"] * 2.0 ** -24, f"config3 {op}")
    assert np.all(got[lay.valid:] == SENTINEL), "rows past the valid prefix were written"
    print(f"config3 {op} rows {rows[0]}..{rows[-1]}: normwise {err[0]:.2e} ratio {err[1]:.3f}")


@pytest.mark.parametrize("op", ["dlhs_wi", "dlhs_wo"])
def test_dlhs_config3_bit_identity(op):
    """The whole config-3 dLHS from the codes equals, bit for bit, the same
    main loop fed with dequantize_fp8_codes' bf16 weights: the on-chip tiles
    are the standalone dequantization."""
    import fp8_moe_grouped_amd as G
    d, out, _ = _cfg3_dlhs(op)
    w = G.dequantize_fp8_codes(dev(d["codes"]), dev(d["scale"]))
    ref = sentinel(*out.shape)
    G.gmm_bf16_dlhs(dev(d["dout"]), w, dev(d["group_sizes"]), out=ref)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "dLHS tiles differ from dequantize_fp8_codes"


def test_dlhs_edges_and_stale_tail():
    r = np.random.default_rng(4)
    G_, M, K, N = 5, 200, 256, 384
    codes = np.empty((G_, K, N), np.uint8)
    scale = np.empty((G_, N), np.float32)
    for g in range(G_):
        codes[g], scale[g] = W.weight_codes(r.standard_normal((K, N)).astype(np.float32) * 0.02)
    dout = W.to_bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    base = dict(codes=codes, scale=scale, dout=dout)
    gs = [0, 37, 1, 0, 90]
    mv = sum(gs)
    a = dict(base); a["dout"] = dout.copy(); a["dout"][mv:] = 0
    b = dict(base); b["dout"] = dout.copy(); W.fill_garbage(b["dout"], mv)
    check_dlhs(b, gs=gs)
    oa, _ = run_dlhs(a, gs)
    ob, _ = run_dlhs(b, gs)
    assert torch.equal(oa[:mv].view(torch.int16), ob[:mv].view(torch.int16))
    _, st = check_dlhs(base, gs=[150, -2, 100, 0, 0])
    assert st == 3


@pytest.mark.parametrize("N,K", [(128, 256), (256, 128), (512, 384), (640, 256)])
def test_dlhs_cached_block_boundaries(N, K):
    """Contractions on both sides of the cached-block limit: up to 512 a block
    decodes its 128 weight columns over the whole contraction once and keeps
    them in LDS for all its rows, beyond that the ring kernel decodes per
    stage.  The
    experts include one spanning several 2048-row chunks, an empty one, a
    single-row one and a ragged tail before a garbage tail; every row against
    the oracle and the whole result bit for bit against the bf16 main loop on
    dequantize_fp8_codes' output."""
    r = np.random.default_rng(N + K)
    G_, M = 5, 5200
    gs = [2600, 0, 1, 1700, 800]                  # 5101 valid rows, 99 stale
    codes = np.empty((G_, K, N), np.uint8)
    scale = np.empty((G_, N), np.float32)
    for g in range(G_):
        codes[g], scale[g] = W.weight_codes(r.standard_normal((K, N)).astype(np.float32) * 0.02)
    dout = W.to_bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    W.fill_garbage(dout, sum(gs))
    err, st = check_dlhs(dict(codes=codes, scale=scale, dout=dout), gs=gs)
    assert st == 0
    print(f"dlhs N={N} K={K}: normwise {err[0]:.2e} ratio {err[1]:.3f}")


@pytest.mark.parametrize("K", [2048, 1152])
def test_dlhs_skinny_groups(K):
    """Skinny groups (a buffer of at most 64 rows per expert on average):
    the 64-row tiles.  Mixed sizes: empty experts, single rows, experts that
    span two and three tiles, and a garbage tail; K = 1152 also takes the
    128-column tiles."""
    r = np.random.default_rng(21)
    G_, N = 32, 1024
    M = 64 * G_
    sizes = r.integers(0, 24, G_)
    sizes[[3, 17]] = 0
    sizes[5], sizes[9], sizes[30] = 1, 130, 64
    sizes = sizes.astype(np.int64)
    assert sizes.sum() < M
    codes = np.empty((G_, K, N), np.uint8)
    scale = np.empty((G_, N), np.float32)
    for g in range(G_):
        codes[g], scale[g] = W.weight_codes(r.standard_normal((K, N)).astype(np.float32) * 0.02)
    dout = W.to_bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    W.fill_garbage(dout, int(sizes.sum()))
    err, st = check_dlhs(dict(codes=codes, scale=scale, dout=dout), gs=sizes.tolist())
    assert st == 0
    print(f"skinny dlhs K={K}: normwise {err[0]:.2e} ratio {err[1]:.3f}")


# ---------------------------------------------------------------- bf16 forward arm

@pytest.mark.parametrize("config,N,silu", [(2, 2048, False), (0, 384, False), (1, 1536, True), (0, 256, True)])
def test_bf16_forward_arm(config, N, silu):
    """The bf16 arm (the FP8 forward's kernel on bf16 operands) against a
    float64 matmul of the same seeded bf16 inputs: 256-column tiles (N = 2048),
    128-column tiles (N = 384) and the SwiGLU epilogue."""
    import fp8_moe_grouped_amd as G
    d = W.make(config, "wo" if config == 2 else ("wi" if config == 1 else "fwd"))
    K = d["K"]
    w = W.bf16_weights(config, W.W_WO + 100, d["G"], K, N)
    out = sentinel(d["M"], N // 2 if silu else N)
    fn = G.gmm_bf16_silu if silu else G.gmm_bf16_fwd
    fn(dev(d["lhs"]), dev(w), dev(d["group_sizes"]), out=out)
    torch.cuda.synchronize()
    got = bf16_np(out)
    wd = F.bf16_to_f64(w)
    x = F.bf16_to_f64(d["lhs"])
    lay = O.layout(d["group_sizes"], d["M"])
    c_acc = K * 2.0 ** -24
    for g in range(d["G"]):
        a, b = lay.start[g], lay.end[g]
        if b == a:
            continue
        y = x[a:b] @ wd[g]
        absum = np.abs(x[a:b]) @ np.abs(wd[g])
        if not silu:
            check_bf16(got[a:b], y, absum, np.zeros(b - a, int), c_acc, "bf16 forward")
            continue
        I = N // 2
        gate, up = y[:, :I], y[:, I:]
        eg, eu = c_acc * absum[:, :I] + 2.0 ** -21 * np.abs(gate), c_acc * absum[:, I:] + 2.0 ** -21 * np.abs(up)
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-gate))
        extra = np.abs(sig * (1.0 + gate * (1.0 - sig))) * np.abs(up) * eg + np.abs(gate * sig) * eu \
            + 2.0 ** -19 * np.abs(gate * sig * up)
        check_bf16(got[a:b], O.swiglu(gate, up), np.zeros((b - a, I)), np.zeros(b - a, int), 0.0,
                   "bf16 swiglu", extra_tol=extra)
    assert np.all(got[lay.valid:] == SENTINEL)


# ---------------------------------------------------------------- tgmm

def run_tgmm(lhs, dout, gs, grad, debug=True, ws_out=None):
    """Runs tgmm_quant; with ``ws_out`` (a list) the operand code slabs the
    call left in its workspace are appended to it as host arrays (qL, qD)."""
    import fp8_moe_grouped_amd as G
    M, K = lhs.shape
    N = dout.shape[1]
    Gn = len(gs)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(G.workspace_bytes(G.OP_TGMM, M, K, N, Gn, 512), 1), dtype=torch.uint8, device="cuda")
    res = G.tgmm_quant(dev(lhs), dev(dout), dev(np.asarray(gs, np.int32)), grad, 512, debug=debug,
                       dev_status=status, workspace=ws)
    torch.cuda.synchronize()
    if ws_out is not None:
        ql, qd = G.tgmm_workspace_codes(ws, M, K, N, Gn)
        ws_out.extend([ql.cpu().numpy(), qd.cpu().numpy()])
    return res, int(status.item())


def check_tgmm_codes(lhs, dout, gs, grad, ql, qd, k_cols=None, n_cols=None):
    """Every non-empty (expert, tile) pair's operand codes in the workspace
    slabs equal the oracle's per-tile quantization bit for bit (the rows of
    the pair, then zero codes up to the next multiple of 32 rows); with
    k_cols / n_cols only those columns (a column's codes depend on that column
    alone).  Returns the number of pairs checked."""
    gfmt = F.E5M2 if grad == "e5m2" else F.E4M3
    kc = slice(None) if k_cols is None else k_cols
    nc = slice(None) if n_cols is None else n_cols
    tiles = O.tgmm_tiles(gs, lhs.shape[0], 512)
    for i, tl in enumerate(tiles):
        R = tl.row1 - tl.row0
        Rpad = -(-R // 32) * 32
        xl = F.bf16_to_f32(lhs[tl.row0:tl.row1][:, kc])
        xd = F.bf16_to_f32(dout[tl.row0:tl.row1][:, nc])
        qL = O.quantize_cols(xl, O.column_scales(xl, 448.0), F.E4M3)
        qD = O.quantize_cols(xd, O.column_scales(xd, F.FMAX[gfmt]), gfmt)
        assert np.array_equal(ql[i, :R][:, kc], qL), f"lhs codes of pair {i} (expert {tl.group}) differ"
        assert np.array_equal(qd[i, :R][:, nc], qD), f"{grad} gradient codes of pair {i} (expert {tl.group}) differ"
        assert not ql[i, R:Rpad][:, kc].any() and not qd[i, R:Rpad][:, nc].any(), f"pair {i}: padding rows not zero"
    return len(tiles)


def _tgmm_small(seed, M=1500, K=256, N=128):
    r = np.random.default_rng(seed)
    lhs = W.to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    dout = W.to_bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    return lhs, dout


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_tgmm_small_full(grad):
    lhs, dout = _tgmm_small(5)
    gs = [0, 300, 700, 0, 1, 400, 0]          # boundaries inside tiles, empty first/last experts
    slabs = []
    (drhs, sL, sD), st = run_tgmm(lhs, dout, gs, grad, ws_out=slabs)
    assert check_tgmm_codes(lhs, dout, gs, grad, *slabs) == 6
    ref = O.tgmm_quant(lhs, dout, gs, grad, 512)
    Tn = len(ref.tiles)
    assert np.array_equal(sL.cpu().numpy()[:Tn], ref.sL) and np.array_equal(sD.cpu().numpy()[:Tn], ref.sD)
    lay = O.layout(gs, lhs.shape[0])
    tot, per = check_f32(drhs.cpu().numpy(), ref.drhs_f64, ref.absum, None,
                         np.minimum(lay.end - lay.start, 512), f"tgmm {grad}")
    assert np.all(drhs.cpu().numpy()[[0, 3, 6]] == 0)
    print(f"tgmm small {grad}: rel fro {tot:.2e} (max per expert {per:.2e})")


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_tgmm_odd_multiples_of_128(grad):
    """K and N odd multiples of 128 (the smallest unit the ABI accepts):
    codes, scales and the f32 gradient against the oracle."""
    r = np.random.default_rng(384)
    M, K, N = 1300, 384, 640
    lhs = W.to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    dout = W.to_bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    gs = [513, 0, 200, 511]                       # expert boundaries inside and at tile edges, 76 stale rows
    W.fill_garbage(lhs, sum(gs))
    W.fill_garbage(dout, sum(gs))
    slabs = []
    (drhs, sL, sD), st = run_tgmm(lhs, dout, gs, grad, ws_out=slabs)
    assert st == 0
    n = check_tgmm_codes(lhs, dout, gs, grad, *slabs)
    ref = O.tgmm_quant(lhs, dout, gs, grad, 512)
    assert np.array_equal(sL.cpu().numpy()[:n], ref.sL) and np.array_equal(sD.cpu().numpy()[:n], ref.sD)
    lay = O.layout(gs, M)
    tot, per = check_f32(drhs.cpu().numpy(), ref.drhs_f64, ref.absum, None, np.minimum(lay.end - lay.start, 512),
                         f"tgmm {K}x{N} {grad}")
    print(f"tgmm {K}x{N} {grad}: {n} pairs, rel fro {tot:.2e}")


def test_tgmm_stale_tail_and_status():
    lhs, dout = _tgmm_small(6, M=1300)
    gs = [600, 0, 250]
    mv = sum(gs)
    la, da = lhs.copy(), dout.copy()
    la[mv:] = 0; da[mv:] = 0
    lb, db = lhs.copy(), dout.copy()
    W.fill_garbage(lb, mv); W.fill_garbage(db, mv)
    (a, _, _), _ = run_tgmm(la, da, gs, "e5m2")
    (b, _, _), _ = run_tgmm(lb, db, gs, "e5m2")
    assert torch.equal(a, b) and torch.isfinite(b).all()
    _, st = run_tgmm(lhs, dout, [1000, -1, 500], "e4m3")
    assert st == 3


@functools.lru_cache(maxsize=None)
def _cfg4_tgmm(grad):
    """Inputs, the GPU's gradient, scales and operand code slabs of the
    config-4 tgmm (computed once per session and gradient format)."""
    d = W.make(4, "tgmm")
    slabs = []
    (drhs, sL, sD), st = run_tgmm(d["lhs"], d["dout"], d["group_sizes"], grad, ws_out=slabs)
    return d, drhs, sL.cpu().numpy(), sD.cpu().numpy(), slabs[0], slabs[1], st


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_tgmm_config4_sampled(grad):
    """The dropless buffer (7168 x 2048 per expert): every scale of every
    (expert, tile) pair bit for bit, and the f32 gradient on 128 x 128 sampled
    (k, n) columns of every expert against the oracle's exact sums."""
    d, drhs, sL, sD, _, _, st = _cfg4_tgmm(grad)
    assert st == 0
    gfmt = F.E5M2 if grad == "e5m2" else F.E4M3
    tiles = O.tgmm_tiles(d["group_sizes"], d["M"], 512)
    for j, tl in enumerate(tiles):
        xl = F.bf16_to_f32(d["lhs"][tl.row0:tl.row1])
        xd = F.bf16_to_f32(d["dout"][tl.row0:tl.row1])
        assert np.array_equal(sL[j], O.column_scales(xl, 448.0)), f"sL of pair {j}"
        assert np.array_equal(sD[j], O.column_scales(xd, F.FMAX[gfmt])), f"sD of pair {j}"
    r = np.random.default_rng(7)
    kc = np.sort(r.choice(d["K"], 128, replace=False))
    nc = np.sort(r.choice(d["N"], 128, replace=False))
    ref = O.tgmm_quant(d["lhs"], d["dout"], d["group_sizes"], grad, 512, k_cols=kc, n_cols=nc)
    got = drhs[:, torch.from_numpy(kc).cuda()][:, :, torch.from_numpy(nc).cuda()].cpu().numpy()
    lay = O.layout(d["group_sizes"], d["M"])
    tot, per = check_f32(got, ref.drhs_f64, ref.absum, None, np.minimum(lay.end - lay.start, 512), "tgmm cfg4")
    empty = np.nonzero(np.asarray(d["group_sizes"]) == 0)[0]
    for g in empty:
        assert not torch.any(drhs[int(g)] != 0)
    assert torch.isfinite(drhs).all()
    print(f"tgmm config4 {grad}: {len(tiles)} pairs, rel fro {tot:.2e} (max per expert {per:.2e})")


CFG4_K_CHUNKS = 4


@pytest.mark.parametrize("grad,chunk", [(g_, c) for g_ in ("e5m2", "e4m3") for c in range(CFG4_K_CHUNKS)])
def test_tgmm_config4_all_columns(grad, chunk):
    """The dropless buffer: every element of the f32 gradient (a quarter of
    the k columns per case, all n columns, every expert) against the oracle,
    whose tile sums come from float64 products of the integer-valued codes
    here (within 512 * 2^-53 of the exact sums, pinned on the CPU)."""
    d, drhs, _, _, _, _, st = _cfg4_tgmm(grad)
    assert st == 0
    kc = np.array_split(np.arange(d["K"]), CFG4_K_CHUNKS)[chunk]
    ref = O.tgmm_quant(d["lhs"], d["dout"], d["group_sizes"], grad, 512, k_cols=kc, exact=False)
    got = drhs[:, int(kc[0]):int(kc[-1]) + 1].cpu().numpy()
    lay = O.layout(d["group_sizes"], d["M"])
    tot, per = check_f32(got, ref.drhs_f64, ref.absum, None, np.minimum(lay.end - lay.start, 512),
                         f"tgmm cfg4 k {kc[0]}..{kc[-1]}")
    print(f"tgmm config4 {grad} k {kc[0]}..{kc[-1]}: rel fro {tot:.2e} (max per expert {per:.2e})")


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_tgmm_config4_codes(grad):
    """The dropless buffer: the lhs and gradient codes of every (expert, tile)
    pair, every row and column, bit for bit against the oracle."""
    d, _, _, _, ql, qd, _ = _cfg4_tgmm(grad)
    n = check_tgmm_codes(d["lhs"], d["dout"], d["group_sizes"], grad, ql, qd)
    print(f"tgmm config4 {grad}: codes of {n} pairs bit-exact")


@pytest.mark.parametrize("cfg,K,N", [(4, 7168, 2048), (3, 7168, 4096), (3, 384, 2048), (2, 2048, 768)])
def test_tgmm_item_deal(cfg, K, N):
    """The GEMM's work-item deal that the prep pass writes into the workspace
    equals the host model's (tests/tgmm_deal.py), integer for integer, for both
    GEMM geometries (256-row k tiles one block per CU, 128-row two)."""
    import fp8_moe_grouped_amd as G
    from tests import tgmm_deal as D
    gs = np.asarray(W.group_sizes(cfg), np.int32)
    M, Gn = int(W.SHAPES[cfg]["M"]), len(gs)
    lhs = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    dout = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(G.workspace_bytes(G.OP_TGMM, M, K, N, Gn, 512), dtype=torch.uint8, device="cuda")
    G.tgmm_quant(lhs, dout, dev(gs), "e5m2", 512, workspace=ws)
    torch.cuda.synchronize()
    got = G.tgmm_workspace_deal(ws, M, K, N, Gn).cpu().numpy().tolist()
    want = D.deal(gs, M, K, N, torch.cuda.get_device_properties(0).multi_processor_count)
    assert want is not None and got == want


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_tgmm_every_code(grad):
    """Every finite code of both operands passes through the GEMM: row 0 holds
    the format's largest value in every column, so each tile-channel scale is
    exactly 1 and each other entry (an exactly representable 8-bit value)
    quantizes to its own code; the result is compared with the oracle."""
    M, K, N = 512, 256, 128
    gfmt = F.E5M2 if grad == "e5m2" else F.E4M3

    def column_block(fmt, cols, shift):
        codes = np.array([c for c in range(256) if np.isfinite(F.DECODE[fmt][c])], np.uint8)
        idx = (np.arange(M - 1)[:, None] * 7 + np.arange(cols)[None, :] * shift) % len(codes)
        vals = F.DECODE[fmt][codes[idx]]
        top = np.full((1, cols), F.DECODE[fmt][F.MAX_CODE[fmt]])
        return F.f64_to_bf16_bits(np.vstack([top, vals])), len(codes)

    lhs, nl = column_block(F.E4M3, K, 3)
    dout, nd = column_block(gfmt, N, 5)
    assert nl == 254 and nd == (248 if grad == "e5m2" else 254)
    slabs = []
    (drhs, sL, sD), st = run_tgmm(lhs, dout, [M], grad, ws_out=slabs)
    assert st == 0
    assert check_tgmm_codes(lhs, dout, [M], grad, *slabs) == 1
    ref = O.tgmm_quant(lhs, dout, [M], grad, 512)
    assert np.all(ref.sL == 1.0) and np.all(ref.sD == 1.0)
    assert np.array_equal(sL.cpu().numpy()[:1], ref.sL) and np.array_equal(sD.cpu().numpy()[:1], ref.sD)
    tot, per = check_f32(drhs.cpu().numpy(), ref.drhs_f64, ref.absum, None, np.array([M]), f"tgmm codes {grad}")
    print(f"tgmm every code {grad}: rel fro {tot:.2e}")
