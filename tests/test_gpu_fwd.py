"""GPU parity of the native FP8 forward (gmm_fp8_fwd, gmm_silu_fp8) and of
dequantize_fp8_codes against the CPU oracle, through the C ABI."""
import functools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gmm as O
from tests.parity import C_ACC_FP8, bf16_np, check_bf16, swiglu_tol

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA1


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def sentinel(rows, cols):
    return torch.full((rows, cols), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def run_fwd(d, swiglu=False, group_sizes=None):
    import fp8_moe_grouped_amd as G
    gs = d["group_sizes"] if group_sizes is None else group_sizes
    M, N = d["lhs"].shape[0], d["codes"].shape[2]
    out = sentinel(M, N // 2 if swiglu else N)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    fn = G.gmm_silu_fp8 if swiglu else G.gmm_fp8_fwd
    out, codes, scales = fn(dev(d["lhs"]), dev(d["codes"]), dev(d["scale"]), dev(np.asarray(gs, np.int32)),
                            out=out, debug=True, dev_status=status)
    torch.cuda.synchronize()
    return bf16_np(out), codes.cpu().numpy(), scales.cpu().numpy(), int(status.item())


def check_fwd(d, swiglu, rows=None, group_sizes=None):
    gs = d["group_sizes"] if group_sizes is None else group_sizes
    out, codes, scales, status = run_fwd(d, swiglu, gs)
    res = O.gmm_fwd(d["lhs"], d["codes"], d["scale"], gs, swiglu_out=swiglu, rows=rows)
    mv = O.layout(gs, d["lhs"].shape[0]).valid
    assert np.array_equal(codes[res.rows], res.act_codes), "activation codes differ"
    assert np.array_equal(scales[res.rows], res.act_scale), "activation scales differ"
    I = d["codes"].shape[2] // 2
    extra = swiglu_tol(res, I) if swiglu else None
    err = check_bf16(out[res.rows], res.out_f64, res.absum if not swiglu else np.zeros_like(res.out_f64),
                     res.group, C_ACC_FP8, "forward", extra_tol=extra)
    assert np.all(out[mv:] == SENTINEL), "rows past the valid prefix were written"
    return err, status


# ---------------------------------------------------------------- configs 0-2

@pytest.mark.parametrize("variant", [None, "forced"])
def test_fwd_config0(variant):
    d = W.make(0, "fwd", variant)
    err, st = check_fwd(d, False)
    assert st == 0
    print(f"config0 {variant}: normwise {err[0]:.2e}, elementwise ratio {err[1]:.3f}")


def test_silu_small():
    d = W.make(0, "fwd")
    err, _ = check_fwd(d, True)
    print(f"swiglu small: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


@pytest.mark.parametrize("variant", [None, "balanced"])
def test_wi_config1(variant):
    d = W.make(1, "wi", variant)
    err, _ = check_fwd(d, True)
    print(f"config1 wi {variant}: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


def test_wo_config2():
    d = W.make(2, "wo")
    err, _ = check_fwd(d, False)
    print(f"config2 wo: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


# ---------------------------------------------------------------- config 3 (every valid row)

#: the valid rows of the dropless buffer are checked in contiguous chunks, so
#: that no single test spends more than a few tens of seconds in the oracle
CFG3_CHUNKS = {"wi": 6, "wo": 8}


@functools.lru_cache(maxsize=None)
def _cfg3_fwd(op):
    """Inputs and the GPU's outputs (bf16 result, activation codes and row
    scales) of one config-3 forward, computed once per session."""
    d = W.make(3, op)
    return (d,) + run_fwd(d, op == "wi")


@pytest.mark.parametrize("op,chunk", [(op, c) for op in ("wi", "wo") for c in range(CFG3_CHUNKS[op])])
def test_config3_all_rows(op, chunk):
    """The DeepSeek-V3-like dropless shape (19,661 of 32,768 rows valid,
    Zipf-skewed experts, garbage tail): every valid row's activation codes and
    scale bit for bit, and every output element against the bf16 rule."""
    d, out, codes, scales, st = _cfg3_fwd(op)
    assert st == 0
    lay = O.layout(d["group_sizes"], d["M"])
    rows = np.array_split(np.arange(lay.valid), CFG3_CHUNKS[op])[chunk]
    swiglu = op == "wi"
    res = O.gmm_fwd(d["lhs"], d["codes"], d["scale"], d["group_sizes"], swiglu_out=swiglu, rows=rows)
    assert np.array_equal(codes[rows], res.act_codes), "activation codes differ"
    assert np.array_equal(scales[rows], res.act_scale), "activation scales differ"
    extra = swiglu_tol(res, d["N"] // 2) if swiglu else None
    err = check_bf16(out[rows], res.out_f64, res.absum if not swiglu else np.zeros_like(res.out_f64),
                     res.group, C_ACC_FP8, f"config3 {op}", extra_tol=extra)
    assert np.all(out[lay.valid:] == SENTINEL), "rows past the valid prefix were written"
    print(f"config3 {op} rows {rows[0]}..{rows[-1]}: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


# ---------------------------------------------------------------- dequant

@pytest.mark.parametrize("config,op", [(0, "dequant"), (2, "dequant")])
def test_dequant_bit_exact(config, op):
    import fp8_moe_grouped_amd as G
    d = W.make(config, op)
    out = G.dequantize_fp8_codes(dev(d["codes"]), dev(d["scale"]))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_np(out), O.dequantize(d["codes"], d["scale"]))


@pytest.mark.parametrize("which", ["wi", "wo"])
def test_dequant_config3_bit_exact(which):
    """The dropless shape's weights (wi codes [32, 7168, 4096], wo codes
    [32, 2048, 7168]) dequantized in one call; every element against the
    oracle, expert by expert."""
    import fp8_moe_grouped_amd as G
    sh = W.SHAPES[3]
    K, N, stream = (sh["K_wi"], sh["N_wi"], W.W_WI) if which == "wi" else (sh["K_wo"], sh["N_wo"], W.W_WO)
    codes, scale = W.weights(3, stream, sh["G"], K, N)
    out = G.dequantize_fp8_codes(dev(codes), dev(scale))
    torch.cuda.synchronize()
    for g in range(sh["G"]):
        got = bf16_np(out[g])
        assert np.array_equal(got, O.dequantize(codes[g:g + 1], scale[g:g + 1])[0]), f"expert {g} differs"


def test_dequant_all_codes_and_scales():
    import fp8_moe_grouped_amd as G
    r = np.random.default_rng(3)
    codes = np.tile(np.arange(256, dtype=np.uint8), (2, 64, 1))          # [2, 64, 256], NaN codes included
    scale = (r.uniform(0.5, 2, (2, 256)) * 2.0 ** r.integers(-20, 10, (2, 256))).astype(np.float32)
    got = bf16_np(G.dequantize_fp8_codes(dev(codes), dev(scale)))
    ref = O.dequantize(codes, scale)
    nan = np.isnan(F.bf16_to_f64(ref))
    assert np.array_equal(np.isnan(F.bf16_to_f64(got)), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- edge cases

def _tiny(seed, M=300, K=256, N=256, G=5):
    r = np.random.default_rng(seed)
    lhs = W.to_bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    codes = np.empty((G, K, N), np.uint8)
    scale = np.empty((G, N), np.float32)
    for g in range(G):
        codes[g], scale[g] = W.weight_codes(r.standard_normal((K, N)).astype(np.float32) * 0.02)
    return dict(lhs=lhs, codes=codes, scale=scale)


def test_edge_all_empty():
    d = _tiny(1)
    out, _, _, st = run_fwd(d, False, [0, 0, 0, 0, 0])
    assert st == 0 and np.all(out == SENTINEL)


def test_edge_clamped_and_negative():
    d = _tiny(2)
    gs = [100, -5, 150, 80, 10]          # sum 340 > M = 300, one negative size
    err, st = check_fwd(d, False, group_sizes=gs)
    assert st == 3, st
    gs2 = [299, 0, 0, 0, 1]
    err, st = check_fwd(d, True, group_sizes=gs2)
    assert st == 0


def test_edge_small_groups_and_zero_rows():
    d = _tiny(3, M=70)
    d["lhs"][5] = 0                       # all-zero row: scale floor, zero codes
    d["lhs"][6, :] = 0x8000               # all -0.0
    gs = [1, 2, 0, 3, 64]
    check_fwd(d, False, group_sizes=gs)
    check_fwd(d, True, group_sizes=gs)


def test_edge_single_k_step_and_m0():
    import fp8_moe_grouped_amd as G
    d = _tiny(4, M=40, K=128, N=128)
    check_fwd(d, False, group_sizes=[10, 10, 10, 10, 0])
    z = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    out = G.gmm_fp8_fwd(z, dev(d["codes"]), dev(d["scale"]), dev(np.zeros(5, np.int32)))
    assert out.shape == (0, 128)


def test_stale_tail_garbage_is_never_read():
    d = _tiny(5, M=400)
    gs = [50, 70, 0, 60, 33]
    mv = sum(gs)
    a = dict(d); a["lhs"] = d["lhs"].copy(); a["lhs"][mv:] = 0
    b = dict(d); b["lhs"] = d["lhs"].copy(); W.fill_garbage(b["lhs"], mv)
    for swiglu in (False, True):
        oa = run_fwd(a, swiglu, gs)
        ob = run_fwd(b, swiglu, gs)
        assert np.array_equal(oa[0], ob[0]) and np.array_equal(oa[1][:mv], ob[1][:mv])
        assert np.isfinite(F.bf16_to_f64(ob[0][:mv])).all()


def test_quantizer_exhaustive_bf16():
    """Every finite bf16 value is quantized against 512 different row scales:
    each row holds its amax at column 0 and a slice of all bf16 values not
    larger than it; codes and scales must match the oracle bit for bit."""
    K = 8192
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_to_f64(allv)
    finite = allv[np.isfinite(vals)]
    r = np.random.default_rng(9)
    amax_bits = r.choice(finite[(F.bf16_to_f64(finite) > 0)], 512, replace=False)
    rows = []
    for ab in amax_bits:
        a = F.bf16_to_f64(np.array([ab]))[0]
        pool = finite[np.abs(F.bf16_to_f64(finite)) <= a]
        pool = pool[r.permutation(len(pool))][:4 * (K - 1)]
        for s in range(0, len(pool), K - 1):
            row = np.full(K, ab, np.uint16)
            chunk = pool[s:s + K - 1]
            row[1:1 + len(chunk)] = chunk
            rows.append(row)
    lhs = np.stack(rows)
    M = lhs.shape[0]
    codes = np.full((1, K, 128), 0x38, np.uint8)
    d = dict(lhs=lhs, codes=codes, scale=np.ones((1, 128), np.float32))
    _, qc, qs, _ = run_fwd(d, False, [M])
    x = F.bf16_to_f32(lhs)
    s = O.row_scales(x)
    assert np.array_equal(qs, s)
    assert np.array_equal(qc, O.quantize_rows(x, s))


@pytest.mark.parametrize("config,op", [(2, "wo"), (1, "wi")])
def test_split_forward_equals_fused(config, op):
    """quantize_rows_fp8 + gmm_*_q is the fused call, bit for bit."""
    import fp8_moe_grouped_amd as G
    d = W.make(config, op)
    lhs, codes, scale, gs = dev(d["lhs"]), dev(d["codes"]), dev(d["scale"]), dev(d["group_sizes"])
    fused_fn, q_fn = (G.gmm_silu_fp8, G.gmm_silu_fp8_q) if op == "wi" else (G.gmm_fp8_fwd, G.gmm_fp8_fwd_q)
    fused, fc, fs = fused_fn(lhs, codes, scale, gs, debug=True)
    qc, qs = G.quantize_rows_fp8(lhs, gs)
    split = q_fn(qc, qs, codes, scale, gs)
    torch.cuda.synchronize()
    mv = int(d["group_sizes"].sum())
    assert torch.equal(fused[:mv].view(torch.int16), split[:mv].view(torch.int16))
    assert torch.equal(fc[:mv], qc[:mv]) and torch.equal(fs[:mv], qs[:mv])


@pytest.mark.parametrize("G_,K,N", [(3, 37, 48), (2, 16, 1040), (1, 5, 16)])
def test_dequant_ragged_shapes(G_, K, N):
    """K not a multiple of 16 (rows of a block straddle experts) and a
    partial block of column chunks: still bit-exact against the oracle."""
    import fp8_moe_grouped_amd as G
    r = np.random.default_rng(K * 1000 + N)
    codes = r.integers(0, 256, (G_, K, N), dtype=np.uint8)
    scale = (r.uniform(0.5, 2, (G_, N)) * 2.0 ** r.integers(-12, 8, (G_, N))).astype(np.float32)
    got = bf16_np(G.dequantize_fp8_codes(dev(codes), dev(scale)))
    ref = O.dequantize(codes, scale)
    nan = np.isnan(F.bf16_to_f64(ref))
    assert np.array_equal(np.isnan(F.bf16_to_f64(got)), nan)
    assert np.array_equal(got[~nan], ref[~nan])
