"""GPU parity of the fused wo dLHS + dSwiGLU (gmm_dswiglu_fp8), of the
pre-activation kept by gmm_silu_fp8, and of one routed-expert FFN forward +
backward (moe_ffn_fp8_fwd / moe_ffn_fp8_bwd) against the CPU oracle, through
the C ABI.

The FFN chain is compared stage by stage: each oracle stage is fed the GPU's
own upstream tensors (h, the pre-activation, d_preact), so every output is held
to the per-op rules (bf16: per-expert normwise 2e-3 plus the elementwise
bound; f32 weight gradients: 1e-5 relative Frobenius).  The FFN entry points
must also equal the individual calls bit for bit.
"""
import functools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gmm as O
from tests.parity import C_ACC_FP8, bf16_np, check_bf16, check_f32, dswiglu_tol, swiglu_tol

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA1


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def sentinel(rows, cols):
    return torch.full((rows, cols), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def bits(t):
    return t.view(torch.int16)


# ---------------------------------------------------------------- gmm_dswiglu_fp8

def run_dswiglu(d, gs=None):
    import fp8_moe_grouped_amd as G
    gs = d["group_sizes"] if gs is None else gs
    M, K = d["M"], d["K"]
    out = sentinel(M, 2 * K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    G.gmm_dswiglu_fp8(dev(d["dout"]), dev(d["codes"]), dev(d["scale"]), dev(np.asarray(gs, np.int32)),
                      dev(d["preact"]), out=out, dev_status=status)
    torch.cuda.synchronize()
    return bf16_np(out), int(status.item())


def check_dswiglu(d, rows=None):
    got, st = run_dswiglu(d)
    res = O.gmm_dswiglu(d["dout"], d["codes"], d["scale"], d["group_sizes"], d["preact"], rows=rows)
    pre = F.bf16_to_f64(d["preact"][res.rows])
    c_acc = d["N"] * 2.0 ** -24
    err = check_bf16(got[res.rows], res.y, np.zeros_like(res.y), res.group, 0.0, "dswiglu",
                     extra_tol=dswiglu_tol(res, pre, c_acc))
    assert np.all(got[d["valid"]:] == SENTINEL), "rows past the valid prefix were written"
    assert st == 0
    return err


@pytest.mark.parametrize("key", ["small", "small128"])
def test_dswiglu_small(key):
    """Ragged experts (one empty), a stale garbage tail, both column tilings
    (K = 256 and K = 128)."""
    err = check_dswiglu(W.dswiglu(key))
    print(f"dswiglu {key}: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


def test_dswiglu_config2():
    err = check_dswiglu(W.dswiglu(2))
    print(f"dswiglu config2: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


@functools.lru_cache(maxsize=None)
def _cfg3_dswiglu():
    """Inputs and GPU output of the config-3 fused dSwiGLU, computed once per session."""
    d = W.dswiglu(3)
    got, st = run_dswiglu(d)
    return d, got, st


DSWIGLU_CFG3_CHUNKS = 4


@pytest.mark.parametrize("chunk", range(DSWIGLU_CFG3_CHUNKS))
def test_dswiglu_config3_all_rows(chunk):
    """The dropless DeepSeek-V3-like shape (wo K = 2048, N = 7168, 19,661 of
    32,768 rows valid): every valid row against the oracle, a quarter per
    case, with the dSwiGLU elementwise bound."""
    d, got, st = _cfg3_dswiglu()
    assert st == 0
    lay = O.layout(d["group_sizes"], d["M"])
    rows = np.array_split(np.arange(lay.valid), DSWIGLU_CFG3_CHUNKS)[chunk]
    res = O.gmm_dswiglu(d["dout"], d["codes"], d["scale"], d["group_sizes"], d["preact"], rows=rows)
    pre = F.bf16_to_f64(d["preact"][res.rows])
    err = check_bf16(got[res.rows], res.y, np.zeros_like(res.y), res.group, 0.0, "dswiglu config3",
                     extra_tol=dswiglu_tol(res, pre, d["N"] * 2.0 ** -24))
    assert np.all(got[d["valid"]:] == SENTINEL), "rows past the valid prefix were written"
    print(f"dswiglu config3 rows {rows[0]}..{rows[-1]}: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


def test_dswiglu_carries_the_dlhs_bits():
    """With gate = 30 (sigma = 1 in f32, so silu'(gate) = 1 and silu(gate) =
    gate) and up = 1, d_gate = dh exactly: its bits must be gmm_dlhs_fp8's,
    and d_up = bf16(30 dh)."""
    import fp8_moe_grouped_amd as G
    d = W.dswiglu("small")
    M, K = d["M"], d["K"]
    pre = np.empty((M, 2 * K), np.uint16)
    pre[:, :K] = 0x41F0            # 30.0
    pre[:, K:] = 0x3F80            # 1.0
    d = dict(d, preact=pre)
    got, _ = run_dswiglu(d)
    dl = G.gmm_dlhs_fp8(dev(d["dout"]), dev(d["codes"]), dev(d["scale"]), dev(d["group_sizes"]))
    torch.cuda.synchronize()
    mv = d["valid"]
    ref = bf16_np(dl)[:mv]
    assert np.array_equal(got[:mv, :K], ref)
    dh = F.bf16_to_f64(ref)
    # d_up = bf16(30 dh_f32); bf16(dh) is within half an ulp of dh_f32, so
    # |d_up - 30 bf16(dh)| <= 30 ulp(dh) / 2 + ulp(30 dh) / 2 <= 1.5 ulp(30 dh)
    dup = F.bf16_to_f64(got[:mv, K:])
    assert np.all(np.abs(dup - 30 * dh) <= 1.5 * F.ulp_bf16(np.abs(30 * dh)) + 1e-30)


def test_dswiglu_empty_and_all_in_one_expert():
    d = W.dswiglu("small")
    got, st = run_dswiglu(d, gs=np.zeros(d["G"], np.int32))
    assert np.all(got == SENTINEL) and st == 0
    gs = np.array([0, 0, d["valid"], 0], np.int32)
    d1 = dict(d, group_sizes=gs)
    err = check_dswiglu(d1)
    print(f"dswiglu one expert: normwise {err[0]:.2e}")


# ---------------------------------------------------------------- pre-activation of gmm_silu_fp8

@pytest.mark.parametrize("config", [1, 3])
def test_silu_preact_is_plain_forward(config):
    """The pre-activation kept by gmm_silu_fp8 is gmm_fp8_fwd's result bit for
    bit, and keeping it leaves h unchanged."""
    import fp8_moe_grouped_amd as G
    d = W.make(config, "wi")
    lhs, codes, scale, gs = dev(d["lhs"]), dev(d["codes"]), dev(d["scale"]), dev(d["group_sizes"])
    M, N = d["lhs"].shape[0], d["codes"].shape[2]
    pre = sentinel(M, N)
    h1, _ = G.gmm_silu_fp8(lhs, codes, scale, gs, preact=pre)
    h0 = G.gmm_silu_fp8(lhs, codes, scale, gs)
    y = G.gmm_fp8_fwd(lhs, codes, scale, gs)
    qc, qs = G.quantize_rows_fp8(lhs, gs)
    pre_q = sentinel(M, N)
    h2 = G.gmm_silu_fp8_q(qc, qs, codes, scale, gs, preact=pre_q)
    torch.cuda.synchronize()
    mv = int(d["group_sizes"].sum())
    assert torch.equal(bits(pre[:mv]), bits(y[:mv]))
    assert torch.equal(bits(pre_q[:mv]), bits(y[:mv]))
    assert torch.equal(bits(h1[:mv]), bits(h0[:mv])) and torch.equal(bits(h2[:mv]), bits(h0[:mv]))
    assert torch.all(bits(pre[mv:]) == SENTINEL)


# ---------------------------------------------------------------- FFN forward + backward

def run_ffn(d, grad):
    import fp8_moe_grouped_amd as G
    M, H, I = d["M"], d["H"], d["I"]
    t = {k: dev(d[k]) for k in ("x", "wi_codes", "wi_scale", "wo_codes", "wo_scale", "group_sizes", "dy")}
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    h, pre, y = sentinel(M, I), sentinel(M, 2 * I), sentinel(M, H)
    G.moe_ffn_fp8_fwd(t["x"], t["wi_codes"], t["wi_scale"], t["wo_codes"], t["wo_scale"], t["group_sizes"],
                      h=h, preact=pre, y=y, dev_status=status)
    dz, dx = sentinel(M, 2 * I), sentinel(M, H)
    _, dwi, dwo, _ = G.moe_ffn_fp8_bwd(t["x"], h, pre, t["dy"], t["wi_codes"], t["wi_scale"], t["wo_codes"],
                                       t["wo_scale"], t["group_sizes"], grad, d_preact=dz, dx=dx,
                                       dev_status=status)
    torch.cuda.synchronize()
    return dict(h=h, preact=pre, y=y, d_preact=dz, dx=dx, dwi=dwi, dwo=dwo, status=int(status.item()), t=t)


def check_ffn_stages(d, out, grad, rows=None, cols=None):
    """Each stage of the chain against the oracle op fed with the GPU's own
    upstream tensors (so every stage sees exactly the inputs the kernel saw):
      1. wi forward (x): pre-activation and h, the forward's bf16 rule;
      2. wo forward of the GPU's h: the forward's bf16 rule;
      3. fused dSwiGLU of dy with the GPU's pre-activation: the bf16 rule with
         the dSwiGLU elementwise bound;
      4. wi dLHS of the GPU's d_preact: the dLHS bf16 rule;
      5. dwo = tgmm(GPU h, dy), dwi = tgmm(x, GPU d_preact): the f32 rule
         (1e-5 relative Frobenius overall and per expert, elementwise bound).
    ``rows`` restricts the row outputs (stages 1-4) to some valid rows and
    ``cols`` = (k, n) the weight gradients to some columns of each operand
    (every column's scale and codes depend on that column alone)."""
    gs, M, I, H = d["group_sizes"], d["M"], d["I"], d["H"]
    mv = d["valid"]
    sel = np.arange(mv) if rows is None else np.asarray(rows)
    h_g, pre_g, dz_g = bf16_np(out["h"]), bf16_np(out["preact"]), bf16_np(out["d_preact"])
    wi = O.gmm_fwd(d["x"], d["wi_codes"], d["wi_scale"], gs, swiglu_out=True, rows=sel)
    check_bf16(pre_g[sel], wi.y, wi.absum, wi.group, C_ACC_FP8, "ffn preact")
    check_bf16(h_g[sel], wi.out_f64, np.zeros_like(wi.out_f64), wi.group, C_ACC_FP8, "ffn h",
               extra_tol=swiglu_tol(wi, I))
    wo = O.gmm_fwd(h_g, d["wo_codes"], d["wo_scale"], gs, rows=sel)
    e_y = check_bf16(bf16_np(out["y"])[sel], wo.y, wo.absum, wo.group, C_ACC_FP8, "ffn y")
    dsw = O.gmm_dswiglu(d["dy"], d["wo_codes"], d["wo_scale"], gs, pre_g, rows=sel)
    e_dz = check_bf16(dz_g[sel], dsw.y, np.zeros_like(dsw.y), dsw.group, 0.0, "ffn d_preact",
                      extra_tol=dswiglu_tol(dsw, F.bf16_to_f64(pre_g[sel]), H * 2.0 ** -24))
    dx = O.gmm_dlhs(dz_g, d["wi_codes"], d["wi_scale"], gs, rows=sel)
    e_dx = check_bf16(bf16_np(out["dx"])[sel], dx.y, dx.absum, dx.group, 2 * I * 2.0 ** -24, "ffn dx")
    lay = O.layout(gs, M)
    per_group = np.minimum(lay.end - lay.start, 512)

    def grad_check(name, got, a_bits, b_bits, kn):
        kc, ncl = (None, None) if kn is None else kn
        ref = O.tgmm_quant(a_bits, b_bits, gs, grad, 512, k_cols=kc, n_cols=ncl)
        if kn is not None:
            got = got[:, torch.from_numpy(kc).cuda()][:, :, torch.from_numpy(ncl).cuda()]
        return check_f32(got.cpu().numpy(), ref.drhs_f64, ref.absum, None, per_group, name)

    e_wo = grad_check("ffn dwo", out["dwo"], h_g, d["dy"], None if cols is None else (cols[2], cols[3]))
    e_wi = grad_check("ffn dwi", out["dwi"], d["x"], dz_g, None if cols is None else (cols[0], cols[1]))
    for k in ("h", "preact", "y", "d_preact", "dx"):
        assert torch.all(bits(out[k][mv:]) == SENTINEL), f"{k}: rows past the valid prefix were written"
    return dict(y=e_y[0], d_preact=e_dz[0], dx=e_dx[0], dwo=e_wo[0], dwi=e_wi[0])


def _ffn_small(grad, key):
    d = W.ffn(key)
    out = run_ffn(d, grad)
    assert out["status"] == 0
    err = check_ffn_stages(d, out, grad)
    print(f"ffn {key} {grad}: " + ", ".join(f"{k} {v:.2e}" for k, v in err.items()))


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_ffn_small_against_oracle(grad):
    """Ragged experts (one empty) and a garbage tail."""
    _ffn_small(grad, "small")


def test_ffn_sizes_multiple_of_128():
    """H = 384, I = 128: multiples of 128 but not of 256 (the 128-row tgmm
    tiles, the cached-block dLHS of a 256-wide contraction)."""
    _ffn_small("e5m2", "small384")


@functools.lru_cache(maxsize=None)
def _ffn_run(key):
    """Inputs and GPU outputs of one FFN forward + backward (e5m2), once per session."""
    d = W.ffn(key)
    return d, run_ffn(d, "e5m2")


def test_ffn_config3_sampled_against_oracle():
    """The DeepSeek-V3-like dropless shape (H = 7168, I = 2048, 19,661 of
    32,768 rows valid): the stage-fed checks on the first and last rows of
    every non-empty expert plus a seeded sample, and on 64 x 64 sampled
    columns of both weight gradients."""
    d, out = _ffn_run(3)
    assert out["status"] == 0
    lay = O.layout(d["group_sizes"], d["M"])
    r = np.random.default_rng(5)
    edge = [r_ for g in range(d["G"]) if lay.end[g] > lay.start[g] for r_ in (lay.start[g], lay.end[g] - 1)]
    rows = np.unique(np.concatenate([edge, r.choice(lay.valid, 96, replace=False)]))
    H, I = d["H"], d["I"]
    cols = (np.sort(r.choice(H, 64, replace=False)), np.sort(r.choice(2 * I, 64, replace=False)),
            np.sort(r.choice(I, 64, replace=False)), np.sort(r.choice(H, 64, replace=False)))
    err = check_ffn_stages(d, out, "e5m2", rows=rows, cols=cols)
    print(f"ffn config3 ({len(rows)} rows): " + ", ".join(f"{k} {v:.2e}" for k, v in err.items()))


@pytest.mark.parametrize("key", ["small", 3])
def test_ffn_equals_individual_calls(key):
    """moe_ffn_fp8_fwd / _bwd give the individual calls' results bit for bit
    (the DeepSeek-V3-like dropless shape at full size)."""
    import fp8_moe_grouped_amd as G
    d, out = _ffn_run(key)
    t = out["t"]
    mv = d["valid"]
    h, pre = G.gmm_silu_fp8(t["x"], t["wi_codes"], t["wi_scale"], t["group_sizes"], preact=True)
    y = G.gmm_fp8_fwd(out["h"], t["wo_codes"], t["wo_scale"], t["group_sizes"])
    dz = G.gmm_dswiglu_fp8(t["dy"], t["wo_codes"], t["wo_scale"], t["group_sizes"], out["preact"])
    dx = G.gmm_dlhs_fp8(out["d_preact"], t["wi_codes"], t["wi_scale"], t["group_sizes"])
    dwo = G.tgmm_quant(out["h"], t["dy"], t["group_sizes"], "e5m2")
    dwi = G.tgmm_quant(t["x"], out["d_preact"], t["group_sizes"], "e5m2")
    torch.cuda.synchronize()
    for name, a, b in (("h", h, out["h"]), ("preact", pre, out["preact"]), ("y", y, out["y"]),
                       ("d_preact", dz, out["d_preact"]), ("dx", dx, out["dx"])):
        assert torch.equal(bits(a[:mv]), bits(b[:mv])), name
    assert torch.equal(dwo, out["dwo"]) and torch.equal(dwi, out["dwi"])
    assert torch.isfinite(out["dwi"]).all() and torch.isfinite(out["dwo"]).all()


def test_ffn_without_rows():
    """No valid rows: the row outputs stay untouched, the weight gradients are zeros."""
    d = W.ffn("small")
    d = dict(d, group_sizes=np.zeros(d["G"], np.int32))
    out = run_ffn(d, "e4m3")
    for k in ("h", "preact", "y", "d_preact", "dx"):
        assert torch.all(bits(out[k]) == SENTINEL), k
    assert torch.count_nonzero(out["dwi"]) == 0 and torch.count_nonzero(out["dwo"]) == 0
