"""GPU parity of the buffer-wide backward quantization baseline
(tgmm_dense_quant) against the oracle's tgmm_dense, and the failure it
exhibits on a buffer with a garbage tail (the in-kernel tgmm_quant on the
same buffer stays finite)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gmm as O
from tests.parity import check_f32

pytestmark = pytest.mark.gpu


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def run_dense(lhs, dout, gs, grad):
    import fp8_moe_grouped_amd as G
    out, srow, scol = G.tgmm_dense_quant(dev(lhs), dev(dout), dev(np.asarray(gs, np.int32)), grad, debug=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), srow.cpu().numpy(), scol.cpu().numpy()


@pytest.mark.parametrize("grad", ["e5m2", "e4m3"])
def test_dense_small_clean_tail(grad):
    """Stale rows zero: the result is finite and matches the oracle."""
    d = W.ffn("small")
    gs, mv = d["group_sizes"], d["valid"]
    x, dy = d["x"].copy(), d["dy"].copy()
    x[mv:] = 0
    dy[mv:] = 0
    got, srow, scol = run_dense(x, dy, gs, grad)
    res = O.tgmm_dense(x, dy, gs, grad)
    assert np.array_equal(srow, res.sL[0]) and np.array_equal(scol, res.sD[0])
    rows = np.maximum(np.asarray(gs), 0)
    check_f32(got, res.drhs_f64, res.absum, None, rows, f"dense {grad}")


def test_dense_config4_clean_tail_sampled_columns():
    """The dropless buffer with its stale rows zeroed, full size on the GPU;
    the oracle checks 48 lhs columns x 48 gradient columns."""
    d = W.make(4, "tgmm")
    lhs, dout, gs, mv = d["lhs"].copy(), d["dout"].copy(), d["group_sizes"], d["valid"]
    lhs[mv:] = 0
    dout[mv:] = 0
    got, srow, scol = run_dense(lhs, dout, gs, "e5m2")
    r = np.random.default_rng(4)
    kc = np.sort(r.choice(d["K"], 48, replace=False))
    nc = np.sort(r.choice(d["N"], 48, replace=False))
    res = O.tgmm_dense(lhs, dout, gs, "e5m2", k_cols=kc, n_cols=nc)
    assert np.array_equal(srow, res.sL[0])
    assert np.array_equal(scol[nc], res.sD[0])
    check_f32(got[:, kc][:, :, nc], res.drhs_f64, res.absum, None, np.maximum(np.asarray(gs), 0), "dense config4")


def test_garbage_tail_poisons_dense_not_in_kernel():
    """The pages' failure on the dropless buffer with its Inf/NaN tail: every
    non-empty expert's gradient is NaN (empty experts stay zero) and every
    column scale is Inf, as the oracle predicts on the small buffer; the
    in-kernel tgmm_quant of the same buffer is finite."""
    import fp8_moe_grouped_amd as G
    d = W.make(4, "tgmm")
    gs = d["group_sizes"]
    got, srow, scol = run_dense(d["lhs"], d["dout"], gs, "e5m2")
    for g in range(len(gs)):
        if gs[g] > 0:
            assert np.isnan(got[g]).all(), g
        else:
            assert np.all(got[g] == 0), g
    assert np.isinf(scol).all()
    assert np.all(np.isfinite(srow[:d["valid"]])) and np.isinf(srow[d["valid"]:]).any()
    ink = G.tgmm_quant(dev(d["lhs"]), dev(d["dout"]), dev(gs), "e5m2")
    torch.cuda.synchronize()
    assert torch.isfinite(ink).all()
    # the oracle predicts the same pattern on the small FFN buffer (garbage tail)
    s = W.ffn("small")
    got_s, _, _ = run_dense(s["x"], s["dy"], s["group_sizes"], "e5m2")
    ref_s = O.tgmm_dense(s["x"], s["dy"], s["group_sizes"], "e5m2")
    assert np.array_equal(np.isnan(got_s), np.isnan(ref_s.drhs))
    assert np.array_equal(got_s[~np.isnan(got_s)], ref_s.drhs[~np.isnan(ref_s.drhs)])
