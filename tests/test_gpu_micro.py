"""GPU parity of the FP8 forward at the pages' GMM kernel microbenchmark
shape: one call at full fill, 64 experts, 225,280 rows, wi 4096 -> 2x1024
(SwiGLU) and wo 1024 -> 4096.  Every row is computed on the GPU; the oracle
checks the first and last rows of eight experts and a seeded sample of their
rows (decoding every expert's weights on the CPU would take minutes)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import gmm as O
from tests.parity import C_ACC_FP8, bf16_np, check_bf16, swiglu_tol

pytestmark = pytest.mark.gpu


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("op", ["wi", "wo"])
def test_micro_forward_sampled(op):
    import fp8_moe_grouped_amd as G
    d = W.micro(op)
    swiglu = op == "wi"
    gs = d["group_sizes"]
    fn = G.gmm_silu_fp8 if swiglu else G.gmm_fp8_fwd
    out, codes, scales = fn(dev(d["lhs"]), dev(d["codes"]), dev(d["scale"]), dev(gs), debug=True)
    torch.cuda.synchronize()
    lay = O.layout(gs, d["M"])
    r = np.random.default_rng(7)
    experts = np.sort(r.choice(d["G"], 8, replace=False))
    rows = []
    for g in experts:
        a, b = int(lay.start[g]), int(lay.end[g])
        rows += [a, b - 1] + list(r.choice(np.arange(a, b), 14, replace=False))
    rows = np.unique(rows)
    res = O.gmm_fwd(d["lhs"], d["codes"], d["scale"], gs, swiglu_out=swiglu, rows=rows)
    got = bf16_np(out)
    assert np.array_equal(codes.cpu().numpy()[rows], res.act_codes)
    assert np.array_equal(scales.cpu().numpy()[rows], res.act_scale)
    I = d["N"] // 2
    err = check_bf16(got[rows], res.out_f64, res.absum if not swiglu else np.zeros_like(res.out_f64), res.group,
                     C_ACC_FP8, f"micro {op}", extra_tol=swiglu_tol(res, I) if swiglu else None)
    print(f"micro {op} ({len(rows)} rows): normwise {err[0]:.2e}, ratio {err[1]:.3f}")
