"""GPU parity of the forward's LHS-quantization variants (gmm_fp8_fwd_variant)
against the oracle's gmm_fwd_variant: codes and scales bit-exact, outputs
within the forward's bound; with the bf16 accumulator each of the nb folds
may round one bf16 ulp differently (the f32 partial sums differ in order), so
the bound adds the ulp of every running total the oracle reports."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gmm as O
from tests.parity import C_ACC_FP8, bf16_np, check_bf16

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA1


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def run_variant(d, **kw):
    import fp8_moe_grouped_amd as G
    M, N = d["lhs"].shape[0], d["codes"].shape[2]
    out = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out, codes, scales = G.gmm_fp8_fwd_variant(dev(d["lhs"]), dev(d["codes"]), dev(d["scale"]),
                                               dev(d["group_sizes"]), out=out, debug=True, **kw)
    torch.cuda.synchronize()
    return bf16_np(out), codes.cpu().numpy(), scales.cpu().numpy()


def check_variant(d, rows=None, **kw):
    got, codes, scales = run_variant(d, **kw)
    okw = dict(block=kw.get("lhs_block", 0), scale_bf16=kw.get("scale_bf16", False),
               acc_bf16=kw.get("acc_bf16", False) and kw.get("lhs_block", 0) == 512,
               rhs_scale_first=kw.get("rhs_scale_first", False))
    res = O.gmm_fwd_variant(d["lhs"], d["codes"], d["scale"], d["group_sizes"], rows=rows, **okw)
    assert np.array_equal(codes[res.rows], res.act_codes), "codes differ"
    assert np.array_equal(scales[res.rows], res.act_scale), "scales differ"
    extra = F.ulp_bf16(np.abs(res.totals)).sum(axis=0) if okw["acc_bf16"] else None
    err = check_bf16(got[res.rows], res.out_f64, res.absum, res.group, C_ACC_FP8, f"variant {kw}", extra_tol=extra)
    mv = O.layout(d["group_sizes"], d["lhs"].shape[0]).valid
    assert np.all(got[mv:] == SENTINEL)
    return err, res


def test_default_variant_is_the_forward():
    import fp8_moe_grouped_amd as G
    d = W.make(2, "wo")
    got, _, _ = run_variant(d)
    ref = G.gmm_fp8_fwd(dev(d["lhs"]), dev(d["codes"]), dev(d["scale"]), dev(d["group_sizes"]))
    torch.cuda.synchronize()
    mv = int(d["group_sizes"].sum())
    assert np.array_equal(got[:mv], bf16_np(ref)[:mv])


VARIANTS = [dict(rhs_scale_first=True), dict(scale_bf16=True), dict(lhs_block=512),
            dict(lhs_block=512, scale_bf16=True), dict(lhs_block=512, acc_bf16=True),
            dict(lhs_block=512, scale_bf16=True, acc_bf16=True),
            dict(lhs_block=512, scale_bf16=True, acc_bf16=True, rhs_scale_first=True)]


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda k: "-".join(f"{a}={b}" for a, b in k.items()))
def test_variants_config2(kw):
    """wo shape (K = 768: a full and a partial 512-column block), every row."""
    err, _ = check_variant(W.make(2, "wo"), **kw)
    print(f"{kw}: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


def test_block512_bf16_config3_sampled_rows():
    """K = 7168 (14 blocks) on the dropless buffer, sampled rows."""
    d = W.make(3, "wi")
    d = dict(d, codes=np.ascontiguousarray(d["codes"][:, :, :1024]), scale=np.ascontiguousarray(d["scale"][:, :1024]))
    lay = O.layout(d["group_sizes"], d["M"])
    rows = np.unique(np.concatenate([[lay.start[g], lay.end[g] - 1] for g in range(d["G"]) if lay.end[g] > lay.start[g]]
                                    + [np.random.default_rng(1).choice(lay.valid, 64, replace=False)]))
    err, _ = check_variant(d, rows=rows, lhs_block=512, scale_bf16=True, acc_bf16=True)
    print(f"config3 block-512 bf16: normwise {err[0]:.2e}, ratio {err[1]:.3f}")


def test_variant_distances_config3():
    """K = 7168 (the dropless wi input, first 1024 output columns, sampled
    rows): the distances of fake QAT and of the block-512 bf16 mode to the
    full-K f32 forward, from the GPU outputs, match the oracle's, and fake QAT
    is the nearer (the pages' ordering; with K <= 1024, i.e. two blocks or
    fewer, the block-512 codes share most scales with the full-K ones and the
    order reverses)."""
    d = W.make(3, "wi")
    d = dict(d, codes=np.ascontiguousarray(d["codes"][:, :, :1024]), scale=np.ascontiguousarray(d["scale"][:, :1024]))
    rows = np.sort(np.random.default_rng(2).choice(O.layout(d["group_sizes"], d["M"]).valid, 160, replace=False))
    exact = O.fake_qat_reference(d["lhs"], d["codes"], d["scale"], d["group_sizes"], rows=rows)
    fake = F.bf16_to_f64(F.f64_to_bf16_bits(exact))
    full, _, _ = run_variant(d)
    b512, _, _ = run_variant(d, lhs_block=512, scale_bf16=True, acc_bf16=True)
    f, b = F.bf16_to_f64(full[rows]), F.bf16_to_f64(b512[rows])
    of = F.bf16_to_f64(O.gmm_fwd_variant(d["lhs"], d["codes"], d["scale"], d["group_sizes"], rows=rows).out)
    ob = F.bf16_to_f64(O.gmm_fwd_variant(d["lhs"], d["codes"], d["scale"], d["group_sizes"], rows=rows, block=512,
                                         scale_bf16=True, acc_bf16=True).out)
    dist = lambda a, r: np.linalg.norm(a - r) / np.linalg.norm(r)
    g_fake, g_b = dist(fake, f), dist(b, f)
    o_fake, o_b = dist(fake, of), dist(ob, of)
    print(f"to the full-K f32 forward: fake QAT {g_fake:.4f} (oracle {o_fake:.4f}), block-512 bf16 {g_b:.4f} "
          f"(oracle {o_b:.4f}); to the exact product: full-K {dist(f, exact):.4f}, block-512 bf16 {dist(b, exact):.4f}")
    assert abs(g_fake - o_fake) < 0.05 * o_fake and abs(g_b - o_b) < 0.05 * o_b
    assert g_fake < g_b
