"""GPU parity at the limits the C ABI accepts: 1024 experts (most of them
empty), K = 16384 (the row quantizer's limit) and the largest static buffer,
2^24 - 1 rows, whose 32-bit row offsets sit at the edge.  Inputs are seeded
(the largest buffer is drawn on the device by torch's seeded generator and
copied to the host for the oracle, which checks sampled rows)."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gmm as O
from tests.parity import C_ACC_FP8, bf16_np, check_bf16, check_f32

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA1


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _codes(r, G, K, N):
    w = r.standard_normal((G, K, N)).astype(np.float32) * 0.02
    scale = (np.abs(w).max(axis=1) / 448).astype(np.float32)
    codes = torch.from_numpy(np.clip(w / scale[:, None, :], -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_1024_experts_forward_dlhs_tgmm():
    import fp8_moe_grouped_amd as G
    r = np.random.default_rng(1024)
    Gn, M, K, N = 1024, 4096, 256, 128
    gs = np.zeros(Gn, np.int32)
    live = r.choice(Gn, 300, replace=False)
    gs[live] = r.multinomial(M - 200, np.ones(300) / 300)       # 200 stale rows
    codes, scale = _codes(r, Gn, K, N)
    lhs = _bf16(r.standard_normal((M, K)))
    dout = _bf16(r.standard_normal((M, N)) * 1e-3)
    mv = int(gs.sum())
    lhs[mv:] = 0x7F80
    dout[mv:] = 0xFF80
    out = G.gmm_fp8_fwd(dev(lhs), dev(codes), dev(scale), dev(gs))
    dl = G.gmm_dlhs_fp8(dev(dout), dev(codes), dev(scale), dev(gs))
    lt = _bf16(r.standard_normal((M, K)))
    lt[mv:] = 0x7FC0
    tg = G.tgmm_quant(dev(lt), dev(dout), dev(gs), "e5m2")
    torch.cuda.synchronize()
    res = O.gmm_fwd(lhs, codes, scale, gs)
    check_bf16(bf16_np(out)[res.rows], res.y, res.absum, res.group, C_ACC_FP8, "forward, 1024 experts")
    rd = O.gmm_dlhs(dout, codes, scale, gs)
    check_bf16(bf16_np(dl)[rd.rows], rd.y, rd.absum, rd.group, N * 2.0 ** -24, "dLHS, 1024 experts")
    rt = O.tgmm_quant(lt, dout, gs, "e5m2")
    check_f32(tg.cpu().numpy(), rt.drhs_f64, rt.absum, None, np.maximum(gs, 0), "tgmm, 1024 experts")


def test_k16384_forward():
    """The row quantizer's largest K (one wave holds 16384 bf16 per row)."""
    import fp8_moe_grouped_amd as G
    r = np.random.default_rng(16384)
    Gn, M, K, N = 3, 600, 16384, 256
    gs = np.array([250, 0, 300], np.int32)
    codes, scale = _codes(r, Gn, K, N)
    x = r.standard_normal((M, K)).astype(np.float32)
    x[r.random((M, K)) < 0.01] *= 50
    lhs = _bf16(x)
    lhs[550:] = 0x7F80
    out, qc, qs = G.gmm_fp8_fwd(dev(lhs), dev(codes), dev(scale), dev(gs), debug=True)
    torch.cuda.synchronize()
    res = O.gmm_fwd(lhs, codes, scale, gs)
    assert np.array_equal(qc.cpu().numpy()[res.rows], res.act_codes)
    assert np.array_equal(qs.cpu().numpy()[res.rows], res.act_scale)
    check_bf16(bf16_np(out)[res.rows], res.y, res.absum, res.group, C_ACC_FP8, "forward, K=16384")


def test_largest_static_buffer():
    """M = 2^24 - 1 rows (the largest the ABI accepts), K = N = 128, four
    experts and a 1000-row garbage tail: forward and dLHS on every row; the
    oracle checks the first and last rows of every expert and rows near the
    top of the buffer."""
    import fp8_moe_grouped_amd as G
    M, K, N, Gn = (1 << 24) - 1, 128, 128, 4
    valid = M - 1000
    q = valid // 4
    gs = np.array([q, q + 7, q - 7, valid - 3 * q], np.int32)
    r = np.random.default_rng(24)
    codes, scale = _codes(r, Gn, K, N)
    g = torch.Generator(device="cuda").manual_seed(24)
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    d = (torch.randn((M, N), generator=g, device="cuda") * 1e-3).to(torch.bfloat16)
    x[valid:] = float("inf")
    d[valid:] = float("nan")
    out = G.gmm_fp8_fwd(x, dev(codes), dev(scale), dev(gs))
    dl = G.gmm_dlhs_fp8(d, dev(codes), dev(scale), dev(gs))
    torch.cuda.synchronize()
    lhs_h, dout_h = bf16_np(x), bf16_np(d)
    lay = O.layout(gs, M)
    rows = np.unique(np.concatenate([[lay.start[e], lay.end[e] - 1] for e in range(Gn)] +
                                    [np.arange(valid - 64, valid), r.choice(valid, 64, replace=False)]))
    res = O.gmm_fwd(lhs_h, codes, scale, gs, rows=rows)
    got = bf16_np(out)
    check_bf16(got[rows], res.y, res.absum, res.group, C_ACC_FP8, "forward, 2^24-1 rows")
    rd = O.gmm_dlhs(dout_h, codes, scale, gs, rows=rows)
    check_bf16(bf16_np(dl)[rows], rd.y, rd.absum, rd.group, N * 2.0 ** -24, "dLHS, 2^24-1 rows")
