"""Pins of the oracle's SwiGLU derivative, fused wo dLHS + dSwiGLU and MoE FFN
forward/backward (oracle/gmm.py: dswiglu, gmm_dswiglu, moe_ffn).

What pins what:
* torch autograd in float64 of torch's own silu, and central finite
  differences, for the elementwise derivative;
* closed forms: z = 0, |z| large, and the minimum of silu, which sits at
  z* = -(1 + W(1/e)) with value -W(1/e) (W = Lambert's W; scipy);
* finite differences of the wo loss <dy, swiglu(z) @ w> with respect to the
  pre-activation z, for the fused op (operand order, transposition, expert
  mapping);
* the straight-through gradient of the whole FFN, computed by torch autograd
  in float64 on inputs whose forward activation quantization is exact, for
  the FFN composition.
"""
import numpy as np
import pytest
import torch
from scipy.special import lambertw

from oracle import formats as F
from oracle import gmm as O

U_BF16 = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits)
SILU1_MAX = 1.0999          # max |silu'(z)|  (about 1.0998 at z ~ 2.4)
SILU2_MAX = 0.5             # max |silu''(z)| (at z = 0)


def _bits(x32):
    return (np.asarray(x32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_bits(x):
    """bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _dequant_torch(codes, scale):
    """w = bf16(f32(dec(code)) * scale) by torch's float8 / bf16 casts."""
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32)
    w = c * torch.from_numpy(scale)[:, None, :]
    return w.to(torch.bfloat16).to(torch.float64).numpy()


def _weights(r, G, K, N, std=0.3):
    w = r.standard_normal((G, K, N)).astype(np.float32) * np.float32(std)
    scale = (np.abs(w).max(axis=1) / np.float32(448)).astype(np.float32)
    q = np.clip(w / scale[:, None, :], -448, 448).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


# ---------------------------------------------------------------- elementwise derivative

def test_dswiglu_matches_autograd_and_finite_differences():
    r = np.random.default_rng(11)
    g = np.concatenate([r.uniform(-12, 12, 400), [-1.5, -1.27, 0.0, 1e-3, -1e-3, 3.0]])
    u = r.standard_normal(g.size) * 2
    d = r.standard_normal(g.size)
    dg, du = O.dswiglu(d, g, u)
    gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    ut = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    (torch.nn.functional.silu(gt) * ut * torch.from_numpy(d)).sum().backward()
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(du, ut.grad.numpy(), rtol=1e-13, atol=1e-15)
    # central differences of torch's silu, step 1e-5: truncation ~ 1e-10
    silu = lambda z: torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    e = 1e-5
    fd_g = d * (silu(g + e) - silu(g - e)) / (2 * e) * u
    fd_u = d * silu(g)
    np.testing.assert_allclose(dg, fd_g, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(du, fd_u, rtol=1e-12, atol=1e-15)


def test_dswiglu_closed_forms():
    d = np.array([3.0, -2.0, 0.5])
    u = np.array([1.5, 4.0, -7.0])
    # z = 0: sigma = 1/2, silu'(0) = 1/2, silu(0) = 0
    dg, du = O.dswiglu(d, np.zeros(3), u)
    np.testing.assert_array_equal(dg, d * u / 2)
    np.testing.assert_array_equal(du, np.zeros(3))
    # z -> +inf: silu'(z) -> 1, silu(z) -> z
    z = np.full(3, 60.0)
    dg, du = O.dswiglu(d, z, u)
    np.testing.assert_allclose(dg, d * u, rtol=1e-15)
    np.testing.assert_allclose(du, d * z, rtol=1e-15)
    # z -> -inf: both vanish, without NaN from exp overflow
    dg, du = O.dswiglu(d, np.full(3, -800.0), u)
    assert np.all(np.isfinite(dg)) and np.all(np.isfinite(du))
    assert np.all(np.abs(dg) == 0) and np.all(np.abs(du) == 0)
    # the minimum of silu: z* = -(1 + W(1/e)), silu(z*) = -W(1/e), silu'(z*) = 0
    w = float(lambertw(np.exp(-1.0)).real)
    zs = np.full(3, -(1.0 + w))
    dg, du = O.dswiglu(d, zs, u)
    np.testing.assert_allclose(dg, 0.0, atol=1e-15)
    np.testing.assert_allclose(du, d * -w, rtol=1e-14)


# ---------------------------------------------------------------- fused wo dLHS + dSwiGLU

def test_gmm_dswiglu_is_gradient_of_wo_loss():
    """d_preact is the gradient of L(z) = sum dy * (silu(z_g) z_u @ w_e) with
    respect to the pre-activation z (expert e of the row), by central finite
    differences in float64 on every entry of z."""
    r = np.random.default_rng(5)
    G, I, H, M = 3, 4, 6, 11
    sizes = np.array([3, 0, 5], np.int32)          # 8 valid rows, an empty expert, 3 stale rows
    codes, scale = _weights(r, G, I, H)
    w = _dequant_torch(codes, scale)               # [G, I, H]
    z_bits = _bf16_bits(r.standard_normal((M, 2 * I)) * 2)
    dy_bits = _bf16_bits(r.standard_normal((M, H)))
    z_bits[8:] = 0x7FC0
    dy_bits[8:] = 0x7F80                           # stale rows: NaN / Inf, never read
    res = O.gmm_dswiglu(dy_bits, codes, scale, sizes, z_bits)
    assert np.array_equal(res.rows, np.arange(8))
    z = F.bf16_to_f64(z_bits[:8])
    dy = F.bf16_to_f64(dy_bits[:8])
    grp = np.array([0] * 3 + [2] * 5)

    def loss(zz):
        silu = zz[:, :I] / (1.0 + np.exp(-zz[:, :I]))
        h = silu * zz[:, I:]
        return sum(float(dy[i] @ (h[i] @ w[grp[i]])) for i in range(8))

    e = 1e-6
    fd = np.zeros_like(z)
    for i in range(8):
        for j in range(2 * I):
            zp = z.copy(); zp[i, j] += e
            zm = z.copy(); zm[i, j] -= e
            fd[i, j] = (loss(zp) - loss(zm)) / (2 * e)
    np.testing.assert_allclose(res.y, fd, rtol=1e-6, atol=1e-8)
    # the unrounded wo dLHS it carries is dy @ w^T
    np.testing.assert_allclose(res.dh, np.stack([dy[i] @ w[grp[i]].T for i in range(8)]), rtol=1e-12)
    assert np.array_equal(res.out, F.f64_to_bf16_bits(res.y))


def test_gmm_dswiglu_row_subset_matches_full():
    r = np.random.default_rng(8)
    G, I, H, M = 2, 8, 16, 20
    sizes = np.array([7, 9], np.int32)
    codes, scale = _weights(r, G, I, H)
    z = _bf16_bits(r.standard_normal((M, 2 * I)))
    dy = _bf16_bits(r.standard_normal((M, H)) * 1e-3)
    full = O.gmm_dswiglu(dy, codes, scale, sizes, z)
    rows = np.array([15, 0, 6, 7])
    sub = O.gmm_dswiglu(dy, codes, scale, sizes, z, rows=rows)
    assert np.array_equal(sub.out, full.out[rows])
    assert np.array_equal(sub.group, np.array([1, 0, 0, 1]))


# ---------------------------------------------------------------- MoE FFN forward + backward

def _exact_x(r, M, H, valid):
    """Rows of e4m3 values times 2^-4 with one entry of magnitude 448 * 2^-4:
    the row scale is exactly 2^-4 and the forward quantization is lossless."""
    finite = np.array([c for c in range(256) if np.isfinite(F.DECODE[F.E4M3][c])
                       and abs(F.DECODE[F.E4M3][c]) <= 240], np.uint8)
    v = F.DECODE[F.E4M3][r.choice(finite, size=(valid, H))] * 2.0 ** -4
    v[np.arange(valid), r.integers(0, H, valid)] = 28.0 * np.where(r.random(valid) < 0.5, -1, 1)
    x = np.full((M, H), 0xFF80, np.uint16)          # stale rows: -Inf
    x[:valid] = _bits(v.astype(np.float32))
    return x


@pytest.mark.parametrize("grad_fmt", [F.E5M2, F.E4M3])
def test_moe_ffn_matches_straight_through_gradient(grad_fmt):
    """The FFN backward is the straight-through gradient of
    L = <dy, swiglu(x @ wi) @ wo> with the dequantized weights (the forward
    activation quantization is made lossless by construction), up to the bf16
    roundings of the pre-activation, d_preact and dx; the tgmm weight
    gradients are within their operand quantization noise."""
    r = np.random.default_rng(21)
    G, H, I, M, tile_m = 2, 16, 8, 14, 4
    sizes = np.array([5, 6], np.int32)
    valid = 11
    wi_codes, wi_scale = _weights(r, G, H, 2 * I, std=0.05)
    wo_codes, wo_scale = _weights(r, G, I, H, std=0.3)
    x_bits = _exact_x(r, M, H, valid)
    dy_bits = np.full((M, H), 0x7FC0, np.uint16)
    dy_bits[:valid] = _bf16_bits(r.standard_normal((valid, H)))
    res = O.moe_ffn(x_bits, wi_codes, wi_scale, wo_codes, wo_scale, sizes, dy_bits, grad_fmt, tile_m)

    grp = np.repeat(np.arange(G), sizes)
    # the forward multiplies by dec(code) * scale exactly; the backward dLHS
    # reads the bf16 dequantized weight (torch casts in both cases)
    wi_f = torch.from_numpy(np.ascontiguousarray(wi_codes)).view(torch.float8_e4m3fn).to(torch.float64) \
        * torch.from_numpy(wi_scale).to(torch.float64)[:, None, :]
    wi = torch.tensor(_dequant_torch(wi_codes, wi_scale), requires_grad=True)
    wo = torch.tensor(_dequant_torch(wo_codes, wo_scale), requires_grad=True)
    x = torch.tensor(F.bf16_to_f64(x_bits[:valid]), requires_grad=True)
    dy = torch.from_numpy(F.bf16_to_f64(dy_bits[:valid]))
    z = torch.stack([x[i].detach() @ wi_f[grp[i]] for i in range(valid)]).requires_grad_(True)
    h = torch.nn.functional.silu(z[:, :I]) * z[:, I:]
    y = torch.stack([h[i] @ wo[grp[i]] for i in range(valid)])
    (y * dy).sum().backward()
    # straight through: dx and dwi are the gradients of <dz, x @ wi>
    dz_ex = z.grad.detach()
    (torch.stack([x[i] @ wi[grp[i]] for i in range(valid)]) * dz_ex).sum().backward()

    z_ex = z.detach().numpy()
    # forward: the pre-activation is the bf16 rounding of the exact product
    assert np.array_equal(res.preact, F.f64_to_bf16_bits(z_ex))
    # d_preact before its rounding, against z.grad
    dh = np.stack([dy[i].numpy() @ wo.detach().numpy()[grp[i]].T for i in range(valid)])
    g, u = np.abs(z_ex[:, :I]), np.abs(z_ex[:, I:])
    e_g = np.abs(dh) * (U_BF16 * u * SILU1_MAX + u * SILU2_MAX * U_BF16 * g)
    e_u = np.abs(dh) * SILU1_MAX * U_BF16 * g
    e_dz = np.concatenate([e_g, e_u], axis=1) + 1e-12 * np.abs(z.grad.numpy())
    assert np.all(np.abs(res.dsw.y - z.grad.numpy()) <= e_dz)
    # dx against x.grad: propagate the d_preact error and its bf16 rounding
    e_dzb = e_dz + U_BF16 * (np.abs(z.grad.numpy()) + e_dz)
    wi_abs = np.abs(wi.detach().numpy())
    e_dx = np.stack([e_dzb[i] @ wi_abs[grp[i]].T for i in range(valid)])
    dx_ex = x.grad.numpy()
    e_dx = e_dx + U_BF16 * (np.abs(dx_ex) + e_dx) + 1e-12
    assert np.all(np.abs(F.bf16_to_f64(res.dx.out) - dx_ex) <= e_dx)
    # weight gradients: e4m3 x (e5m2 | e4m3) operand noise, ~8 % relative
    for got, ref in ((res.dwi.drhs_f64, wi.grad.numpy()), (res.dwo.drhs_f64, wo.grad.numpy())):
        assert got.shape == ref.shape
        for e in range(G):
            rel = np.linalg.norm(got[e] - ref[e]) / np.linalg.norm(ref[e])
            assert rel < 0.15, rel
    # the wo forward: h is requantized, so y carries e4m3 noise
    y_ex = y.detach().numpy()
    for e in range(G):
        sel = grp == e
        assert np.linalg.norm(res.fwd_wo.y[sel] - y_ex[sel]) / np.linalg.norm(y_ex[sel]) < 0.1
