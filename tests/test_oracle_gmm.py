"""Pins of the oracle's GMM functions (oracle/gmm.py).

What pins what:
* a hand-derived worked example (tests/golden/fwd_worked_example.json);
* exact rational brute force on tiny shapes (tests/exact.py, torch value tables);
* lossless constructions that reduce the method to a textbook f64 matmul;
* closed-form special cases of the scale formula;
* invariants (power-of-two row scaling, group splitting, row permutation,
  stale-tail independence, clamping of the group sizes);
* torch library cross-checks for dequantization.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import gmm as O
from tests import exact as X

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_1EM12 = Fraction(float(np.float32(1e-12)))


# ---------------------------------------------------------------- helpers

def bf16_bits(x):
    return X_to_bits(np.asarray(x, np.float32))


def X_to_bits(x32):
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def rand_codes(r, shape, fmt=F.E4M3, lo_exp=None):
    """Random finite codes (never NaN)."""
    d = F.DECODE[fmt]
    finite = np.array([c for c in range(256) if np.isfinite(d[c])], np.uint8)
    return r.choice(finite, size=shape)


def tiny_fwd_inputs(seed, G=3, M=12, K=32, N=16, sizes=(0, 5, 4)):
    r = np.random.default_rng(seed)
    lhs = bf16_bits(r.standard_normal((M, K)).astype(np.float32) * 3)
    w = r.standard_normal((G, K, N)).astype(np.float32) * 0.02
    scale = (np.abs(w).max(axis=1) / 448).astype(np.float32)
    codes = torch.from_numpy(np.clip(w / scale[:, None, :], -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return lhs, codes, scale, np.array(sizes, np.int32)


def _bits_to_frac(b):
    v = float(np.array([b], np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)[0])
    return Fraction(v), math.copysign(1.0, v) < 0


def brute_forward(lhs, codes, scale, sizes, swiglu=False):
    """Pure-Python exact forward: dict row -> list of bf16 bit patterns."""
    M, K = lhs.shape
    G, _, N = codes.shape
    _, tab = X.torch_table("e4m3")
    out, start = {}, 0
    for g in range(G):
        n = max(int(sizes[g]), 0)
        end = min(start + n, M)
        for r in range(start, end):
            xs = [_bits_to_frac(b) for b in lhs[r]]
            amax = max(abs(v) for v, _ in xs)
            s = X.to_f32(max(amax, F32_1EM12) / 448)
            q = []
            for v, neg in xs:
                quo = X.to_f32(v / s)
                c = X.encode_brute(-float(quo) if (neg and quo == 0) else float(quo), "e4m3")
                q.append(c)
            ys = []
            for n_ in range(N):
                acc = sum(Fraction(float(tab[q[k]])) * Fraction(float(tab[codes[g, k, n_]])) for k in range(K))
                ys.append(acc * s * Fraction(float(scale[g, n_])))
            if swiglu:
                I = N // 2
                vals = []
                for i in range(I):
                    gt, up = float(ys[i]), float(ys[I + i])
                    vals.append(X.to_bf16(Fraction(gt / (1.0 + math.exp(-gt)) * up)))
            else:
                vals = [X.to_bf16(y) for y in ys]
            out[r] = [X.bf16_bits_of(v) for v in vals]
        start = end
    return out


# ---------------------------------------------------------------- worked example

def test_golden_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "fwd_worked_example.json")))
    lhs = np.array(d["lhs_bf16_bits"], np.uint16)
    assert np.array_equal(lhs, bf16_bits(np.array(d["lhs_values"], np.float32)))
    codes = np.array(d["weight_codes_KxN"], np.uint8)[None]
    scale = np.array([d["weight_scale"]], np.float32)
    res = O.gmm_fwd(lhs, codes, scale, d["group_sizes"])
    assert np.array_equal(res.act_codes, np.array(d["act_codes"], np.uint8))
    assert np.array_equal(res.act_scale, np.array(d["act_scale"], np.float32))
    assert np.array_equal(res.out, np.array(d["out_bf16_bits"], np.uint16))
    assert np.array_equal(F.bf16_to_f64(res.out), np.array(d["out_values"]))
    sw = O.gmm_fwd(lhs, codes, scale, d["group_sizes"], swiglu_out=True)
    assert np.array_equal(sw.out, np.array(d["swiglu_bf16_bits"], np.uint16))
    assert np.array_equal(F.bf16_to_f64(sw.out), np.array(d["swiglu_values"]))


# ---------------------------------------------------------------- scale special cases

def test_scale_zero_row_and_powers_of_two():
    K = 64
    x = np.zeros((1, K), np.float32)
    s = O.row_scales(x)
    ref = X.to_f32(F32_1EM12 / 448)
    assert Fraction(float(s[0])) == ref
    assert np.all(O.quantize_rows(x, s) == 0)
    r = np.random.default_rng(3)
    for j in range(-20, 20):
        row = (r.uniform(-1, 1, (1, K)) * 2.0 ** j).astype(np.float32)
        row[0, 7] = -448.0 * 2.0 ** j
        sj = O.row_scales(row)
        assert sj[0] == np.float32(2.0 ** j)
        assert O.quantize_rows(row, sj)[0, 7] == 0xFE
    # the floor only binds below 1e-12
    tiny = np.full((1, K), 1e-13, np.float32)
    assert O.row_scales(tiny)[0] == np.float32(np.float32(1e-12) / np.float32(448))
    assert np.all(O.quantize_rows(tiny, O.row_scales(tiny)) == F.encode(np.float32(1e-13) / O.row_scales(tiny), F.E4M3))


def test_quotient_rounding_at_scale():
    """The activation quotient is the correctly rounded f32 of x / s.  Checked on
    2^20 values placed near e4m3 rounding midpoints against the f64 route
    fl32(fl64(x) / fl64(s)), which is correctly rounded because 53 >= 2*24 + 2
    (double rounding is innocuous for division, Figueroa 1995)."""
    r = np.random.default_rng(31)
    R, K = 4096, 256
    pos = F.DECODE[F.E4M3][:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    s = (2.0 ** r.uniform(-8, 8, R)).astype(np.float32)
    target = r.choice(mids, (R, K)) * np.where(r.random((R, K)) < 0.5, -1, 1)
    x = (target * s[:, None].astype(np.float64)).astype(np.float32)
    x = np.nextafter(x, np.where(r.random((R, K)) < 0.5, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)) \
        * (r.random((R, K)) < 0.5) + x * (r.random((R, K)) >= 0.5)
    x = x.astype(np.float32)
    q64 = (x.astype(np.float64) / s[:, None].astype(np.float64)).astype(np.float32)
    assert np.array_equal(O.quantize_rows(x, s), F.encode(q64, F.E4M3))


def test_scale_spans_full_k():
    """The scale of a row is taken over all of K: a large value at the far end of
    the row changes the codes of the first columns (a per-tile scale would not)."""
    K = 1024
    r = np.random.default_rng(4)
    row = r.standard_normal((1, K)).astype(np.float32)
    row2 = row.copy()
    row2[0, K - 1] = 1000.0
    q1 = O.quantize_rows(row, O.row_scales(row))
    q2 = O.quantize_rows(row2, O.row_scales(row2))
    assert not np.array_equal(q1[0, :128], q2[0, :128])


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("sizes", [(0, 5, 4), (3, 9, 0), (4, 4, 4)])
def test_forward_brute_force(sizes):
    lhs, codes, scale, gs = tiny_fwd_inputs(5, sizes=sizes)
    res = O.gmm_fwd(lhs, codes, scale, gs)
    ref = brute_forward(lhs, codes, scale, gs)
    assert sorted(ref) == list(res.rows)
    for i, r in enumerate(res.rows):
        assert list(res.out[i]) == ref[r], r


def test_forward_swiglu_brute_force():
    lhs, codes, scale, gs = tiny_fwd_inputs(6, sizes=(2, 6, 4))
    res = O.gmm_fwd(lhs, codes, scale, gs, swiglu_out=True)
    ref = brute_forward(lhs, codes, scale, gs, swiglu=True)
    for i, r in enumerate(res.rows):
        assert list(res.out[i]) == ref[r], r


def test_activation_codes_brute_force():
    lhs, codes, scale, gs = tiny_fwd_inputs(7, sizes=(12, 0, 0))
    lhs[3, 5] = 0x8000                          # -0.0 must keep its sign
    res = O.gmm_fwd(lhs, codes, scale, gs)
    for r in range(12):
        xs = [_bits_to_frac(b) for b in lhs[r]]
        amax = max(abs(v) for v, _ in xs)
        s = X.to_f32(max(amax, F32_1EM12) / 448)
        assert Fraction(float(res.act_scale[r])) == s
        for k, (v, neg) in enumerate(xs):
            quo = X.to_f32(v / s)
            c = X.encode_brute(-float(quo) if (neg and quo == 0) else float(quo), "e4m3")
            assert res.act_codes[r, k] == c
    assert res.act_codes[3, 5] == 0x80


# ---------------------------------------------------------------- lossless construction

def test_forward_lossless_construction():
    """Rows built as dec(q) * 2^j with one element = +-448 * 2^j quantize back to
    exactly q with scale 2^j, so the op must equal bf16(X @ dec(C) * scale) from a
    plain f64 matmul on the activation values themselves."""
    r = np.random.default_rng(8)
    G, M, K, N = 3, 40, 64, 24
    gs = np.array([15, 0, 25], np.int32)
    q = rand_codes(r, (M, K))
    q[np.arange(M), r.integers(0, K, M)] = np.where(r.random(M) < 0.5, 0x7E, 0xFE)
    j = r.integers(-6, 7, M)
    x = F.decode(q, F.E4M3) * 2.0 ** j[:, None]
    lhs = bf16_bits(x.astype(np.float32))
    assert np.array_equal(F.bf16_to_f64(lhs), x)          # exact in bf16
    codes = rand_codes(r, (G, K, N))
    scale = (r.uniform(0.5, 2, (G, N)) * 2.0 ** -10).astype(np.float32)
    res = O.gmm_fwd(lhs, codes, scale, gs)
    assert np.array_equal(res.act_codes, q)
    assert np.array_equal(res.act_scale, (2.0 ** j).astype(np.float32))
    gid = O.layout(gs, M).group_of_rows(M)
    for g in range(G):
        rows = np.nonzero(gid == g)[0]
        if len(rows) == 0:
            continue
        ref = (x[rows] @ F.decode(codes[g], F.E4M3)) * scale[g].astype(np.float64)[None, :]
        assert np.array_equal(res.out[np.isin(res.rows, rows)], F.f64_to_bf16_bits(ref))


# ---------------------------------------------------------------- invariants

def test_forward_power_of_two_row_scaling():
    lhs, codes, scale, gs = tiny_fwd_inputs(9, M=20, sizes=(8, 0, 12))
    base = O.gmm_fwd(lhs, codes, scale, gs)
    x = F.bf16_to_f64(lhs)
    for j in (-5, 3):
        lhs2 = bf16_bits((x * 2.0 ** j).astype(np.float32))
        res = O.gmm_fwd(lhs2, codes, scale, gs)
        assert np.array_equal(res.act_codes, base.act_codes)
        assert np.array_equal(res.y, base.y * 2.0 ** j)
        assert np.array_equal(F.bf16_to_f64(res.out), F.bf16_to_f64(base.out) * 2.0 ** j)


def test_forward_group_split_and_permutation():
    lhs, codes, scale, _ = tiny_fwd_inputs(10, M=20)
    codes2 = codes.copy(); codes2[1] = codes2[0]
    scale2 = scale.copy(); scale2[1] = scale2[0]
    one = O.gmm_fwd(lhs, codes2, scale2, [14, 0, 6])
    split = O.gmm_fwd(lhs, codes2, scale2, [9, 5, 6])
    assert np.array_equal(one.out, split.out)
    perm = np.concatenate([np.random.default_rng(1).permutation(14), np.arange(14, 20)])
    permuted = O.gmm_fwd(lhs[perm], codes2, scale2, [14, 0, 6])
    assert np.array_equal(permuted.out, one.out[perm])


def test_stale_tail_never_read():
    from workloads import fill_garbage
    lhs, codes, scale, gs = tiny_fwd_inputs(11, M=20, sizes=(3, 6, 4))
    a = lhs.copy(); a[13:] = 0
    b = lhs.copy(); fill_garbage(b, 13)
    ra, rb = O.gmm_fwd(a, codes, scale, gs), O.gmm_fwd(b, codes, scale, gs)
    assert np.array_equal(ra.out, rb.out) and len(ra.rows) == 13
    assert np.isfinite(rb.y).all()


def test_layout_clamp_and_negative():
    lay = O.layout([5, 10], 12)
    assert lay.clamped and not lay.negative and lay.valid == 12
    assert list(lay.start) == [0, 5] and list(lay.end) == [5, 12]
    lay = O.layout([-3, 4, 2], 12)
    assert lay.negative and not lay.clamped and list(lay.start) == [0, 0, 4] and lay.valid == 6
    lay = O.layout([0, 0], 5)
    assert lay.valid == 0
    lay = O.layout([7, 7, 7], 10)
    assert list(lay.start) == [0, 7, 10] and list(lay.end) == [7, 10, 10]


# ---------------------------------------------------------------- dequant

def test_dequant_matches_torch_and_exact_cases():
    r = np.random.default_rng(12)
    codes = rand_codes(r, (8, 512, 512))
    scale = (r.uniform(0.1, 3, (8, 512)) * 2.0 ** r.integers(-12, 4, (8, 512))).astype(np.float32)
    ours = O.dequantize(codes, scale)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scale)[:, None, :]
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    one = O.dequantize(codes, np.ones_like(scale))
    assert np.array_equal(F.bf16_to_f64(one), F.decode(codes, F.E4M3))
    p2 = O.dequantize(codes, np.full_like(scale, 2.0 ** -7))
    assert np.array_equal(F.bf16_to_f64(p2), F.decode(codes, F.E4M3) * 2.0 ** -7)
    # hand-derived: 1.0 * 0.1f -> bf16 0x3DCD; 448 * 0.1f -> f32 44.79999923706055 -> bf16 44.75 (0x4233)
    hd = O.dequantize(np.array([[[0x38, 0x7E]]], np.uint8), np.array([[0.1, 0.1]], np.float32))
    assert list(hd[0, 0]) == [0x3DCD, 0x4233]
    # products whose f32 rounding lands on a bf16 midpoint: the result is the
    # f32 product rounded to bf16, not the exact product rounded to bf16
    _, tab = X.torch_table("e4m3")
    cases = [(0x3F, 1066366840), (0x3F, 1067415415), (0x3B, 1070548434), (0x3B, 1069499857)]
    for code, sbits in cases:
        sc = np.array([[sbits]], np.uint32).view(np.float32)
        exact = Fraction(float(tab[code])) * Fraction(float(sc[0, 0]))
        via_f32 = X.bf16_bits_of(X.to_bf16(X.to_f32(exact)))
        assert via_f32 != X.bf16_bits_of(X.to_bf16(exact))
        assert O.dequantize(np.array([[[code]]], np.uint8), sc)[0, 0, 0] == via_f32


# ---------------------------------------------------------------- dLHS

def test_dlhs_one_hot_selects_weight_column():
    r = np.random.default_rng(13)
    G, M, K, N = 2, 6, 24, 16
    codes = rand_codes(r, (G, K, N))
    scale = r.uniform(0.001, 0.01, (G, N)).astype(np.float32)
    dout = np.zeros((M, N), np.uint16)
    cols = [0, 5, 15, 3, 9, 1]
    for i, n in enumerate(cols):
        dout[i, n] = 0x3F80                                   # 1.0
    res = O.gmm_dlhs(dout, codes, scale, [4, 2])
    w = O.dequantize(codes, scale)
    for i, n in enumerate(cols):
        g = 0 if i < 4 else 1
        assert np.array_equal(res.out[i], w[g, :, n])


def test_dlhs_brute_force():
    r = np.random.default_rng(14)
    G, M, K, N = 3, 10, 12, 20
    codes = rand_codes(r, (G, K, N))
    scale = r.uniform(0.001, 0.01, (G, N)).astype(np.float32)
    dout = bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    gs = [0, 6, 4]
    res = O.gmm_dlhs(dout, codes, scale, gs)
    _, tab = X.torch_table("e4m3")
    for i, row in enumerate(res.rows):
        g = 1 if row < 6 else 2
        for k in range(K):
            acc = Fraction(0)
            for n in range(N):
                w = X.to_bf16(X.to_f32(Fraction(float(tab[codes[g, k, n]])) * Fraction(float(scale[g, n]))))
                acc += _bits_to_frac(dout[row, n])[0] * w
            assert res.out[i, k] == X.bf16_bits_of(X.to_bf16(acc)), (row, k)


def test_dlhs_stale_tail():
    from workloads import fill_garbage
    r = np.random.default_rng(15)
    codes = rand_codes(r, (2, 8, 16)); scale = r.uniform(0.01, 0.1, (2, 16)).astype(np.float32)
    dout = bf16_bits(r.standard_normal((10, 16)).astype(np.float32))
    d2 = dout.copy(); fill_garbage(d2, 7)
    a = O.gmm_dlhs(dout, codes, scale, [3, 4]); b = O.gmm_dlhs(d2, codes, scale, [3, 4])
    assert np.array_equal(a.out, b.out)


# ---------------------------------------------------------------- tgmm

def brute_tgmm(lhs, dout, sizes, grad_fmt, tile_m):
    M, K = lhs.shape
    N = dout.shape[1]
    G = len(sizes)
    _, t4 = X.torch_table("e4m3")
    _, tg = X.torch_table(grad_fmt)
    fm_g = 448 if grad_fmt == "e4m3" else 57344
    out = [[[Fraction(0)] * N for _ in range(K)] for _ in range(G)]
    start = 0
    scales = []
    for g in range(G):
        end = min(start + max(int(sizes[g]), 0), M)
        t = start // tile_m
        while start < end and t * tile_m < end:
            r0, r1 = max(start, t * tile_m), min(end, (t + 1) * tile_m)
            L = [[_bits_to_frac(lhs[r, k]) for k in range(K)] for r in range(r0, r1)]
            D = [[_bits_to_frac(dout[r, n]) for n in range(N)] for r in range(r0, r1)]
            sL = [X.to_f32(max(max(abs(L[i][k][0]) for i in range(r1 - r0)), F32_1EM12) / 448) for k in range(K)]
            sD = [X.to_f32(max(max(abs(D[i][n][0]) for i in range(r1 - r0)), F32_1EM12) / fm_g) for n in range(N)]
            enc = lambda v, neg, s, fmt: X.encode_brute(-0.0 if (neg and X.to_f32(v / s) == 0) else float(X.to_f32(v / s)), fmt)
            qL = [[Fraction(float(t4[enc(*L[i][k], sL[k], "e4m3")])) for k in range(K)] for i in range(r1 - r0)]
            qD = [[Fraction(float(tg[enc(*D[i][n], sD[n], grad_fmt)])) for n in range(N)] for i in range(r1 - r0)]
            for k in range(K):
                for n in range(N):
                    tile = sum(qL[i][k] * qD[i][n] for i in range(r1 - r0))
                    out[g][k][n] += tile * sL[k] * sD[n]
            scales.append((g, t, sL, sD))
            t += 1
        start = end
    return out, scales


@pytest.mark.parametrize("grad_fmt", [F.E5M2, F.E4M3])
def test_tgmm_brute_force(grad_fmt):
    r = np.random.default_rng(16)
    M, K, N, tile_m = 14, 6, 5, 4
    sizes = [0, 5, 7, 0]                     # empty first/last experts, a boundary inside a tile
    lhs = bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    dout = bf16_bits(r.standard_normal((M, N)).astype(np.float32) * 1e-3)
    res = O.tgmm_quant(lhs, dout, sizes, grad_fmt, tile_m)
    ref, scales = brute_tgmm(lhs, dout, sizes, grad_fmt, tile_m)
    assert [(t.group, t.tile) for t in res.tiles] == [(g, t) for g, t, _, _ in scales]
    for i, (_, _, sL, sD) in enumerate(scales):
        assert [Fraction(float(v)) for v in res.sL[i]] == sL
        assert [Fraction(float(v)) for v in res.sD[i]] == sD
    for g in range(len(sizes)):
        for k in range(K):
            for n in range(N):
                assert Fraction(float(res.drhs[g, k, n])) == X.to_f32(ref[g][k][n]), (g, k, n)
    assert np.all(res.drhs[0] == 0) and np.all(res.drhs[3] == 0)


@pytest.mark.parametrize("grad_fmt", [F.E5M2, F.E4M3])
def test_tgmm_lossless_construction(grad_fmt):
    """Per (expert, tile, channel) blocks built as dec(code) * 2^j with one element
    at +-FMAX * 2^j quantize losslessly, so drhs[g] must equal lhs_g^T @ dout_g from
    a plain f64 matmul."""
    r = np.random.default_rng(17)
    M, K, N, tile_m = 40, 12, 10, 8
    sizes = np.array([11, 0, 21, 5], np.int32)
    tiles = O.tgmm_tiles(sizes, M, tile_m)
    L = np.zeros((M, K)); D = np.zeros((M, N))
    for tl in tiles:
        rows = slice(tl.row0, tl.row1)
        n = tl.row1 - tl.row0
        for mat, fmt, fm, cols in ((L, F.E4M3, 448.0, K), (D, grad_fmt, F.FMAX[grad_fmt], N)):
            c = rand_codes(r, (n, cols), fmt)
            c[r.integers(0, n, cols), np.arange(cols)] = np.where(r.random(cols) < 0.5, F.MAX_CODE[fmt], F.MAX_CODE[fmt] | 0x80)
            j = r.integers(-8, 3, cols)
            mat[rows] = F.decode(c, fmt) * 2.0 ** j[None, :]
    lhs, dout = bf16_bits(L.astype(np.float32)), bf16_bits(D.astype(np.float32))
    assert np.array_equal(F.bf16_to_f64(lhs), L) and np.array_equal(F.bf16_to_f64(dout), D)
    res = O.tgmm_quant(lhs, dout, sizes, grad_fmt, tile_m)
    lay = O.layout(sizes, M)
    for g in range(len(sizes)):
        a, b = lay.start[g], lay.end[g]
        ref = (L[a:b].T @ D[a:b]).astype(np.float32)
        assert np.array_equal(res.drhs[g], ref), g


@pytest.mark.parametrize("grad_fmt", [F.E5M2, F.E4M3])
def test_tgmm_float64_products_match_exact_sums(grad_fmt):
    """The float64-product path (for the largest shapes) against the exact
    integer sums: full 512-row tiles of seeded data with outliers, so the
    products span many binades; the difference stays within 512 * 2^-53 of
    the magnitude sum, and the f32 results agree."""
    r = np.random.default_rng(19)
    M, K, N = 1300, 48, 40
    sizes = [600, 0, 700]
    x = r.standard_normal((M, K)).astype(np.float32)
    x[r.integers(0, M, 60), r.integers(0, K, 60)] *= 50
    lhs = bf16_bits(x)
    dout = bf16_bits((r.standard_normal((M, N)) * 1e-3).astype(np.float32))
    ex = O.tgmm_quant(lhs, dout, sizes, grad_fmt, 512)
    fp = O.tgmm_quant(lhs, dout, sizes, grad_fmt, 512, exact=False)
    assert np.array_equal(ex.sL, fp.sL) and np.array_equal(ex.sD, fp.sD)
    assert np.all(np.abs(fp.drhs_f64 - ex.drhs_f64) <= 512 * 2.0 ** -53 * ex.absum + 1e-300)
    assert np.array_equal(fp.absum, ex.absum)
    mism = np.count_nonzero(fp.drhs != ex.drhs)
    assert mism <= 2, mism     # at most a rare tie of the final f32 rounding


def test_tgmm_stale_tail_and_tiles():
    from workloads import fill_garbage
    r = np.random.default_rng(18)
    M, K, N = 30, 8, 6
    sizes = [7, 9, 0, 4]
    lhs = bf16_bits(r.standard_normal((M, K)).astype(np.float32))
    dout = bf16_bits(r.standard_normal((M, N)).astype(np.float32))
    l2, d2 = lhs.copy(), dout.copy()
    fill_garbage(l2, 20); fill_garbage(d2, 20)
    a = O.tgmm_quant(lhs, dout, sizes, F.E5M2, 8)
    b = O.tgmm_quant(l2, d2, sizes, F.E5M2, 8)
    assert np.array_equal(a.drhs, b.drhs) and np.isfinite(b.drhs).all()
    tl = O.tgmm_tiles(sizes, M, 8)
    assert [(t.group, t.tile, t.row0, t.row1) for t in tl] == [
        (0, 0, 0, 7), (1, 0, 7, 8), (1, 1, 8, 16), (3, 2, 16, 20)]
    # bound on the number of (expert, tile) pairs
    for seed in range(20):
        rr = np.random.default_rng(seed)
        G = int(rr.integers(1, 9)); Mx = int(rr.integers(1, 100)); tm = int(rr.integers(1, 16))
        s = rr.integers(0, Mx // 2 + 2, G)
        assert len(O.tgmm_tiles(s, Mx, tm)) <= -(-Mx // tm) + G - 1
    # column restriction is exact
    sub = O.tgmm_quant(lhs, dout, sizes, F.E5M2, 8, k_cols=[1, 6], n_cols=[0, 5])
    assert np.array_equal(sub.drhs, a.drhs[:, [1, 6]][:, :, [0, 5]])


def test_forward_row_subset_matches_full():
    lhs, codes, scale, gs = tiny_fwd_inputs(19, M=20, sizes=(8, 5, 7))
    full = O.gmm_fwd(lhs, codes, scale, gs)
    sub = O.gmm_fwd(lhs, codes, scale, gs, rows=[19, 3, 8])
    assert np.array_equal(sub.out, full.out[[19, 3, 8]])
