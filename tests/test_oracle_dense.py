"""Pins of the oracle's buffer-wide backward quantization (oracle/gmm.py:
tgmm_dense), the baseline the in-kernel tgmm replaces.

* exact-rational brute force on a tiny buffer with stale rows;
* a lossless construction that reduces it to an f64 matmul;
* invariance: zero stale rows change nothing (the dense result over the
  valid prefix alone);
* the failure the pages describe: with Inf in a stale row every non-empty
  expert's gradient is NaN (empty experts stay zero) while the in-kernel
  tgmm on the same buffer is finite.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gmm as O
from tests import exact as X

F32_1EM12 = Fraction(float(np.float32(1e-12)))


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _brute(lhs, dout, sizes, fmt):
    M, K = lhs.shape
    N = dout.shape[1]
    fmax = Fraction(57344 if fmt == F.E5M2 else 448)
    _, tabL = X.torch_table("e4m3")
    _, tabD = X.torch_table("e5m2" if fmt == F.E5M2 else "e4m3")
    x = [[Fraction(float(v)) for v in F.bf16_to_f64(lhs[r])] for r in range(M)]
    d = [[Fraction(float(v)) for v in F.bf16_to_f64(dout[r])] for r in range(M)]
    sL = [X.to_f32(max(max(abs(v) for v in row), F32_1EM12) / 448) for row in x]
    qL = [[X.encode_brute(float(X.to_f32(v / sL[r])), "e4m3") for v in x[r]] for r in range(M)]
    dp = [[X.to_f32(d[r][n] * sL[r]) for n in range(N)] for r in range(M)]
    sD = [X.to_f32(max(max(abs(dp[r][n]) for r in range(M)), F32_1EM12) / fmax) for n in range(N)]
    qD = [[X.encode_brute(float(X.to_f32(dp[r][n] / sD[n])), "e5m2" if fmt == F.E5M2 else "e4m3")
           for n in range(N)] for r in range(M)]
    out = np.zeros((len(sizes), K, N))
    start = 0
    for g, sz in enumerate(sizes):
        rows = range(start, min(start + max(sz, 0), M))
        for k in range(K):
            for n in range(N):
                s = sum(Fraction(float(tabL[qL[r][k]])) * Fraction(float(tabD[qD[r][n]])) for r in rows)
                out[g, k, n] = float(X.to_f32(s * sD[n]))
        start = rows.stop if len(rows) else start
    return out, [float(v) for v in sL], [float(v) for v in sD]


@pytest.mark.parametrize("fmt", [F.E5M2, F.E4M3])
def test_dense_brute_force(fmt):
    r = np.random.default_rng(31)
    M, K, N = 9, 5, 4
    lhs = _bf16(r.standard_normal((M, K)) * 3)
    dout = _bf16(r.standard_normal((M, N)) * 0.01)
    sizes = [3, 0, 4]                     # 7 valid rows, 2 stale (finite) rows that still feed the scales
    res = O.tgmm_dense(lhs, dout, np.array(sizes, np.int32), fmt)
    ref, sL, sD = _brute(lhs, dout, sizes, fmt)
    assert np.array_equal(res.drhs, ref.astype(np.float32))
    assert list(res.sL[0]) == [np.float32(v) for v in sL]
    assert list(res.sD[0]) == [np.float32(v) for v in sD]


def test_dense_lossless_construction():
    """Rows of e4m3 values times 2^-4 with an entry 448 * 2^-4 (row scale
    2^-4 exactly), gradients whose scaled columns are e5m2 values with a
    column maximum of 57344 * 2^-20: every quantization is exact and the
    result is the plain f64 product."""
    r = np.random.default_rng(32)
    M, K, N, valid = 12, 6, 5, 10
    codesL = [c for c in range(256) if np.isfinite(F.DECODE[F.E4M3][c]) and abs(F.DECODE[F.E4M3][c]) <= 224]
    x = F.DECODE[F.E4M3][r.choice(codesL, (M, K))] * 2.0 ** -4
    x[np.arange(M), r.integers(0, K, M)] = 28.0
    codesD = [c for c in range(256) if np.isfinite(F.DECODE[F.E5M2][c]) and 2.0 ** -10 <= abs(F.DECODE[F.E5M2][c]) <= 8192]
    # d' = d * 2^-4 must be e5m2 * 2^-20 with column max 57344 * 2^-20: d = e5m2 * 2^-16
    d = F.DECODE[F.E5M2][r.choice(codesD, (M, N))] * 2.0 ** -16
    d[0, :] = 57344 * 2.0 ** -16
    sizes = np.array([4, 6], np.int32)
    d[valid:] = 0.0
    x[valid:] = 0.0
    res = O.tgmm_dense(_bf16(x), _bf16(d), sizes, F.E5M2)
    exp = np.stack([x[:4].T @ d[:4], x[4:10].T @ d[4:10]])
    np.testing.assert_array_equal(res.drhs_f64, exp)


def test_zero_stale_rows_change_nothing():
    d = W.ffn("small")
    gs, mv = d["group_sizes"], d["valid"]
    lhs, dy = d["x"].copy(), d["dy"].copy()
    lhs[mv:] = 0
    dy[mv:] = 0
    full = O.tgmm_dense(lhs, dy, gs, F.E5M2)
    valid_only = O.tgmm_dense(lhs[:mv], dy[:mv], gs, F.E5M2)
    assert np.array_equal(full.drhs, valid_only.drhs)
    assert np.isfinite(full.drhs).all()


def test_stale_inf_poisons_dense_but_not_in_kernel():
    """The pages' failure: a stale row's Inf reaches the column amax, the
    column scale is Inf, every valid code is 0 and Inf * 0 = NaN; the
    in-kernel tgmm never reads the stale rows."""
    d = W.ffn("small")
    gs = d["group_sizes"]
    res = O.tgmm_dense(d["x"], d["dy"], gs, F.E5M2)
    for g in range(len(gs)):
        if gs[g] > 0:
            assert np.isnan(res.drhs[g]).all(), g
        else:
            assert np.all(res.drhs[g] == 0)
    assert np.isinf(res.sD).all()
    ink = O.tgmm_quant(d["x"], d["dy"], gs, F.E5M2)
    assert np.isfinite(ink.drhs).all()
