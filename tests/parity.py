"""Comparison helpers for the GPU parity tests (HIP library vs CPU oracle).

Tolerances (the task's parity rule made concrete):

* integer / byte / index results (activation codes, scales, dequantized
  weights, dLHS tiles): bit-exact;
* bf16 GEMM outputs: per non-empty expert, the normwise relative error
  ||Y_gpu - bf16(Y_ref)||_F / ||bf16(Y_ref)||_F must be <= 2e-3, and every
  element must satisfy an elementwise bound derived from the arithmetic:
      |y_gpu - y_ref| <= ulp_bf16(max(|y_gpu|, |y_ref|)) + C_ACC * A + 2^-21 |y_ref|
  where A = s_row * |s_col| * sum_k |dec(q) dec(c)| (or sum_n |dout w| for the
  dLHS) comes from the oracle.  C_ACC covers the f32 accumulation: for the FP8
  MFMA (whose 128-product dot is summed in a narrower adder; measured up to
  2^-16 * A on this hardware) C_ACC = 2^-12; for bf16 MFMA (exact products,
  f32 sums) C_ACC = K * 2^-23;
* f32 outputs (tgmm): ||D_gpu - D_ref||_F / ||D_ref||_F <= 1e-5 overall and
  per expert, plus an elementwise bound of the same form.
"""
from __future__ import annotations

import numpy as np

from oracle import formats as F

NORMWISE_BF16 = 2e-3
FROBENIUS_F32 = 1e-5
C_ACC_FP8 = 2.0 ** -12


def bf16_np(t) -> np.ndarray:
    """uint16 numpy view of a torch bf16 tensor (moved to the host)."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_bf16(gpu_bits, ref_f64, absum, groups, c_acc, what, extra_tol=None):
    """Assert the bf16 tolerance rule; returns (max normwise error, max elementwise ratio)."""
    gpu = F.bf16_to_f64(gpu_bits)
    ref_b = F.bf16_to_f64(F.f64_to_bf16_bits(ref_f64))
    assert np.isfinite(gpu).all() == np.isfinite(ref_b).all(), f"{what}: non-finite values differ"
    tol = F.ulp_bf16(np.maximum(np.abs(gpu), np.abs(ref_f64))) + c_acc * absum + 2.0 ** -21 * np.abs(ref_f64)
    if extra_tol is not None:
        tol = tol + extra_tol
    err = np.abs(gpu - ref_f64)
    ratio = err / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
    assert ratio.size == 0 or ratio.max() <= 1.0, (
        f"{what}: elementwise bound exceeded at {worst}: gpu {gpu[worst]} ref {ref_f64[worst]} tol {tol[worst]}")
    worst_norm = 0.0
    for g in np.unique(groups):
        sel = groups == g
        den = np.linalg.norm(ref_b[sel])
        num = np.linalg.norm(gpu[sel] - ref_b[sel])
        e = num / den if den > 0 else (0.0 if num == 0 else np.inf)
        worst_norm = max(worst_norm, e)
        assert e <= NORMWISE_BF16, f"{what}: expert {g} normwise error {e:.3e} > {NORMWISE_BF16}"
    return worst_norm, (float(ratio.max()) if ratio.size else 0.0)


def swiglu_tol(res, I):
    """Extra elementwise tolerance of the SwiGLU output from the errors of the
    gate and up GEMM values (first-order propagation) and the exp evaluation."""
    g, u = res.y[:, :I], res.y[:, I:]
    eg = C_ACC_FP8 * res.absum[:, :I] + 2.0 ** -21 * np.abs(g)
    eu = C_ACC_FP8 * res.absum[:, I:] + 2.0 ** -21 * np.abs(u)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    return dsilu * np.abs(u) * eg + np.abs(silu) * eu + 2.0 ** -19 * np.abs(silu * u)


def check_f32(gpu, ref_f64, absum, groups_axis0, rows_per_group, what):
    """tgmm rule: relative Frobenius <= 1e-5 overall and per expert, plus an
    elementwise bound from the f32 accumulation over rows."""
    gpu = np.asarray(gpu, np.float64)
    den = np.linalg.norm(ref_f64)
    tot = np.linalg.norm(gpu - ref_f64) / den if den > 0 else float(np.linalg.norm(gpu))
    assert tot <= FROBENIUS_F32, f"{what}: relative Frobenius error {tot:.3e} > {FROBENIUS_F32}"
    per = []
    for g in range(gpu.shape[0]):
        d = np.linalg.norm(ref_f64[g])
        n = np.linalg.norm(gpu[g] - ref_f64[g])
        if d == 0:
            assert n == 0, f"{what}: expert {g} must be exactly zero"
            per.append(0.0)
            continue
        per.append(n / d)
        assert n / d <= FROBENIUS_F32, f"{what}: expert {g} relative Frobenius {n / d:.3e}"
    tol = (np.asarray(rows_per_group, np.float64)[:, None, None] + 8) * 2.0 ** -23 * absum \
        + 2.0 ** -22 * np.abs(ref_f64) + 1e-45
    ratio = np.abs(gpu - ref_f64) / tol
    assert ratio.max() <= 1.0, f"{what}: elementwise bound exceeded ({ratio.max():.3f})"
    return tot, max(per)


#: largest |silu'(z)| and |silu''(z)| over the reals (about 1.0998 and 0.5)
SILU1_MAX = 1.0999
SILU2_MAX = 0.5


def dswiglu_tol(res, preact_f64, c_acc, d_preact=None):
    """Extra elementwise tolerance of the fused dSwiGLU output [d_gate | d_up]:
    first-order propagation of the f32 accumulation error of dh (c_acc * A +
    2^-21 |dh|), the f32 evaluation of sigma / silu' (exp, reciprocal, fma),
    and, with ``d_preact`` (a bound on how far the pre-activation the kernel
    read may be from the oracle's), the change of the derivative over that
    distance (|silu''| <= 1/2, |silu'| <= 1.1)."""
    I = res.dh.shape[1]
    g, u = preact_f64[:, :I], preact_f64[:, I:]
    dh = res.dh
    e_dh = c_acc * res.dh_absum + 2.0 ** -21 * np.abs(dh)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    s1 = sig * (1.0 + g * (1.0 - sig))
    e_sig = 2.0 ** -22 * (4.0 + np.abs(g))
    e_s1 = 2.0 ** -20 * (4.0 + np.abs(g))
    tg = np.abs(u * s1) * e_dh + np.abs(dh * u) * e_s1 + 2.0 ** -20 * np.abs(res.y[:, :I])
    tu = np.abs(g * sig) * e_dh + np.abs(dh * g) * e_sig + 2.0 ** -20 * np.abs(res.y[:, I:])
    if d_preact is not None:
        dg_, du_ = d_preact[:, :I], d_preact[:, I:]
        a = np.abs(dh) + e_dh
        tg = tg + a * ((np.abs(u) + du_) * SILU2_MAX * dg_ + SILU1_MAX * du_)
        tu = tu + a * SILU1_MAX * dg_
    return np.concatenate([tg, tu], axis=1)
