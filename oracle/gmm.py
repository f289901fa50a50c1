"""Plain CPU reference of the routed-expert FP8 grouped matmul (GMM) family.

Test infrastructure only: nothing on the product path imports this module.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Every function restates the method of two pages:

* "MoE: native FP8 QAT for routed-expert GMMs" (maxtext PR #5969):
  Description ("What the new flags change"), Data flow (table), Implementation.
* "MoE fp8 backward: in-kernel drhs operand quantization + configurable
  gradient dtype" (maxtext PR #4971): What.

Conventions (one reading each; the list of readings is kept with the design notes):

* ``lhs`` is a static ragged buffer ``[M, K]`` of bf16 bit patterns (uint16).
  Rows ``[off_g, off_g + size_g)`` belong to expert ``g`` with
  ``off_g = sum(size_h, h < g)``; rows at or past ``sum(group_sizes)`` are stale
  and never read.  Negative sizes count as 0 and the running sum is clamped to M.
* Weight codes are ``[G, K, N]`` e4m3fn codes (uint8, N fastest); the weight
  scale is one f32 per (expert, output channel), ``[G, N]``.
* Quantities the pages fix in f32 (activation scale, the quotient x/s, the
  dequantized weight before its bf16 rounding) are computed in f32; everything
  else is float64.  The FP8 contraction itself is exact in float64: every e4m3
  value is a multiple of 2^-9 and below 2^9, so for K <= 8192 every partial sum
  is a multiple of 2^-18 below 2^31 and fits the 53-bit significand.
* Results are returned for valid rows only; what a kernel leaves in the rows
  past the valid prefix is checked separately (they must stay untouched).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F

AMAX_FLOOR = np.float32(1e-12)
E4M3_MAX = np.float32(448.0)


# --------------------------------------------------------------------------- layout

@dataclass
class Layout:
    """Row ranges of each expert in the static buffer.

    ``start[g]``, ``end[g]``: valid rows of expert g are ``[start[g], end[g])``.
    ``valid``: number of valid rows M_v.  ``clamped``/``negative`` report the
    two repairs (sum past M, negative size).
    """
    start: np.ndarray
    end: np.ndarray
    valid: int
    clamped: bool
    negative: bool

    def group_of_rows(self, M: int) -> np.ndarray:
        """Expert id of each row, -1 for rows past the valid prefix."""
        gid = np.full(M, -1, dtype=np.int64)
        for g in range(len(self.start)):
            gid[self.start[g]:self.end[g]] = g
        return gid


def layout(group_sizes, M: int) -> Layout:
    """Group offsets from ``group_sizes`` ("MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype", What: the in-kernel path touches
    only the tiles covered by group_sizes).  Negative sizes are treated as 0 and
    the running sum is clamped to the static row count M, so no row index ever
    leaves the buffer."""
    gs = np.asarray(group_sizes, dtype=np.int64)
    negative = bool(np.any(gs < 0))
    gs = np.maximum(gs, 0)
    ends_raw = np.cumsum(gs)
    clamped = bool(len(gs) and ends_raw[-1] > M)
    end = np.minimum(ends_raw, M)
    start = np.concatenate([[0], end[:-1]]) if len(gs) else np.zeros(0, np.int64)
    valid = int(end[-1]) if len(gs) else 0
    return Layout(start.astype(np.int64), end.astype(np.int64), valid, clamped, negative)


# --------------------------------------------------------------------------- forward

def row_scales(x_f32: np.ndarray) -> np.ndarray:
    """One f32 scale per activation row over the whole K axis:
    ``s = max(amax, 1e-12) / 448`` evaluated in f32 ("MoE: native FP8 QAT for routed-expert GMMs", Implementation: LHS
    quantization options, lhs_f32_scale; the native forward always uses the full
    K with an f32 scale)."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    return (np.maximum(amax, AMAX_FLOOR) / E4M3_MAX).astype(np.float32)


def quantize_rows(x_f32: np.ndarray, s: np.ndarray) -> np.ndarray:
    """e4m3fn codes of ``x / s`` with the quotient rounded to f32 first ("MoE: native FP8 QAT for routed-expert GMMs",
    Description: the forward quantizes the activation inside the kernel)."""
    q = (np.asarray(x_f32, np.float32) / np.asarray(s, np.float32)[:, None]).astype(np.float32)
    return F.encode(q, F.E4M3)


def _fwd_rows(x_bits, codes_g, scale_g):
    """Exact f64 pre-rounding result ``(sum_k dec(q)*dec(c)) * s_row * scale``
    for rows of one expert, plus the abs-sum bound term."""
    x = F.bf16_to_f32(x_bits)
    s = row_scales(x)
    q = quantize_rows(x, s)
    qd = F.decode(q, F.E4M3)
    cd = F.decode(codes_g, F.E4M3)
    acc = qd @ cd                                     # exact (see module doc)
    y = (acc * s.astype(np.float64)[:, None]) * scale_g.astype(np.float64)[None, :]
    absum = ((np.abs(qd) @ np.abs(cd)) * s.astype(np.float64)[:, None]) \
        * np.abs(scale_g.astype(np.float64))[None, :]
    return y, absum, q, s


@dataclass
class FwdResult:
    rows: np.ndarray        # buffer row index of each result row
    group: np.ndarray       # expert of each result row
    y: np.ndarray           # f64 pre-rounding GEMM result [R, N] (scaled)
    absum: np.ndarray       # s_row * |scale| * sum_k |dec q * dec c|   [R, N]
    out: np.ndarray         # bf16 bits of the op's output [R, N or N/2]
    out_f64: np.ndarray     # exact f64 value before the bf16 rounding
    act_codes: np.ndarray   # e4m3 codes of the quantized rows [R, K]
    act_scale: np.ndarray   # f32 row scales [R]


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """``silu(gate) * up`` in float64, silu(z) = z / (1 + exp(-z)) ("MoE: native FP8 QAT for routed-expert GMMs",
    Implementation: gmm_silu_fp8 is wi with a fused SwiGLU)."""
    with np.errstate(over="ignore"):
        return gate / (1.0 + np.exp(-gate)) * up


def gmm_fwd(lhs_bits, codes, scale, group_sizes, *, swiglu_out=False, rows=None) -> FwdResult:
    """Native FP8 forward GMM ("MoE: native FP8 QAT for routed-expert GMMs", Description and Data flow table: wi/wo run
    FP8 x FP8 with f32 accumulation, read the codes and per-channel scale, and
    quantize the activation rows in the kernel).

    ``rows``: optional subset of buffer rows to evaluate (each row is
    independent given its own scale); default all valid rows.  With
    ``swiglu_out`` the N columns are ``[gate | up]`` and the output is
    ``bf16(silu(gate) * up)`` of width N/2 ("MoE: native FP8 QAT for routed-expert GMMs", Implementation: gmm_silu_fp8).
    """
    lhs_bits = np.asarray(lhs_bits)
    M, K = lhs_bits.shape
    G, K2, N = codes.shape
    assert K2 == K and scale.shape == (G, N)
    lay = layout(group_sizes, M)
    gid = lay.group_of_rows(M)
    if rows is None:
        rows = np.arange(lay.valid, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    assert np.all(gid[rows] >= 0), "requested rows must be valid rows"
    R = len(rows)
    y = np.zeros((R, N)); absum = np.zeros((R, N))
    act_codes = np.zeros((R, K), np.uint8); act_scale = np.zeros(R, np.float32)
    for g in range(G):
        sel = np.nonzero(gid[rows] == g)[0]
        if len(sel) == 0:
            continue
        yy, aa, q, s = _fwd_rows(lhs_bits[rows[sel]], codes[g], scale[g])
        y[sel], absum[sel], act_codes[sel], act_scale[sel] = yy, aa, q, s
    if swiglu_out:
        assert N % 2 == 0
        I = N // 2
        out_f64 = swiglu(y[:, :I], y[:, I:])
    else:
        out_f64 = y
    out = F.f64_to_bf16_bits(out_f64)
    return FwdResult(rows, gid[rows], y, absum, out, out_f64, act_codes, act_scale)


# --------------------------------------------------------------------------- dequant

def dequantize(codes, scale) -> np.ndarray:
    """``bf16(f32(dec(code) * scale))`` for ``codes[G,K,N]`` and ``scale[G,N]``
    ("MoE: native FP8 QAT for routed-expert GMMs", Implementation: dequantize_fp8_codes; the f32 product rounded once to
    bf16).  Returns bf16 bit patterns [G, K, N]."""
    w32 = F.decode(codes, F.E4M3).astype(np.float32) * np.asarray(scale, np.float32)[:, None, :]
    return F.f64_to_bf16_bits(w32.astype(np.float32).astype(np.float64))


# --------------------------------------------------------------------------- dLHS

@dataclass
class DlhsResult:
    rows: np.ndarray
    group: np.ndarray
    y: np.ndarray        # f64 result before the bf16 rounding [R, K]
    absum: np.ndarray    # sum_n |dout * w|   [R, K]
    out: np.ndarray      # bf16 bits [R, K]


def gmm_dlhs(dout_bits, codes, scale, group_sizes, *, rows=None) -> DlhsResult:
    """Backward dLHS: ``dlhs[r, k] = bf16(sum_n dout[r, n] * w[g, k, n])`` with
    ``w = dequantize(codes, scale)`` ("MoE: native FP8 QAT for routed-expert GMMs", Description: the backward dLHS GMM
    reads the codes and dequantizes each tile, bit-identical to the dequant
    path; Implementation: the rhs_contract_dequant path).  The sum over n is
    float64."""
    dout_bits = np.asarray(dout_bits)
    M, N = dout_bits.shape
    G, K, N2 = codes.shape
    assert N2 == N
    lay = layout(group_sizes, M)
    gid = lay.group_of_rows(M)
    if rows is None:
        rows = np.arange(lay.valid, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    assert np.all(gid[rows] >= 0)
    R = len(rows)
    y = np.zeros((R, K)); absum = np.zeros((R, K))
    for g in range(G):
        sel = np.nonzero(gid[rows] == g)[0]
        if len(sel) == 0:
            continue
        w = F.bf16_to_f64(dequantize(codes[g:g + 1], scale[g:g + 1])[0])   # [K, N]
        d = F.bf16_to_f64(dout_bits[rows[sel]])
        y[sel] = d @ w.T
        absum[sel] = np.abs(d) @ np.abs(w).T
    return DlhsResult(rows, gid[rows], y, absum, F.f64_to_bf16_bits(y))


# --------------------------------------------------------------------------- tgmm

@dataclass
class TgmmTile:
    group: int
    tile: int          # buffer-aligned tile index (rows [tile*tile_m, (tile+1)*tile_m))
    row0: int          # first row of the tile within the group
    row1: int          # one past the last row


def tgmm_tiles(group_sizes, M: int, tile_m: int) -> list[TgmmTile]:
    """Non-empty (expert, gm-tile) pairs in (expert, tile) order.  Tiles are
    aligned to the buffer and intersected with each expert's rows, so a tile
    that straddles an expert boundary gives one entry per expert ("MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype", What:
    per-gm-tile-per-channel quantization that touches only the tiles covered
    by group_sizes)."""
    lay = layout(group_sizes, M)
    out = []
    for g in range(len(lay.start)):
        a, b = int(lay.start[g]), int(lay.end[g])
        if b <= a:
            continue
        for t in range(a // tile_m, (b - 1) // tile_m + 1):
            out.append(TgmmTile(g, t, max(a, t * tile_m), min(b, (t + 1) * tile_m)))
    return out


def column_scales(x_f32: np.ndarray, fmax) -> np.ndarray:
    """Per-channel f32 scale of one tile: ``max(amax over the tile's rows,
    1e-12) / fmax`` in f32 (same formula as the forward row scale)."""
    amax = np.max(np.abs(np.asarray(x_f32, np.float32)), axis=0)
    return (np.maximum(amax, AMAX_FLOOR) / np.float32(fmax)).astype(np.float32)


def quantize_cols(x_f32, s, fmt) -> np.ndarray:
    q = (np.asarray(x_f32, np.float32) / np.asarray(s, np.float32)[None, :]).astype(np.float32)
    return F.encode(q, fmt)


#: decoded values times these factors are integers (multiples of 2^-9 / 2^-16)
_INT_SHIFT = {F.E4M3: 9, F.E5M2: 16}


@dataclass
class TgmmResult:
    drhs: np.ndarray            # f32 [G, Kc, Nc] (selected columns)
    drhs_f64: np.ndarray        # f64 before the final f32 rounding
    absum: np.ndarray           # sum_t sL sD sum_r |dec qL dec qD|
    tiles: list                 # TgmmTile list (order of the scale rows)
    sL: np.ndarray              # f32 [T, Kc]
    sD: np.ndarray              # f32 [T, Nc]


def tgmm_quant(lhs_bits, dout_bits, group_sizes, grad_fmt: str, tile_m: int = 512,
               k_cols=None, n_cols=None, exact: bool = True) -> TgmmResult:
    """Weight-gradient tgmm with in-kernel operand quantization:
    ``drhs[g] = sum_t (sum_{r in T} dec(qL[r,:])^T dec(qD[r,:])) * (sL[t] x sD[t])``
    where for each non-empty (expert, tile) pair T the lhs is quantized to e4m3
    with one scale per lhs channel and dout to the gradient format with one
    scale per dout channel, both over T's rows only ("MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype", What:
    moe_bwd_inkernel_quant and bwd_quantization_dtype).  The tile sums are exact
    integer sums; scaling and the sum over tiles are float64, rounded once to
    f32.  An expert without rows gets exact zeros.

    ``k_cols``/``n_cols`` restrict the output to some columns; every channel's
    scale depends only on its own column, so the restriction is exact.

    ``exact=False`` forms the tile sums with a float64 matrix product of the
    same integer-valued operands instead of int64 arithmetic (for the largest
    shapes): every product is exact in float64, and a sum of at most
    ``tile_m`` of them is within ``tile_m * 2**-53`` of the sum of their
    magnitudes, far below the f32 rounding of the result.
    """
    lhs_bits = np.asarray(lhs_bits); dout_bits = np.asarray(dout_bits)
    M, K = lhs_bits.shape
    M2, N = dout_bits.shape
    assert M2 == M
    G = len(group_sizes)
    kc = np.arange(K) if k_cols is None else np.asarray(k_cols)
    nc = np.arange(N) if n_cols is None else np.asarray(n_cols)
    tiles = tgmm_tiles(group_sizes, M, tile_m)
    acc = np.zeros((G, len(kc), len(nc)))
    absum = np.zeros((G, len(kc), len(nc)))
    sLs = np.zeros((len(tiles), len(kc)), np.float32)
    sDs = np.zeros((len(tiles), len(nc)), np.float32)
    fmax_g = F.FMAX[grad_fmt]
    for i, tl in enumerate(tiles):
        xl = F.bf16_to_f32(lhs_bits[tl.row0:tl.row1][:, kc])
        xd = F.bf16_to_f32(dout_bits[tl.row0:tl.row1][:, nc])
        sL = column_scales(xl, 448.0)
        sD = column_scales(xd, fmax_g)
        qL = quantize_cols(xl, sL, F.E4M3)
        qD = quantize_cols(xd, sD, grad_fmt)
        iL = (F.decode(qL, F.E4M3) * 2.0 ** _INT_SHIFT[F.E4M3]).astype(np.int64)
        iD = (F.decode(qD, grad_fmt) * 2.0 ** _INT_SHIFT[grad_fmt]).astype(np.int64)
        if not exact:
            iL, iD = iL.astype(np.float64), iD.astype(np.float64)
        tile_sum = (iL.T @ iD).astype(np.float64) * 2.0 ** -(_INT_SHIFT[F.E4M3] + _INT_SHIFT[grad_fmt])
        tile_abs = (np.abs(iL).T @ np.abs(iD)).astype(np.float64) * 2.0 ** -(_INT_SHIFT[F.E4M3] + _INT_SHIFT[grad_fmt])
        outer = sL.astype(np.float64)[:, None] * sD.astype(np.float64)[None, :]
        acc[tl.group] += tile_sum * outer
        absum[tl.group] += tile_abs * outer
        sLs[i], sDs[i] = sL, sD
    return TgmmResult(acc.astype(np.float32), acc, absum, tiles, sLs, sDs)


# --------------------------------------------------------------------------- dSwiGLU

def dswiglu(dprod: np.ndarray, gate: np.ndarray, up: np.ndarray):
    """Gradients of ``silu(gate) * up`` with respect to gate and up, given the
    gradient ``dprod`` of the product, in float64 ("MoE: native FP8 QAT for routed-expert GMMs", Implementation:
    gmm_dswiglu_fp8 is the wo op whose backward carries the SwiGLU derivative;
    the derivative itself is calculus on the forward SwiGLU above).

    With sigma(z) = 1 / (1 + exp(-z)) and silu(z) = z * sigma(z):
    silu'(z) = sigma(z) + z * sigma(z) * (1 - sigma(z)), so
    ``d_gate = dprod * up * silu'(gate)`` and ``d_up = dprod * silu(gate)``.
    """
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-gate))
    dsilu = sig * (1.0 + gate * (1.0 - sig))
    return dprod * up * dsilu, dprod * gate * sig


@dataclass
class DswigluResult:
    rows: np.ndarray
    group: np.ndarray
    dh: np.ndarray       # f64 wo dLHS before any rounding [R, I]
    dh_absum: np.ndarray # sum_n |dout * w|   [R, I]
    y: np.ndarray        # f64 [R, 2I]: [d_gate | d_up] before the bf16 rounding
    out: np.ndarray      # bf16 bits [R, 2I]


def gmm_dswiglu(dout_bits, codes, scale, group_sizes, preact_bits, *, rows=None) -> DswigluResult:
    """wo backward dLHS with the SwiGLU derivative fused after it ("MoE: native FP8 QAT for routed-expert GMMs",
    Implementation: gmm_dswiglu_fp8 for wo; _run_wo_gmm_dswiglu).

    ``codes``/``scale`` are the wo weight ``[G, I, H]``; ``dout`` is the wo
    output gradient ``[M, H]``; ``preact`` is the wi pre-activation
    ``[M, 2I]`` (bf16, ``[gate | up]``) kept by the forward.  The wo dLHS
    ``dh = dout @ dequantize(codes, scale)^T`` stays unrounded (float64 here)
    and only the two gradients are rounded to bf16:
    ``out = bf16([dh * up * silu'(gate) | dh * silu(gate)])``.
    """
    preact_bits = np.asarray(preact_bits)
    G, I, H = codes.shape
    M = np.asarray(dout_bits).shape[0]
    assert preact_bits.shape == (M, 2 * I)
    dl = gmm_dlhs(dout_bits, codes, scale, group_sizes, rows=rows)
    z = F.bf16_to_f64(preact_bits[dl.rows])
    dg, du = dswiglu(dl.y, z[:, :I], z[:, I:])
    y = np.concatenate([dg, du], axis=1)
    return DswigluResult(dl.rows, dl.group, dl.y, dl.absum, y, F.f64_to_bf16_bits(y))


# --------------------------------------------------------------------------- MoE FFN

#: bf16 NaN written to buffer rows an op does not produce (never read)
_STALE_BF16 = np.uint16(0x7FC0)


def _full_rows(valid_bits: np.ndarray, M: int) -> np.ndarray:
    out = np.full((M, valid_bits.shape[1]), _STALE_BF16, dtype=np.uint16)
    out[:valid_bits.shape[0]] = valid_bits
    return out


@dataclass
class FfnResult:
    fwd_wi: FwdResult          # wi forward with SwiGLU (out = h, y = pre-activation)
    preact: np.ndarray         # bf16 bits [Mv, 2I]: the pre-activation the backward reads
    h: np.ndarray              # bf16 bits [Mv, I]
    fwd_wo: FwdResult          # wo forward (out = y)
    dsw: DswigluResult         # wo dLHS + dSwiGLU (out = d preact)
    dx: DlhsResult             # wi dLHS (out = dx)
    dwo: TgmmResult            # [G, I, H]
    dwi: TgmmResult            # [G, H, 2I]


def moe_ffn(x_bits, wi_codes, wi_scale, wo_codes, wo_scale, group_sizes, dy_bits, grad_fmt: str,
            tile_m: int = 512) -> FfnResult:
    """Forward and backward of one routed-expert FFN on a static ragged buffer
    ("MoE: native FP8 QAT for routed-expert GMMs", Implementation: gmm_up_or_silu runs gmm_silu_fp8 for wi and
    _run_wo_gmm_dswiglu runs gmm_dswiglu_fp8 for wo; "MoE fp8 backward: in-kernel drhs operand quantization + configurable gradient dtype", What: both weight
    gradients are tgmm with in-kernel operand quantization).

    x ``[M, H]``, wi ``[G, H, 2I]``, wo ``[G, I, H]``, dy ``[M, H]`` (the
    gradient of the FFN output).  Steps, each an oracle op above:
      1. wi forward with SwiGLU: h = bf16(silu(gate) * up); the pre-activation
         [gate | up] is kept as bf16 for the backward;
      2. wo forward: y = gmm_fwd(h, wo);
      3. wo dLHS + dSwiGLU: d_preact = gmm_dswiglu(dy, wo, preact);
      4. wi dLHS: dx = gmm_dlhs(d_preact, wi);
      5. weight gradients: dwo = tgmm(h, dy), dwi = tgmm(x, d_preact).
    """
    x_bits = np.asarray(x_bits)
    M = x_bits.shape[0]
    fwd_wi = gmm_fwd(x_bits, wi_codes, wi_scale, group_sizes, swiglu_out=True)
    preact = F.f64_to_bf16_bits(fwd_wi.y)
    h = fwd_wi.out
    h_full = _full_rows(h, M)
    fwd_wo = gmm_fwd(h_full, wo_codes, wo_scale, group_sizes)
    dsw = gmm_dswiglu(dy_bits, wo_codes, wo_scale, group_sizes, _full_rows(preact, M))
    dz_full = _full_rows(dsw.out, M)
    dx = gmm_dlhs(dz_full, wi_codes, wi_scale, group_sizes)
    dwo = tgmm_quant(h_full, dy_bits, group_sizes, grad_fmt, tile_m)
    dwi = tgmm_quant(x_bits, dz_full, group_sizes, grad_fmt, tile_m)
    return FfnResult(fwd_wi, preact, h, fwd_wo, dsw, dx, dwo, dwi)


# --------------------------------------------------------------------------- LHS-quant variants

LHS_BLOCK = 512


@dataclass
class VariantResult(FwdResult):
    totals: np.ndarray = None   # [n_blocks, R, N]: the running total after each block (bf16 values with acc_bf16)


def gmm_fwd_variant(lhs_bits, codes, scale, group_sizes, *, block: int = 0, scale_bf16: bool = False,
                    acc_bf16: bool = False, rhs_scale_first: bool = False, rows=None) -> VariantResult:
    """The forward's LHS-quantization options kept as ops-level arguments for
    benchmarks and tests ("MoE: native FP8 QAT for routed-expert GMMs", Implementation: lhs_quant_block_size 512 or the
    full K, lhs_f32_scale, rhs_scale_first; review thread on the conversation page of "MoE: native FP8 QAT for routed-expert GMMs" on the defaults:
    a bf16 scale per 512-column block with a bf16 accumulator was the earlier
    default).

    * ``block``: columns per activation scale (0 = the full K).  Each row's K
      axis is cut into blocks of ``block`` columns (the last may be shorter);
      every block b gets ``s_b = f32(max(amax_b, 1e-12) / 448)``, rounded once
      more to bf16 with ``scale_bf16``; its codes are ``e4m3(f32(x / s_b))``.
    * block contribution ``t_b[n] = (P_b[n] * s_b) * scale[n]`` with
      ``P_b = sum_{k in b} dec(q) dec(c)`` (exact); with ``rhs_scale_first``
      the weight scale is applied first.  Both orders are the same real number:
      the option only moves an f32 rounding, which float64 does not model.
    * accumulation over blocks: float64 sum, or with ``acc_bf16`` a bf16
      accumulator ``a <- bf16(f32(a + t_b))`` in block order.
    * output ``bf16(sum)`` (``a`` itself with ``acc_bf16``).

    ``FwdResult.act_scale`` holds the scales [R, n_blocks]; ``absum`` the sum
    over blocks of ``s_b |scale| sum |dec q dec c|``.
    """
    lhs_bits = np.asarray(lhs_bits)
    M, K = lhs_bits.shape
    G, K2, N = codes.shape
    assert K2 == K and scale.shape == (G, N)
    bw = K if block <= 0 else block
    edges = list(range(0, K, bw)) + [K]
    nb = len(edges) - 1
    lay = layout(group_sizes, M)
    gid = lay.group_of_rows(M)
    if rows is None:
        rows = np.arange(lay.valid, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    assert np.all(gid[rows] >= 0), "requested rows must be valid rows"
    R = len(rows)
    y = np.zeros((R, N)); absum = np.zeros((R, N)); acc = np.zeros((R, N))
    act_codes = np.zeros((R, K), np.uint8); act_scale = np.zeros((R, nb), np.float32)
    totals = np.zeros((nb, R, N))
    for g in range(G):
        sel = np.nonzero(gid[rows] == g)[0]
        if len(sel) == 0:
            continue
        x = F.bf16_to_f32(lhs_bits[rows[sel]])
        cd = F.decode(codes[g], F.E4M3)
        sc = scale[g].astype(np.float64)
        a = np.zeros((len(sel), N))
        for b in range(nb):
            k0, k1 = edges[b], edges[b + 1]
            s = row_scales(x[:, k0:k1])
            if scale_bf16:
                s = F.round_to_bf16(s.astype(np.float64)).astype(np.float32)
            q = quantize_rows(x[:, k0:k1], s)
            qd = F.decode(q, F.E4M3)
            t = (qd @ cd[k0:k1]) * s.astype(np.float64)[:, None] * sc[None, :]
            absum[sel] += (np.abs(qd) @ np.abs(cd[k0:k1])) * s.astype(np.float64)[:, None] * np.abs(sc)[None, :]
            y[sel] += t
            if acc_bf16:
                a = F.round_to_bf16(F.round_to_f32(a + t))
            totals[b, sel] = a if acc_bf16 else y[sel]
            act_codes[sel, k0:k1] = q
            act_scale[sel, b] = s
        acc[sel] = a
    out_f64 = acc if acc_bf16 else y
    return VariantResult(rows, gid[rows], y, absum, F.f64_to_bf16_bits(out_f64), out_f64, act_codes, act_scale,
                         totals)


def fake_qat_reference(lhs_bits, codes, scale, group_sizes, rows=None) -> np.ndarray:
    """What the quantized forward approximates: the bf16 activations times the
    weights code * scale, exactly (float64), per valid row ("MoE: native FP8 QAT for routed-expert GMMs", Why: fake QAT
    runs bf16 GMMs on dequantized weights)."""
    lhs_bits = np.asarray(lhs_bits)
    M = lhs_bits.shape[0]
    lay = layout(group_sizes, M)
    gid = lay.group_of_rows(M)
    rows = np.arange(lay.valid, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((len(rows), codes.shape[2]))
    for g in range(codes.shape[0]):
        sel = np.nonzero(gid[rows] == g)[0]
        if len(sel):
            w = F.decode(codes[g], F.E4M3) * scale[g].astype(np.float64)[None, :]
            out[sel] = F.bf16_to_f64(lhs_bits[rows[sel]]) @ w
    return out


# --------------------------------------------------------------------------- dense backward quantization

def tgmm_dense(lhs_bits, dout_bits, group_sizes, grad_fmt: str, k_cols=None, n_cols=None) -> TgmmResult:
    """The buffer-wide backward quantization that the in-kernel tgmm replaces
    ("MoE fp8 backward: in-kernel drhs operand quantization + configurable
    gradient dtype", What).  That page describes three operations sized by the
    static buffer rather than by the valid rows: each lhs row is quantized
    again with its own scale, that row scale is multiplied into the gradient,
    and the gradient gets one scale per output column.  Because stale rows take
    part, an infinite value in one of them makes a column scale infinite, and
    the rescaled product of an infinite scale with a zero code is NaN.

    Over every row of the static buffer, stale rows included:
      sL[r]   = f32(max(amax_k |lhs[r,k]|, 1e-12) / 448),  qL = e4m3(f32(lhs / sL))
      d'[r,n] = f32(dout[r,n] * sL[r])
      sD[n]   = f32(max(amax_r |d'[r,n]|, 1e-12) / FMAX),  qD = grad(f32(d' / sD))
    and per expert ``drhs[g,k,n] = sD[n] * sum_{r in g} dec(qL[r,k]) dec(qD[r,n])``
    (exact integer sums, float64, rounded once to f32).  The amax ignores NaN
    (IEEE maxNum, as a max instruction does); an expert without rows gets zeros.
    ``sL`` of the result holds the row scales [M] (as [1, M]), ``sD`` the
    column scales [1, N].  ``k_cols``/``n_cols`` restrict the output to some
    columns: the row scales still span all of K, and a gradient column's
    scale depends on that column alone, so the restriction is exact.
    """
    lhs_bits = np.asarray(lhs_bits); dout_bits = np.asarray(dout_bits)
    M, K = lhs_bits.shape
    N = dout_bits.shape[1]
    G = len(group_sizes)
    lay = layout(group_sizes, M)
    x = F.bf16_to_f32(lhs_bits)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        amax_r = np.fmax.reduce(np.abs(x), axis=1) if K else np.zeros(M, np.float32)
        sL = (np.maximum(np.nan_to_num(amax_r, nan=0.0, posinf=np.inf), AMAX_FLOOR) / E4M3_MAX).astype(np.float32)
        if k_cols is not None:
            x = x[:, np.asarray(k_cols)]
        qL = F.encode((x / sL[:, None]).astype(np.float32), F.E4M3)
        d = F.bf16_to_f32(dout_bits if n_cols is None else np.asarray(dout_bits)[:, np.asarray(n_cols)])
        dp = (d * sL[:, None]).astype(np.float32)
        amax_n = np.fmax.reduce(np.abs(dp), axis=0)
        sD = (np.maximum(np.nan_to_num(amax_n, nan=0.0, posinf=np.inf), AMAX_FLOOR)
              / np.float32(F.FMAX[grad_fmt])).astype(np.float32)
        qD = F.encode((dp / sD[None, :]).astype(np.float32), grad_fmt)
    K, N = x.shape[1], d.shape[1]
    acc = np.zeros((G, K, N)); absum = np.zeros((G, K, N))
    sh = _INT_SHIFT[F.E4M3] + _INT_SHIFT[grad_fmt]
    for g in range(G):
        a, b = int(lay.start[g]), int(lay.end[g])
        if b == a:
            continue
        dl = F.decode(qL[a:b], F.E4M3)
        dd = F.decode(qD[a:b], grad_fmt)
        with np.errstate(invalid="ignore"):
            iL = np.where(np.isfinite(dl), dl * 2.0 ** _INT_SHIFT[F.E4M3], 0).astype(np.int64)
            iD = np.where(np.isfinite(dd), dd * 2.0 ** _INT_SHIFT[grad_fmt], 0).astype(np.int64)
            s = (iL.T @ iD).astype(np.float64) * 2.0 ** -sh
            sa = (np.abs(iL).T @ np.abs(iD)).astype(np.float64) * 2.0 ** -sh
            # a NaN code anywhere in the expert's rows makes the sums NaN
            nanL = ~np.isfinite(dl); nanD = ~np.isfinite(dd)
            if nanL.any() or nanD.any():
                bad = (nanL.astype(np.int64).T @ np.ones_like(iD) + np.ones_like(iL).T @ nanD.astype(np.int64)) > 0
                s = np.where(bad, np.nan, s)
            acc[g] = s * sD.astype(np.float64)[None, :]
            absum[g] = sa * np.abs(sD.astype(np.float64))[None, :]
    return TgmmResult(acc.astype(np.float32), acc, absum, [], sL[None, :], sD[None, :])
