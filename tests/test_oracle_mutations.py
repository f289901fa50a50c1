"""Plants plausible mistakes in the oracle (on the CPU, via monkeypatch) and
checks that at least one pin catches each, so the pins are known to bite."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import gmm as O
from tests import test_oracle_dense as TE
from tests import test_oracle_dswiglu as TD
from tests import test_oracle_formats as TF
from tests import test_oracle_gmm as TG
from tests import test_oracle_variants as TV

PINS = [
    TG.test_golden_worked_example,
    TG.test_scale_zero_row_and_powers_of_two,
    TG.test_quotient_rounding_at_scale,
    lambda: TG.test_forward_brute_force((0, 5, 4)),
    TG.test_forward_swiglu_brute_force,
    TG.test_activation_codes_brute_force,
    TG.test_forward_lossless_construction,
    TG.test_forward_group_split_and_permutation,
    TG.test_layout_clamp_and_negative,
    TG.test_dequant_matches_torch_and_exact_cases,
    TG.test_dlhs_one_hot_selects_weight_column,
    TG.test_dlhs_brute_force,
    lambda: TG.test_tgmm_brute_force(F.E5M2),
    lambda: TG.test_tgmm_brute_force(F.E4M3),
    lambda: TG.test_tgmm_lossless_construction(F.E5M2),
    TG.test_tgmm_stale_tail_and_tiles,
    TF.test_encode_specials,
    lambda: TF.test_encode_roundtrip_all_finite_codes(F.E4M3),
    TF.test_bf16_specials,
    TD.test_dswiglu_matches_autograd_and_finite_differences,
    TD.test_dswiglu_closed_forms,
    TD.test_gmm_dswiglu_is_gradient_of_wo_loss,
    lambda: TD.test_moe_ffn_matches_straight_through_gradient(F.E4M3),
    lambda: TV.test_variant_brute_force(True, True),
    TV.test_equal_block_amax_reduces_to_full_k,
    lambda: TE.test_dense_brute_force(F.E5M2),
    TE.test_stale_inf_poisons_dense_but_not_in_kernel,
]


def _mut_scale_240(x):
    x = np.asarray(x, np.float32)
    return (np.maximum(np.max(np.abs(x), axis=1), O.AMAX_FLOOR) / np.float32(240)).astype(np.float32)


def _mut_scale_no_floor(x):
    x = np.asarray(x, np.float32)
    return (np.max(np.abs(x), axis=1) / np.float32(448)).astype(np.float32)


def _mut_quant_reciprocal(x, s):
    r = (np.float32(1) / np.asarray(s, np.float32)).astype(np.float32)
    return F.encode((np.asarray(x, np.float32) * r[:, None]).astype(np.float32), F.E4M3)


_real_encode = F.encode


def _mut_encode_ties_away(values, fmt):
    v = np.asarray(values, np.float64)
    out = _real_encode(v, fmt)
    d = F.DECODE[fmt]
    a = np.abs(v)
    pos = d[: F.MAX_CODE[fmt] + 1]
    hi = np.clip(np.searchsorted(pos, a), 1, F.MAX_CODE[fmt])
    tie = (pos[hi] - a) == (a - pos[hi - 1])
    out = np.where(tie & (a < F.FMAX[fmt]), (hi | (np.signbit(v) << 7)).astype(np.uint8), out)
    return out.astype(np.uint8)


def _mut_encode_no_saturation(values, fmt):
    v = np.asarray(values, np.float64)
    out = _real_encode(v, fmt)
    return np.where(np.abs(v) > F.FMAX[fmt], np.uint8(0x7F), out).astype(np.uint8)


_real_layout = O.layout


def _mut_layout_shift(gs, M):
    lay = _real_layout(gs, M)
    lay.start = np.minimum(lay.start + (lay.start > 0), lay.end)
    return lay


_real_swiglu = O.swiglu
_real_tiles = O.tgmm_tiles
_real_col_scales = O.column_scales
_real_fwd_rows = O._fwd_rows
_real_dequant = O.dequantize
_real_dswiglu = O.dswiglu
_real_variant = O.gmm_fwd_variant
_real_dense = O.tgmm_dense


def _mut_dense_valid_rows_only(lhs, dout, gs, fmt):
    mv = O.layout(gs, np.asarray(lhs).shape[0]).valid
    return _real_dense(np.asarray(lhs)[:mv], np.asarray(dout)[:mv], gs, fmt)
_real_gmm_dswiglu = O.gmm_dswiglu


def _mut_dswiglu_sigma_only(d, g, u):
    sig = 1.0 / (1.0 + np.exp(-np.clip(g, -700, 700)))
    return d * u * sig, d * g * sig


def _mut_dswiglu_outputs_swapped(d, g, u):
    dg, du = _real_dswiglu(d, g, u)
    return du, dg


def _mut_dswiglu_preact_halves_swapped(dout, codes, scale, gs, preact, rows=None):
    p = np.asarray(preact)
    I = p.shape[1] // 2
    return _real_gmm_dswiglu(dout, codes, scale, gs, np.concatenate([p[:, I:], p[:, :I]], axis=1), rows=rows)


def _mut_tiles_group_aligned(gs, M, tile_m):
    lay = _real_layout(gs, M)
    out = []
    for g in range(len(lay.start)):
        a, b = int(lay.start[g]), int(lay.end[g])
        for i, r0 in enumerate(range(a, b, tile_m)):
            out.append(O.TgmmTile(g, i, r0, min(b, r0 + tile_m)))
    return out


def _mut_grad_scale_448(x, fmax):
    return _real_col_scales(x, 448.0)


def _mut_scale_first_channel(x_bits, codes_g, scale_g):
    return _real_fwd_rows(x_bits, codes_g, np.full_like(scale_g, scale_g[0]))


def _mut_dequant_f64_product(codes, scale):
    w = F.decode(codes, F.E4M3) * np.asarray(scale, np.float64)[:, None, :]
    return F.f64_to_bf16_bits(w)


def _mut_bf16_truncate(x):
    x = np.asarray(x, np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    ue = np.maximum(e - 8, -133)
    out[fin] = np.ldexp(np.trunc(np.ldexp(x[fin], -ue)), ue)
    return out


MUTATIONS = {
    "scale divisor 240": (O, "row_scales", _mut_scale_240),
    "scale without 1e-12 floor": (O, "row_scales", _mut_scale_no_floor),
    "quantize by reciprocal multiply": (O, "quantize_rows", _mut_quant_reciprocal),
    "encode ties away from zero": (F, "encode", _mut_encode_ties_away),
    "encode without saturation": (F, "encode", _mut_encode_no_saturation),
    "group offsets off by one": (O, "layout", _mut_layout_shift),
    "swiglu operands swapped": (O, "swiglu", lambda g, u: _real_swiglu(u, g)),
    "tgmm tiles aligned to expert start": (O, "tgmm_tiles", _mut_tiles_group_aligned),
    "gradient scale uses 448": (O, "column_scales", _mut_grad_scale_448),
    "weight scale of channel 0 only": (O, "_fwd_rows", _mut_scale_first_channel),
    "dequant product in f64": (O, "dequantize", _mut_dequant_f64_product),
    "bf16 rounding truncates": (F, "round_to_bf16", _mut_bf16_truncate),
    "dswiglu drops the z sigma (1 - sigma) term": (O, "dswiglu", _mut_dswiglu_sigma_only),
    "dswiglu gate and up gradients swapped": (O, "dswiglu", _mut_dswiglu_outputs_swapped),
    "dswiglu reads the pre-activation halves swapped": (O, "gmm_dswiglu", _mut_dswiglu_preact_halves_swapped),
    "dswiglu sign flipped": (O, "dswiglu", lambda d, g, u: tuple(-v for v in _real_dswiglu(d, g, u))),
    "variant ignores the bf16 accumulator": (O, "gmm_fwd_variant",
                                             lambda *a, **kw: _real_variant(*a, **{**kw, "acc_bf16": False})),
    "variant ignores the bf16 scale": (O, "gmm_fwd_variant",
                                       lambda *a, **kw: _real_variant(*a, **{**kw, "scale_bf16": False})),
    "dense quantization skips the stale rows": (O, "tgmm_dense", _mut_dense_valid_rows_only),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"no pin caught the planted mistake: {name}"
