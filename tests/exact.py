"""Exact rational arithmetic for brute-force pins of the oracle.

Independent of ``oracle/``: rounding is done on ``fractions.Fraction`` values
with integer arithmetic, and the 8-bit formats' values come from torch's own
float8 dtypes, not from the oracle's decode table.
"""
from __future__ import annotations

import functools
import math
from fractions import Fraction

import numpy as np
import torch


def floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    r = q - fl
    if r > Fraction(1, 2):
        return fl + 1
    if r < Fraction(1, 2):
        return fl
    return fl + (fl % 2)


def round_binary(x: Fraction, p: int, emin: int, max_finite: Fraction | None = None) -> Fraction | float:
    """Round to nearest (ties to even significand) in a binary format with p
    significant bits and smallest normal exponent emin; beyond the overflow
    threshold returns +-inf."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = max(floor_log2(a), emin)
    unit = Fraction(2) ** (e - p + 1)
    n = round_half_even(a / unit)
    r = n * unit
    if max_finite is not None and r > max_finite:
        return s * math.inf
    return s * r


F32_MAX = Fraction((2 ** 24 - 1)) * Fraction(2) ** (127 - 23)
BF16_MAX = Fraction((2 ** 8 - 1)) * Fraction(2) ** (127 - 7)


def to_f32(x: Fraction) -> Fraction:
    return round_binary(x, 24, -126, F32_MAX)


def to_bf16(x: Fraction) -> Fraction:
    return round_binary(x, 8, -126, BF16_MAX)


@functools.lru_cache(maxsize=None)
def torch_table(fmt: str):
    """(code, Fraction value) for every finite code, from torch's float8 dtypes."""
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    vals = torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float64).numpy()
    return [(c, Fraction(float(v))) for c, v in enumerate(vals) if np.isfinite(v)], vals


def encode_brute(x, fmt: str) -> int:
    """Nearest finite code by exhaustive search, ties to the even code,
    saturating at the largest finite magnitude; sign kept on zero."""
    table, _ = torch_table(fmt)
    fmax = max(v for _, v in table)
    if isinstance(x, float) and math.isnan(x):
        return 0x7F
    neg = (x < 0) or (isinstance(x, float) and math.copysign(1.0, x) < 0)
    a = abs(Fraction(x)) if not (isinstance(x, float) and math.isinf(x)) else None
    if a is None or a >= fmax:
        mag = max(c for c, v in table if v == fmax and c < 0x80)
        return mag | (0x80 if neg else 0)
    best = None
    for c, v in table:
        if c >= 0x80:
            continue
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if neg else 0)


def bf16_bits_of(v: Fraction) -> int:
    """bf16 bit pattern of an exactly representable bf16 value."""
    return int(np.array([float(v)], np.float32).view(np.uint32)[0] >> 16)
