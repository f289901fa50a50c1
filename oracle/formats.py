"""Number formats used by the routed-expert FP8 grouped matmul, written out from
their definitions.

Test infrastructure only: nothing on the product path imports this module.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.

Sources
-------
* The weight codes are ``float8_e4m3fn`` and the gradient code of the tgmm is
  ``e5m2`` or ``e4m3`` ("MoE: native FP8 QAT for routed-expert GMMs", Data flow
  table: FP8 codes stored as float8_e4m3fn; "MoE fp8 backward: in-kernel drhs
  operand quantization + configurable gradient dtype", What: bwd_quantization_dtype).
* Bit layouts follow the OCP 8-bit floating point specification (OFP8):
  E4M3 has bias 7, no infinities, a single NaN mantissa (S.1111.111) and a
  largest finite magnitude of 448; E5M2 has bias 15, IEEE-style infinities and
  NaNs and a largest finite magnitude of 57344.
* Encoding rounds to nearest with ties to the even code and saturates
  out-of-range magnitudes (including infinities) to the largest finite code;
  a negative value that rounds to zero keeps its sign.  The pages only name the
  dtype; saturation and round-to-nearest-even are the OCP conversion mode with
  saturation, the plainest reading for a quantizer whose scale maps the row
  maximum onto 448.
* bfloat16 is binary32 with the low 16 bits removed; conversions round to
  nearest, ties to even.

All arithmetic here is in float64, in which every e4m3/e5m2/bf16/f32 value and
every midpoint between neighbouring values of those formats is exact.
"""
from __future__ import annotations

import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"
FORMATS = (E4M3, E5M2)

#: largest finite magnitude of each format
FMAX = {E4M3: 448.0, E5M2: 57344.0}
#: code of the largest finite positive magnitude
MAX_CODE = {E4M3: 0x7E, E5M2: 0x7B}
#: canonical NaN code (sign bit added on top)
NAN_CODE = {E4M3: 0x7F, E5M2: 0x7F}


def _decode_code(code: int, fmt: str) -> float:
    """Value of one 8-bit code (OFP8 bit layout)."""
    sign = -1.0 if code & 0x80 else 1.0
    if fmt == E4M3:
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            return float("nan")
        if e == 0:
            return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    if fmt == E5M2:
        e = (code >> 2) & 0x1F
        m = code & 0x3
        if e == 0x1F:
            return sign * float("inf") if m == 0 else float("nan")
        if e == 0:
            return sign * m * 2.0 ** -16         # subnormal: m/4 * 2^(1-15)
        return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)
    raise ValueError(f"unknown format {fmt!r}")


#: decode table, float64[256] per format
DECODE = {fmt: np.array([_decode_code(c, fmt) for c in range(256)], dtype=np.float64)
          for fmt in FORMATS}


def decode(codes, fmt: str) -> np.ndarray:
    """Exact value of each code, as float64."""
    return DECODE[fmt][np.asarray(codes, dtype=np.uint8)]


def encode(values, fmt: str) -> np.ndarray:
    """Saturating round-to-nearest-even encoding of float values into codes.

    ``values`` may be float32 or float64; the rounding is done on the exact
    value.  NaN encodes to the canonical NaN code with the input's sign.
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    maxc = MAX_CODE[fmt]
    mags = DECODE[fmt][: maxc + 1]          # codes 0..maxc, strictly increasing
    hi = np.searchsorted(mags, a, side="left")
    hi = np.clip(hi, 1, maxc)
    lo = hi - 1
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    # nearest; on a tie the even code (least significant bit 0)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(take_hi, hi, lo)
    mag = np.where(a >= FMAX[fmt], maxc, mag)          # saturation, infinities included
    code = mag.astype(np.uint16) | (neg.astype(np.uint16) << 7)
    code = np.where(np.isnan(v), NAN_CODE[fmt] | (neg.astype(np.uint16) << 7), code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------- bf16

def bf16_to_f64(bits) -> np.ndarray:
    """Value of bf16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_to_f32(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 (or float32) values to the nearest bf16 value, ties to even.

    Returns the rounded values as float64.  bf16 has 8 significant bits, the
    float32 exponent range and gradual underflow (spacing 2^-133 below 2^-126).
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                       # xf = f * 2^e, 0.5 <= |f| < 1
    ulp_exp = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(xf, -ulp_exp)), ulp_exp)   # rint: ties to even
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, y), y)
    out[fin] = y
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of round_to_bf16(x); NaN maps to 0x7FC0 with its sign."""
    r = round_to_bf16(x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(r)
    bits = np.where(nan, np.uint16(0x7FC0) | (np.signbit(r).astype(np.uint16) << 15), bits)
    return bits.astype(np.uint16)


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (the gap above |x|'s binade floor)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.where(a == 0, 2.0 ** -133, ulp)


def round_to_f32(x) -> np.ndarray:
    """Round float64 values to float32 (round to nearest, ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
