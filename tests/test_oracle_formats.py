"""Pins of the oracle's number formats (oracle/formats.py) against closed-form
values of the OCP 8-bit formats, torch's float8/bfloat16 dtypes (library
cross-check) and exhaustive brute-force rounding."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import exact as X


def _torch_decode(fmt):
    dt = torch.float8_e4m3fn if fmt == F.E4M3 else torch.float8_e5m2
    return torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float64).numpy()


# ---------------------------------------------------------------- decode

E4M3_POINTS = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
               0x40: 2.0, 0x74: 192.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
E5M2_POINTS = {0x00: 0.0, 0x01: 2.0 ** -16, 0x04: 2.0 ** -14, 0x3C: 1.0, 0x7B: 57344.0, 0x7C: math.inf,
               0xFC: -math.inf, 0xBC: -1.0}


def test_decode_closed_form_points():
    for c, v in E4M3_POINTS.items():
        assert F.DECODE[F.E4M3][c] == v, hex(c)
    for c, v in E5M2_POINTS.items():
        assert F.DECODE[F.E5M2][c] == v, hex(c)
    assert np.signbit(F.DECODE[F.E4M3][0x80]) and F.DECODE[F.E4M3][0x80] == 0
    assert np.isnan(F.DECODE[F.E4M3][[0x7F, 0xFF]]).all()
    assert np.isnan(F.DECODE[F.E5M2][[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]).all()
    # the largest finite magnitudes are the quantizer's divisors
    assert F.FMAX[F.E4M3] == np.nanmax(F.DECODE[F.E4M3]) == 448.0
    assert F.FMAX[F.E5M2] == np.max(F.DECODE[F.E5M2][np.isfinite(F.DECODE[F.E5M2])]) == 57344.0


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_decode_matches_torch(fmt):
    ref = _torch_decode(fmt)
    ours = F.DECODE[fmt]
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


@pytest.mark.parametrize("fmt,nfinite", [(F.E4M3, 254), (F.E5M2, 248)])
def test_decode_monotonic_and_counts(fmt, nfinite):
    d = F.DECODE[fmt]
    assert np.isfinite(d).sum() == nfinite
    pos = d[: F.MAX_CODE[fmt] + 1]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(d[0x80: 0x80 + F.MAX_CODE[fmt] + 1], -pos)


# ---------------------------------------------------------------- encode

@pytest.mark.parametrize("fmt", F.FORMATS)
def test_encode_roundtrip_all_finite_codes(fmt):
    codes = np.array([c for c in range(256) if np.isfinite(F.DECODE[fmt][c])], np.uint8)
    assert np.array_equal(F.encode(F.DECODE[fmt][codes], fmt), codes)


def test_encode_specials():
    e = lambda v, fmt=F.E4M3: int(F.encode(np.array([v]), fmt)[0])
    assert e(448.0) == 0x7E and e(464.0) == 0x7E and e(470.0) == 0x7E and e(1e30) == 0x7E
    assert e(math.inf) == 0x7E and e(-math.inf) == 0xFE and e(-500.0) == 0xFE
    assert e(1e-9) == 0x00 and e(-1e-9) == 0x80 and e(-0.0) == 0x80
    assert e(2.0 ** -10) == 0x00                       # tie between 0 and 2^-9: even code
    assert e(3 * 2.0 ** -10) == 0x02                   # tie between codes 1 and 2
    assert e(7.5 * 2.0 ** -9) == 0x08                  # tie across the subnormal/normal edge
    assert e(1.0 + 2.0 ** -4) == 0x38                  # tie between 1.0 and 1.125: even code 0x38
    assert e(1.0 + 3 * 2.0 ** -4) == 0x3A              # tie between 1.125 (0x39) and 1.25 (0x3A)
    assert e(math.nan) == 0x7F
    assert e(57344.0, F.E5M2) == 0x7B and e(61440.0, F.E5M2) == 0x7B and e(1e9, F.E5M2) == 0x7B
    assert e(math.inf, F.E5M2) == 0x7B and e(-2.0 ** -18, F.E5M2) == 0x80
    assert e(2.0 ** -17, F.E5M2) == 0x00 and e(3 * 2.0 ** -17, F.E5M2) == 0x02


def _probe_values(fmt, n_random, seed):
    d = F.DECODE[fmt]
    pos = d[: F.MAX_CODE[fmt] + 1]
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids, [F.FMAX[fmt] * 1.03, F.FMAX[fmt] * 1.0625, F.FMAX[fmt] * 4]])
    f32 = pts.astype(np.float32)
    nb = np.concatenate([f32, np.nextafter(f32, np.float32(np.inf)), np.nextafter(f32, np.float32(0))])
    r = np.random.default_rng(seed)
    lo, hi = (-12, 10) if fmt == F.E4M3 else (-19, 17)
    rnd = (2.0 ** r.uniform(lo, hi, n_random)).astype(np.float32)
    vals = np.concatenate([nb, rnd]).astype(np.float32)
    return np.concatenate([vals, -vals])


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_encode_exhaustive_nearest(fmt):
    """Vectorised exhaustive nearest-value search (not a binary search) on all
    codes, midpoints, their f32 neighbours and 10^6 log-uniform values."""
    vals = _probe_values(fmt, 1_000_000, 11)
    d = F.DECODE[fmt]
    maxc = F.MAX_CODE[fmt]
    pos = d[: maxc + 1]
    ours = F.encode(vals, fmt)
    for s in range(0, len(vals), 50_000):
        v = vals[s:s + 50_000].astype(np.float64)
        a = np.abs(v)
        dist = np.abs(a[:, None] - pos[None, :])
        dmin = dist.min(axis=1, keepdims=True)
        cand = dist == dmin
        even = cand & (np.arange(maxc + 1)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        pick = np.where(a >= F.FMAX[fmt], maxc, pick)
        ref = (pick | (np.signbit(v) << 7)).astype(np.uint8)
        assert np.array_equal(ours[s:s + 50_000], ref)


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_encode_brute_force_rational(fmt):
    """Pure-Python exact search over torch's value table, 4000 values."""
    vals = _probe_values(fmt, 1000, 12)
    r = np.random.default_rng(13)
    vals = vals[r.choice(len(vals), min(4000, len(vals)), replace=False)]
    ours = F.encode(vals, fmt)
    for v, o in zip(vals, ours):
        assert X.encode_brute(float(v), fmt) == int(o), float(v)


@pytest.mark.parametrize("fmt", F.FORMATS)
def test_encode_matches_torch_cast_after_clamp(fmt):
    dt = torch.float8_e4m3fn if fmt == F.E4M3 else torch.float8_e5m2
    vals = _probe_values(fmt, 1_000_000, 14)
    clamped = np.clip(vals, -F.FMAX[fmt], F.FMAX[fmt]).astype(np.float32)
    ref = torch.from_numpy(clamped).to(dt).view(torch.uint8).numpy()
    assert np.array_equal(F.encode(vals, fmt), ref)


# ---------------------------------------------------------------- bf16

def test_bf16_matches_torch_cast():
    r = np.random.default_rng(21)
    u = r.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f64_to_bf16_bits(x.astype(np.float64)), ref)


def test_bf16_f64_rational():
    r = np.random.default_rng(22)
    x = r.standard_normal(3000) * 2.0 ** r.integers(-140, 127, 3000)
    for v in x:
        ref = X.to_bf16(Fraction(float(v)))
        got = F.round_to_bf16(np.array([v]))[0]
        assert (math.isinf(ref) and math.isinf(got) and (ref > 0) == (got > 0)) or Fraction(float(got)) == ref, v


def test_bf16_specials():
    rb = lambda v: float(F.round_to_bf16(np.array([v]))[0])
    assert rb(1.0 + 2.0 ** -8) == 1.0                       # tie: even
    assert rb(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6       # tie: even (up)
    assert rb(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert rb(3.3962e38) == math.inf and rb(3.39e38) == 3.3895313892515355e38
    assert rb(2.0 ** -134) == 0.0 and rb(3 * 2.0 ** -134) == 2.0 ** -132
    assert F.f64_to_bf16_bits(np.array([224.0]))[0] == 0x4360
    assert F.ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7 and F.ulp_bf16(np.array([-3.0]))[0] == 2.0 ** -6
