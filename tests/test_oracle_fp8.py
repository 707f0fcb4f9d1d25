"""Pins for the oracle's FP8 E4M3 codec and per-tensor quantizer.

The codec is checked against an independent brute force: every finite E4M3
magnitude is enumerated from its fields with exact rationals, and each input
is matched to the nearest one (ties to the even mantissa, saturating at the
largest finite value).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import fp8


def _e4m3_magnitudes():
    """(value Fraction, code) for all finite non-negative E4M3 codes."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                          # NaN
            if e == 0:
                v = Fraction(m, 8) * Fraction(1, 64)
            else:
                v = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            out.append((v, (e << 3) | m))
    return out


MAGS = _e4m3_magnitudes()


def _nearest_code(q):
    """Brute-force nearest E4M3 code for an exact value q (Fraction or float)."""
    qf = Fraction(q)
    a = abs(qf)
    best = None
    for v, c in MAGS:
        d = abs(a - v)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1)):
            best = (d, c)
    sign = 1 if (qf < 0 or (qf == 0 and math.copysign(1.0, float(q)) < 0)) else 0
    return (sign << 7) | best[1]


def test_decode_known_codes():
    d = oracle.e4m3_decode(np.array([0x7E, 0x01, 0x08, 0x38, 0x80, 0xFE, 0x07], dtype=np.uint8))
    assert d[0] == 448.0 and d[1] == 2.0 ** -9 and d[2] == 2.0 ** -6
    assert d[3] == 1.0 and d[4] == 0.0 and math.copysign(1.0, d[4]) == -1.0
    assert d[5] == -448.0 and d[6] == 7 * 2.0 ** -9
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_decode_matches_field_enumeration():
    for v, c in MAGS:
        assert oracle.e4m3_decode(np.uint8(c)) == float(v)
        assert oracle.e4m3_decode(np.uint8(c | 0x80)) == -float(v)


def test_encode_exhaustive_bf16_against_nearest_search():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).view(np.float32).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    codes = oracle.e4m3_encode(vals)
    # far above the largest finite magnitude the nearest code is +-448; float64
    # distances there are too coarse to compare, so check saturation directly
    big = np.abs(vals) > 1024.0
    assert np.array_equal(codes[big], np.where(vals[big] < 0, 0xFE, 0x7E).astype(np.uint8))
    vals, codes = vals[~big], codes[~big]
    # vectorised nearest search over the finite magnitudes, ties to even code
    mags = np.array([float(v) for v, _ in MAGS])
    mcode = np.array([c for _, c in MAGS])
    a = np.abs(vals)[:, None]
    dist = np.abs(a - mags[None, :])
    dmin = dist.min(axis=1, keepdims=True)
    cand = dist == dmin
    # among tied candidates prefer an even mantissa
    even = (mcode % 2 == 0)[None, :]
    pick = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    expect = mcode[pick] | (np.signbit(vals).astype(np.int64) << 7)
    assert np.array_equal(codes.astype(np.int64), expect)


def test_encode_scalar_brute_force_ties_and_saturation():
    cases = [0.0, -0.0, 1.9375, 1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 464.0, 465.0,
             1e30, -1e30, 2.0 ** -6 - 2.0 ** -10, 0.01171875, -240.0, 17.0]
    for q in cases:
        got = int(oracle.e4m3_encode(np.array([q]))[0])
        assert got == _nearest_code(q), q


def test_decode_encode_identity_and_monotone():
    allc = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    v = oracle.e4m3_decode(allc)
    assert np.array_equal(oracle.e4m3_encode(v), allc)
    rng = np.random.default_rng(2)
    x = np.sort(rng.normal(0, 100, 20000).astype(np.float32).astype(np.float64))
    dec = oracle.e4m3_decode(oracle.e4m3_encode(x))
    assert np.all(np.diff(dec) >= 0)


def _rn_f32(fr):
    """Exact round-to-nearest-even of a Fraction to binary32 (normal range)."""
    if fr == 0:
        return 0.0
    s = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * float(fl * ulp)


def test_fp32_quotients_are_correctly_rounded():
    rng = np.random.default_rng(7)
    v = rng.normal(0, 3, 400).astype(np.float32)
    amax = float(np.max(np.abs(v)))
    s = fp8.f32_scale(amax)
    assert s == _rn_f32(Fraction(amax) / 448)
    q = (v.astype(np.float64) / s).astype(np.float32)
    for vi, qi in zip(v, q):
        assert float(qi) == _rn_f32(Fraction(float(vi)) / Fraction(s))


def test_quant_per_tensor_properties():
    rng = np.random.default_rng(3)
    v = rng.normal(0, 1, 5000).astype(np.float32).astype(np.float64)
    codes, s, amax = oracle.quant_per_tensor(v)
    assert amax == np.max(np.abs(v))
    i = int(np.argmax(np.abs(v)))
    assert codes[i] == (0xFE if v[i] < 0 else 0x7E)       # amax lands on +-448
    deq = oracle.e4m3_decode(codes) * s
    # error at most half an E4M3 step of the scaled value (relative 2^-4), or
    # half the subnormal step
    err = np.abs(deq - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
    assert np.all(err <= bound)
    z, s0, a0 = oracle.quant_per_tensor(np.zeros(7))
    assert s0 == 1.0 and a0 == 0.0 and not z.any()
    with pytest.raises(ValueError):
        oracle.quant_per_tensor(np.array([0.1]))          # not fp32-representable
