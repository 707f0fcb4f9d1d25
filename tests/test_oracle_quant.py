"""Pins of the oracle's BF16 -> MXFP4 weight quantiser (CPU only).

The pages describe the block quantiser's steps (gpt-oss page, "Conversion
Methodology": per-block amax, scale, E2M1 rounding, packing) but print no
quantised values, so the oracle is pinned by hand-derived rounding cases,
exact round trips, the closed form of the scale rule and the error bound of
round-to-nearest.
"""

import os

import numpy as np
import pytest

import oracle
from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_quant_cases.txt")
SMALL_BLOCK = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_small_block_case.txt")


def small_block_case():
    """The hand-worked block of tests/golden/mxfp4_small_block_case.txt:
    (values float64 [32], codes uint8 [32], scale byte)."""
    vals, codes, sbyte = [], [], None
    with open(SMALL_BLOCK) as f:
        for line in f:
            if line.startswith("# scale_byte"):
                sbyte = int(line.split()[2])
            line = line.split("#")[0].strip()
            if line:
                m, e, c = (int(t) for t in line.split())
                vals.append(np.ldexp(float(m), e))
                codes.append(c)
    v = np.zeros(32)
    c = np.zeros(32, dtype=np.uint8)
    v[:len(vals)] = vals
    c[:len(codes)] = codes
    return v, c, sbyte


def _cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                q, c = line.split()
                out.append((float(q), int(c)))
    return out


def test_rounding_cases_from_the_value_set():
    cases = _cases()
    q = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases], dtype=np.uint8)
    assert np.array_equal(quant.e2m1_nearest(q), want)


def test_scale_rule_closed_form():
    # X = floor(log2 amax) - 2: the block max lands in [4, 8) after scaling
    rng = np.random.default_rng(0)
    amax = np.ldexp(rng.uniform(1.0, 2.0, 2000), rng.integers(-100, 100, 2000))
    x = quant.block_exponent(amax)
    r = amax / np.ldexp(1.0, x)
    assert np.all((r >= 4) & (r < 8))
    # exact powers of two and the clamps
    assert quant.block_exponent(np.array([1.0, 4.0, 6.0, 7.99, 8.0]))[:].tolist() == [-2, 0, 0, 0, 1]
    assert quant.block_exponent(np.array([0.0]))[0] == -116
    assert quant.block_exponent(np.array([2.0 ** -130]))[0] == -116
    assert quant.block_exponent(np.array([2.0 ** -114]))[0] == -116
    assert quant.block_exponent(np.array([2.0 ** -115]))[0] == -116
    assert quant.block_exponent(np.array([3.3e38]))[0] == 125


def test_block_below_the_clamp_hand_worked():
    # amax = 2^-115 < 2^-114: the library's clamp (X >= -116) departs from the
    # unclamped OCP exponent (-117) here; codes and scale byte worked by hand
    v, want, sbyte = small_block_case()
    assert sbyte == 11
    b, s = oracle.quantize_mxfp4(v[None, :])
    assert s.tolist() == [[sbyte]]
    assert np.array_equal(oracle.unpack_nibbles(b)[0], want)
    # every value is a bf16 value (the quantiser's input type)
    assert np.array_equal(oracle.bf16_bits_to_f64(
        (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)), v)


def test_round_trip_of_representable_blocks():
    # every block holds a +-4 or +-6, so its amax fixes the scale it was built with
    rng = np.random.default_rng(1)
    N, K = 37, 320
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    nb = K // 32
    where = rng.integers(0, 32, (N, nb))
    big = rng.choice(np.array([6, 7, 14, 15], dtype=np.uint8), (N, nb))
    cb = codes.reshape(N, nb, 32)
    cb[np.arange(N)[:, None], np.arange(nb)[None, :], where] = big
    codes = cb.reshape(N, K)
    scales = rng.integers(11, 253, (N, nb)).astype(np.uint8)
    blocks = oracle.pack_nibbles(codes)
    w = oracle.dequant(blocks, scales)
    b2, s2 = oracle.quantize_mxfp4(w)
    assert np.array_equal(s2, scales)
    assert np.array_equal(b2, blocks)       # including -0 codes (sign kept)


def test_nearest_and_error_bound_on_random_weights():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((64, 256)) * np.ldexp(1.0, rng.integers(-20, 20, (64, 1)))
    blocks, scales = oracle.quantize_mxfp4(w)
    d = oracle.dequant(blocks, scales)
    sc = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    # brute force over all 16 codes: the chosen value is at minimal distance
    cand = oracle.E2M1_TABLE[None, None, :] * sc[..., None]
    dist = np.abs(w[..., None] - cand).min(axis=-1)
    assert np.all(np.abs(w - d) <= dist + 0.0)
    # within half the widest E2M1 gap (2, between 4 and 6) below 6 * scale, and
    # within 2 * scale in the saturated range (6, 8) * scale
    assert np.all(np.abs(w - d) <= np.where(np.abs(w) <= 6 * sc, 1.0, 2.0) * sc)
    assert np.all(np.sign(d) * np.sign(w) >= 0)


def test_zero_block_and_signs():
    w = np.zeros((2, 64))
    w[1, 32:] = -1e-40            # tiny negatives round to -0
    b, s = oracle.quantize_mxfp4(w)
    assert s.tolist() == [[11, 11], [11, 11]]
    codes = oracle.unpack_nibbles(b)
    assert np.all(codes[0] == 0) and np.all(codes[1, :32] == 0) and np.all(codes[1, 32:] == 8)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.zeros((1, 33)))
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.full((1, 32), np.inf))
