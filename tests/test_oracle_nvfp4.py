"""Pins of the oracle's NVFP4 weight decode (CPU only).

The gpt-oss page ("The MXFP4 -> NVFP4 Conversion") defines NVFP4 against
MXFP4: the same E2M1 element code, 16-element blocks, E4M3 block scales and
a global scale.  The pins tie the NVFP4 decode to the independently pinned
MXFP4 decode and to the page's property table.
"""

import numpy as np
import pytest

import oracle
from oracle import nvfp4


def _pow2_e4m3(e):
    """E4M3 code of 2**e for e in [-9, 8] (normal for e >= -6, else subnormal)."""
    if e >= -6:
        return (e + 7) << 3
    return 1 << (e + 9)          # subnormal: m * 2^-9 with m a power of two


def _mx_as_nv(blocks, scales):
    """MXFP4 (codes, E8M0 scales with exponents in [-9, 8]) as NVFP4 with the
    same values: each 32-element block becomes two 16-element blocks with the
    power-of-two scale written as an E4M3 code, global scale 1."""
    nb = blocks.shape[-2]
    nv_blocks = blocks.reshape(blocks.shape[:-2] + (2 * nb, 8))
    codes = np.vectorize(_pow2_e4m3)(scales.astype(np.int64) - 127).astype(np.uint8)
    nv_scales = np.repeat(codes, 2, axis=-1)
    return nv_blocks, nv_scales


def test_reduces_to_mxfp4_for_power_of_two_scales():
    rng = np.random.default_rng(0)
    blocks = rng.integers(0, 256, (5, 7, 9, 16)).astype(np.uint8)
    scales = rng.integers(127 - 9, 127 + 9, (5, 7, 9)).astype(np.uint8)
    nb, ns = _mx_as_nv(blocks, scales)
    assert np.array_equal(oracle.dequant_nvfp4(nb, ns, 1.0), oracle.dequant(blocks, scales))


def test_scale_grid_of_the_property_table():
    # E4M3 scales: 8 mantissa levels per binade, normal range from 2^-6, top
    # binade from 2^8 (gpt-oss page, MXFP4/NVFP4 property table)
    vals = oracle.e4m3_decode(np.arange(0, 0x7f, dtype=np.uint8))
    for e in range(1, 16):
        lv = vals[(e << 3):(e << 3) + 8] if e < 15 else vals[(e << 3):(e << 3) + 7]
        base = 2.0 ** (e - 7)
        assert np.allclose(np.diff(lv), base / 8) and lv[0] == base
    assert vals[1 << 3] == 2.0 ** -6 and vals[15 << 3] == 2.0 ** 8
    # the page's examples of fractional factors
    assert oracle.e4m3_decode(np.array([0x39, 0x3a, 0x3b], dtype=np.uint8)).tolist() == [1.125, 1.25, 1.375]


def test_element_scale_and_global_placement():
    # one row, two blocks: code c at element i of block b, scale codes s0, s1
    blocks = np.zeros((1, 2, 8), dtype=np.uint8)
    blocks[0, 0, 3] = 0x1 | (0x7 << 4)      # elements 6 (0.5) and 7 (6.0)
    blocks[0, 1, 0] = 0xB                    # element 16: -1.5
    scales = np.array([[0x39, 0x30]], dtype=np.uint8)   # 1.125, 0.5
    w = oracle.dequant_nvfp4(blocks, scales, 0.25)
    want = np.zeros((1, 32))
    want[0, 6] = 0.5 * 1.125 * 0.25
    want[0, 7] = 6.0 * 1.125 * 0.25
    want[0, 16] = -1.5 * 0.5 * 0.25
    assert np.array_equal(w, want)


@pytest.mark.parametrize("act_mode", [oracle.ACT_BF16, oracle.ACT_FP8_E4M3])
def test_moe_forward_with_nvfp4_equals_mxfp4_for_the_same_values(act_mode):
    rng = np.random.default_rng(3)
    E, H, I, T, k = 4, 64, 96, 7, 2
    w13 = rng.integers(0, 256, (E, 2 * I, H // 32, 16)).astype(np.uint8)
    s13 = rng.integers(124, 131, (E, 2 * I, H // 32)).astype(np.uint8)
    w2 = rng.integers(0, 256, (E, H, I // 32, 16)).astype(np.uint8)
    s2 = rng.integers(124, 131, (E, H, I // 32)).astype(np.uint8)
    b13 = (rng.standard_normal((E, 2 * I)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b2 = (rng.standard_normal((E, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    wts = rng.random((T, k))
    ref = oracle.moe_forward_routed(x, ids, wts, w13, s13, b13, w2, s2, b2, act_mode=act_mode)
    n13, m13 = _mx_as_nv(w13, s13)
    n2, m2 = _mx_as_nv(w2, s2)
    got = oracle.moe_forward_routed(x, ids, wts, n13, m13, b13, n2, m2, b2, act_mode=act_mode,
                                    weight_format=("nvfp4", 1.0, 1.0))
    assert np.array_equal(got["out"], ref["out"])
    # a power-of-two global scale of w2 scales y minus its bias exactly
    got2 = oracle.moe_forward_routed(x, ids, wts, n13, m13, b13, n2, m2, b2, act_mode=act_mode,
                                     weight_format=("nvfp4", 1.0, 4.0))
    bias = oracle.bf16_bits_to_f64(b2)[ids]
    assert np.array_equal(got2["y"] - bias, 4.0 * (ref["y"] - bias))
    # a power-of-two global scale of w13 is the MXFP4 layer with every w13
    # scale byte raised by its exponent (the weights are the same values)
    got3 = oracle.moe_forward_routed(x, ids, wts, n13, m13, b13, n2, m2, b2, act_mode=act_mode,
                                     weight_format=("nvfp4", 8.0, 1.0))
    ref3 = oracle.moe_forward_routed(x, ids, wts, w13, s13 + 3, b13, w2, s2, b2, act_mode=act_mode)
    assert np.array_equal(got3["out"], ref3["out"])
    assert not np.array_equal(got3["out"], ref["out"])
