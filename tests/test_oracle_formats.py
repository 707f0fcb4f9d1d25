"""Pins for the oracle's MXFP4 decoding (E2M1, nibble order, E8M0, dequant)."""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_numbers(name):
    vals = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.append(line)
    return vals


def _read_kv(name):
    return {k: float(v) for k, v in (l.split() for l in _read_numbers(name))}


def test_e2m1_table_is_the_printed_value_set():
    printed = sorted(float(v) for v in _read_numbers("e2m1_values.txt"))
    mags = sorted(set(abs(v) for v in oracle.E2M1_TABLE))
    assert mags == printed
    # codes 0..7 positive and increasing, 8..15 their negatives
    pos = oracle.E2M1_TABLE[:8]
    assert list(pos) == printed
    for c in range(16):
        assert oracle.E2M1_TABLE[c ^ 8] == -oracle.E2M1_TABLE[c]
        assert math.copysign(1.0, oracle.E2M1_TABLE[c]) == (-1.0 if c & 8 else 1.0)


def test_e2m1_closed_form_fields():
    # exponent field 0 is subnormal, others 2^(e-1) * (1 + m/2)
    assert oracle.e2m1_value(0b0001) == 0.5
    assert oracle.e2m1_value(0b0010) == 1.0
    assert oracle.e2m1_value(0b0111) == 6.0
    assert oracle.e2m1_value(0b1101) == -3.0
    with pytest.raises(ValueError):
        oracle.e2m1_value(16)


def test_unpack_low_nibble_first():
    blk = np.zeros((1, 16), dtype=np.uint8)
    blk[0, 0] = 0x21          # element 0 <- 1, element 1 <- 2
    blk[0, 15] = 0xF7         # element 30 <- 7, element 31 <- 15
    codes = oracle.unpack_nibbles(blk)
    assert codes.shape == (32,)
    assert codes[0] == 1 and codes[1] == 2
    assert codes[30] == 7 and codes[31] == 15
    assert not codes[2:30].any()


def test_pack_unpack_round_trip_all_bytes():
    allb = np.arange(256, dtype=np.uint8).reshape(16, 16)   # 16 blocks
    codes = oracle.unpack_nibbles(allb)
    assert codes.shape == (16 * 32,)
    assert np.array_equal(oracle.pack_nibbles(codes), allb)
    rng = np.random.default_rng(5)
    c = rng.integers(0, 16, size=(3, 7, 96), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_nibbles(oracle.pack_nibbles(c)), c)


def test_e8m0_closed_form_and_range():
    fmt = _read_kv("mxfp4_format.txt")
    bias = int(fmt["e8m0_bias"])
    s = np.arange(255)
    sc = oracle.e8m0_scale(s)
    for b in range(255):
        assert sc[b] == math.ldexp(1.0, b - bias)
    assert oracle.e8m0_scale(127) == 1.0
    assert math.log2(sc.min()) == fmt["scale_log2_min"]
    assert math.log2(sc.max()) == fmt["scale_log2_max"]
    assert np.isnan(oracle.e8m0_scale(255))


def test_dequant_hand_built_blocks():
    fmt = _read_kv("mxfp4_format.txt")
    assert int(fmt["block_elements"]) == mxfp4.BLOCK
    assert int(fmt["block_bytes"]) == mxfp4.BLOCK_BYTES
    # row 0: two blocks, all codes 7 (6.0) with scale 2^2, then all 0x9 (-0.5) with 2^-3
    blocks = np.zeros((2, 2, 16), dtype=np.uint8)
    blocks[0, 0, :] = 0x77
    blocks[0, 1, :] = 0x99
    blocks[1, 0, :] = 0x1A      # even elements code 0xA (-1.0), odd code 1 (0.5)
    blocks[1, 1, :] = 0x00
    scales = np.array([[129, 124], [127, 200]], dtype=np.uint8)
    W = oracle.dequant(blocks, scales)
    assert W.shape == (2, 64)
    assert np.all(W[0, :32] == 24.0)
    assert np.all(W[0, 32:] == -0.5 / 8)
    assert np.all(W[1, 0:32:2] == -1.0) and np.all(W[1, 1:32:2] == 0.5)
    assert np.all(W[1, 32:] == 0.0)


def test_dequant_brute_force_random():
    rng = np.random.default_rng(11)
    blocks = rng.integers(0, 256, size=(5, 3, 16), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(5, 3), dtype=np.uint8)
    W = oracle.dequant(blocks, scales)
    for n in range(5):
        for k in range(96):
            byte = int(blocks[n, k // 32, (k % 32) // 2])
            code = (byte >> 4) if k % 2 else (byte & 15)
            sign = -1.0 if code & 8 else 1.0
            e, m = (code >> 1) & 3, code & 1
            mag = m / 2 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
            assert W[n, k] == sign * mag * 2.0 ** (int(scales[n, k // 32]) - 127)


def test_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3F81], dtype=np.uint16)
    v = oracle.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0
    assert math.copysign(1.0, v[3]) == -1.0 and v[4] == math.inf
    assert v[5] == 1.0 + 2.0 ** -7


def test_gpt_oss_dense_shapes_match_the_page():
    import synth
    g = _read_kv("gpt_oss_shapes.txt")
    assert synth.H_GPT_OSS == g["hidden"]
    assert synth.E_GPT_OSS == g["experts"] and synth.TOPK_GPT_OSS == g["active_experts"]
    assert synth.QKV_N == (g["attention_heads"] + 2 * g["kv_heads"]) * g["head_dim"] == g["qkv_rows"]
    assert synth.O_K == g["attention_heads"] * g["head_dim"] == g["o_in"]
    assert synth.VOCAB_GPT_OSS == g["vocab"]
