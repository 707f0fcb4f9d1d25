"""MXFP4 weight format, decoded in float64 (oracle; test infrastructure only).

Source: gpt-oss page, sections "GPT-OSS-120B Architecture" (published format:
E2M1 data, E8M0 scales, block size 32) and "MXFP4 Tensor Structure" (tensor
names, shapes, the E2M1 value set and the E8M0 bias), plus the MXFP4/NVFP4
property table (scale range) and "Conversion Methodology" step 1 (unpack,
look up, multiply by two to the stored exponent minus 127).
"""

import numpy as np

BLOCK = 32          # elements per MX block (gpt-oss page, format row: block_size=32)
BLOCK_BYTES = 16    # two E2M1 nibbles per byte (gpt-oss page, *_blocks bullet)
E8M0_BIAS = 127     # gpt-oss page, "MXFP4 Tensor Structure"


def e2m1_value(code):
    """Value of one 4-bit E2M1 code, from its bit fields.

    Reading (the page gives only the name "E2M1" and the value set): bit 3 is
    the sign, bits 2..1 a 2-bit exponent with bias 1, bit 0 a 1-bit mantissa;
    exponent field 0 is subnormal (0.5 * mantissa).  This is the only field
    layout that reproduces the printed set {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    """
    code = int(code)
    if not 0 <= code <= 15:
        raise ValueError("E2M1 code out of range")
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


# 16-entry decode table built from the closed form above (float64).
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def unpack_nibbles(blocks):
    """uint8 [..., nb, 16] -> E2M1 codes uint8 [..., nb*32].

    Reading (the page says only "2 per byte"): byte i of a block holds
    element 2i in its low nibble and element 2i+1 in its high nibble.
    """
    b = np.asarray(blocks, dtype=np.uint8)
    if b.shape[-1] != BLOCK_BYTES:
        raise ValueError("last axis of *_blocks must be 16 bytes")
    lo = b & 0x0F
    hi = b >> 4
    codes = np.stack([lo, hi], axis=-1)            # [..., nb, 16, 2]
    return codes.reshape(b.shape[:-2] + (b.shape[-2] * BLOCK,))


def pack_nibbles(codes):
    """Inverse of unpack_nibbles: codes [..., K] (K % 32 == 0) -> [..., K/32, 16]."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % BLOCK:
        raise ValueError("K must be a multiple of 32")
    if np.any(c > 15):
        raise ValueError("E2M1 codes are 4-bit")
    pairs = c.reshape(c.shape[:-1] + (c.shape[-1] // 2, 2))
    packed = (pairs[..., 0] | (pairs[..., 1] << 4)).astype(np.uint8)
    return packed.reshape(c.shape[:-1] + (c.shape[-1] // BLOCK, BLOCK_BYTES))


def e8m0_scale(s):
    """E8M0 byte -> float64 scale 2**(s - 127).

    gpt-oss page: power-of-two exponent with bias 127; its property table
    gives the range 2^-127 .. 2^127, so byte 255 lies outside it.  Reading:
    255 is not a number (NaN), as in the OCP MX convention.
    """
    s = np.asarray(s)
    out = np.ldexp(1.0, s.astype(np.int64) - E8M0_BIAS)
    return np.where(s == 255, np.nan, out)


def dequant(blocks, scales):
    """W[..., n, k] = E2M1(code[n, k]) * 2**(scales[n, k // 32] - 127), float64.

    gpt-oss page, "Conversion Methodology" step 1.  Every product is exact in
    float64.
    """
    blocks = np.asarray(blocks, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != blocks.shape[:-1]:
        raise ValueError("scales must be blocks.shape[:-1]")
    vals = E2M1_TABLE[unpack_nibbles(blocks)]                 # [..., n, K]
    sc = np.repeat(e8m0_scale(scales), BLOCK, axis=-1)       # [..., n, K]
    return vals * sc


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
