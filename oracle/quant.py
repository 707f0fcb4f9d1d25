"""BF16 -> MXFP4 weight quantiser, in float64 (oracle; test infrastructure only).

The gpt-oss page ("Conversion Methodology", step 2) describes the block
quantiser only for the NVFP4 target: per-block amax, a scale chosen from it,
elements rounded to E2M1 with that scale, packed codes and per-block scales.
MXFP4 takes the same steps with 32-element blocks and power-of-two E8M0 scales
(gpt-oss page, "GPT-OSS-120B Architecture" and the MXFP4/NVFP4 property
table).  The pages leave the MXFP4 scale rule open; the reading taken here is
the OCP Microscaling one, with one departure of this library's own:

  * shared exponent X = floor(log2(amax)) - 2, where 2 is the exponent of the
    largest E2M1 magnitude (6 = 1.5 * 2^2), so every |v| / 2^X is below 8;
  * X clamped to [-116, 125], i.e. scale bytes in [11, 252].  This clamp is
    the library's choice, not the OCP rule: the page's E8M0 range is
    2^-127 .. 2^127 and the OCP rule would give X down to -127 (bytes 0..10)
    to blocks with amax below 2^-114.  The library clamps so that every scale
    byte its quantisers write is one that all of its kernels apply exactly:
    its bf16 and FP8 contractions form each weight in bf16 with the
    hardware's scaled FP4 conversion, which is exact for bytes 11..252 only
    (measured on gfx950).  Only blocks with amax < 2^-114 are affected: for
    finite bf16 or fp32 input floor(log2(amax)) <= 127, so the upper clamp is
    never reached.  An all-zero block gets X = -116.  Pinned by a hand-worked
    block (tests/golden/mxfp4_small_block_case.txt);
  * element code = the E2M1 magnitude nearest to |v| / 2^X, ties to the code
    with an even mantissa bit, values above 6 saturating to 6; the sign bit
    is the input's sign (a negative value that rounds to zero gives -0).
"""

import numpy as np

from .mxfp4 import BLOCK, E2M1_TABLE, pack_nibbles

X_MIN = -116
X_MAX = 125


def block_exponent(amax):
    """Shared exponent of blocks with the given max |v| (float64, >= 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                 # amax = f * 2**e with f in [0.5, 1)
    x = np.where(amax > 0, e.astype(np.int64) - 1 - 2, X_MIN)
    return np.clip(x, X_MIN, X_MAX)


def e2m1_nearest(q):
    """Magnitude code (0..7) of the E2M1 value nearest to q >= 0.

    Distances to all eight magnitudes are compared; a tie goes to the code
    whose mantissa bit (bit 0) is 0.  Everything past 6 is nearest to 6.
    """
    q = np.asarray(q, dtype=np.float64)
    mags = E2M1_TABLE[:8]
    d = np.abs(q[..., None] - mags)                       # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                       # one or two codes
    even = cand & ((np.arange(8) & 1) == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    return np.argmax(pick, axis=-1).astype(np.uint8)


def quantize_mxfp4(w):
    """w [..., K] float64 (K % 32 == 0) -> (blocks uint8 [..., K/32, 16],
    scales uint8 [..., K/32]), in the steps of the conversion the gpt-oss
    page describes: per-block amax, block scale, E2M1 codes, packing."""
    w = np.asarray(w, dtype=np.float64)
    if w.shape[-1] % BLOCK:
        raise ValueError("K must be a multiple of 32")
    if not np.all(np.isfinite(w)):
        raise ValueError("the quantiser takes finite values")
    blocks = w.reshape(w.shape[:-1] + (w.shape[-1] // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)                    # [..., nb]
    x = block_exponent(amax)
    q = np.abs(blocks) / np.ldexp(1.0, x)[..., None]      # exact: power-of-two divide
    codes = e2m1_nearest(q) | (np.signbit(blocks).astype(np.uint8) << 3)
    scales = (x + 127).astype(np.uint8)
    return pack_nibbles(codes.reshape(w.shape)), scales
