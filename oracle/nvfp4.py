"""NVFP4 weight format, decoded in float64 (oracle; test infrastructure only).

Source: gpt-oss page, "The MXFP4 -> NVFP4 Conversion": the same E2M1 element
code as MXFP4, 16-element blocks instead of 32, one E4M3 scale per block
(exponent and mantissa, so fractional factors such as 1.125 are possible),
and one global scale factor per quantised tensor ("Conversion Methodology",
step 2, and the *_weights / *_weights_scaling_factor /
*_weights_scaling_factor_2 tensors of step 3).

Readings where the pages are silent (listed in the design doc):
  * packing as in MXFP4 (two codes per byte, element 2i in the low nibble of
    byte i of a block): a block is 8 bytes;
  * the block scale is an OCP E4M3 code (the same codec as the FP8
    activations); the stored scaling factor is this code's value;
  * the global scale is one fp32 number per weight tensor (w13 and w2 of
    the MoE layer each have one), and a weight is
    E2M1(code) * E4M3(block scale) * global.
"""

import numpy as np

from .fp8 import e4m3_decode
from .mxfp4 import E2M1_TABLE

BLOCK = 16          # elements per NVFP4 block
BLOCK_BYTES = 8     # two E2M1 codes per byte


def unpack_nibbles16(blocks):
    """uint8 [..., nb, 8] -> E2M1 codes uint8 [..., nb*16] (low nibble first)."""
    b = np.asarray(blocks, dtype=np.uint8)
    if b.shape[-1] != BLOCK_BYTES:
        raise ValueError("last axis of NVFP4 blocks must be 8 bytes")
    codes = np.stack([b & 0x0F, b >> 4], axis=-1)           # [..., nb, 8, 2]
    return codes.reshape(b.shape[:-2] + (b.shape[-2] * BLOCK,))


def dequant_nvfp4(blocks, scales, global_scale):
    """W[..., n, k] = E2M1(code) * E4M3(scales[n, k // 16]) * global, float64."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != blocks.shape[:-1]:
        raise ValueError("scales must be blocks.shape[:-1]")
    vals = E2M1_TABLE[unpack_nibbles16(blocks)]
    sc = np.repeat(e4m3_decode(scales), BLOCK, axis=-1)
    return vals * sc * float(global_scale)
