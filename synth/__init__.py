"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds none of the layer's arithmetic: it only draws random
numbers with numpy's PCG64 generator (``numpy.random.default_rng``) and
packs them into the storage types the layer takes (uint8 blocks/scales,
bfloat16 bit patterns, float32 logits).  The distributions follow the
workload definitions; shapes follow the gpt-oss page ("GPT-OSS-120B
Architecture": hidden 2880, 128 experts, top-4, 64 query heads and 8 KV
heads of dimension 64, vocabulary 201,088; "MXFP4 Tensor Structure":
*_blocks [E, N, K/32, 16], *_scales [E, N, K/32], bf16 *_bias).

Recipe:
  layer(seed=1000): draws, in this order, w13_blocks (uniform bytes, i.e. two
    independent uniform E2M1 nibbles), w13_scales (integers uniform on
    [120, 130]), w13_bias (N(0, 0.02) -> float32 -> bfloat16 RNE), then the
    same three for w2.
  moe_inputs(seed, T): logits float32 N(0, 1) [T, E], then
    x = bfloat16(N(0, 1)) [T, H]; the skewed workload adds +2.0 to the logits
    of experts 0..7.
  dense(seed, N, K) and dense_x(seed, M, K): the same weight and activation
    distributions for one projection.
"""

import numpy as np

H_GPT_OSS = 2880
E_GPT_OSS = 128
TOPK_GPT_OSS = 4
VOCAB_GPT_OSS = 201088
QKV_N = (64 + 2 * 8) * 64      # 64 query heads + 8 K + 8 V heads, head dim 64
O_K = 64 * 64

LAYER_SEED = 1000
DENSE_SEEDS = {"qkv_proj": 30, "o_proj": 31, "lm_head": 32}
DENSE_X_SEED = 3
DENSE_SHAPES = {                  # name -> (N, K)
    "qkv_proj": (QKV_N, H_GPT_OSS),
    "o_proj": (H_GPT_OSS, O_K),
    "lm_head": (VOCAB_GPT_OSS, H_GPT_OSS),
}

# MoE workloads: name -> (seed, tokens, act_mode, hot experts)
ACT_BF16 = 0
ACT_FP8_E4M3 = 1
ACT_MXFP4 = 2
MOE_WORKLOADS = {
    "moe_decode_t4": (0, 4, ACT_BF16, 0),
    "moe_decode_t32": (1, 32, ACT_BF16, 0),
    "moe_prefill_t2048_fp8": (2, 2048, ACT_FP8_E4M3, 0),
    "moe_prefill_t8192_fp8_skewed": (4, 8192, ACT_FP8_E4M3, 8),
    # the same token batches with MXFP4 activations (FP4 x FP4)
    "moe_prefill_t2048_fp4": (2, 2048, ACT_MXFP4, 0),
    "moe_prefill_t8192_fp4_skewed": (4, 8192, ACT_MXFP4, 8),
}
HOT_BOOST = 2.0


def f32_to_bf16_bits(a):
    """float32 array -> bfloat16 bit patterns (round to nearest even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns -> float32 (exact widening), for printing/plots."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def _weights(rng, lead, N, K):
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = rng.integers(0, 256, size=lead + (N, K // 32, 16), dtype=np.uint8)
    scales = rng.integers(120, 131, size=lead + (N, K // 32), dtype=np.uint8)
    bias = f32_to_bf16_bits(rng.normal(0.0, 0.02, size=lead + (N,)).astype(np.float32))
    return blocks, scales, bias


def layer(seed=LAYER_SEED, E=E_GPT_OSS, H=H_GPT_OSS, I=H_GPT_OSS):
    """One MoE layer's MXFP4 weights (dict of numpy arrays)."""
    rng = np.random.default_rng(seed)
    w13_blocks, w13_scales, w13_bias = _weights(rng, (E,), 2 * I, H)
    w2_blocks, w2_scales, w2_bias = _weights(rng, (E,), H, I)
    return dict(w13_blocks=w13_blocks, w13_scales=w13_scales, w13_bias=w13_bias,
                w2_blocks=w2_blocks, w2_scales=w2_scales, w2_bias=w2_bias)


NVFP4_LAYER_SEED = 2000


def _nv_weights(rng, lead, N, K):
    """NVFP4 blocks (uniform bytes: two uniform E2M1 codes), E4M3 block scales
    (positive, exponent field 4..10 with any mantissa: 0.125 .. 15.0) and a
    bf16 bias, for [lead.., N, K] weights."""
    blocks = rng.integers(0, 256, lead + (N, K // 16, 8), dtype=np.uint8)
    exp = rng.integers(4, 11, lead + (N, K // 16))
    man = rng.integers(0, 8, lead + (N, K // 16))
    scales = ((exp << 3) | man).astype(np.uint8)
    bias = f32_to_bf16_bits(rng.normal(0.0, 0.02, lead + (N,)).astype(np.float32))
    return blocks, scales, bias


def nvfp4_layer(seed=NVFP4_LAYER_SEED, E=E_GPT_OSS, H=H_GPT_OSS, I=H_GPT_OSS):
    """One MoE layer's NVFP4 weights (dict of numpy arrays and the two fp32
    global scales, 2^-6 and 3 * 2^-8)."""
    rng = np.random.default_rng(seed)
    w13_blocks, w13_scales, w13_bias = _nv_weights(rng, (E,), 2 * I, H)
    w2_blocks, w2_scales, w2_bias = _nv_weights(rng, (E,), H, I)
    return dict(w13_blocks=w13_blocks, w13_scales=w13_scales, w13_global=2.0 ** -6, w13_bias=w13_bias,
                w2_blocks=w2_blocks, w2_scales=w2_scales, w2_global=3.0 * 2.0 ** -8, w2_bias=w2_bias)


def moe_inputs(seed, T, E=E_GPT_OSS, H=H_GPT_OSS, hot=0):
    """Router logits float32 [T, E] and x bf16 bits [T, H]."""
    rng = np.random.default_rng(seed)
    logits = rng.normal(0.0, 1.0, size=(T, E)).astype(np.float32)
    if hot:
        logits[:, :hot] += np.float32(HOT_BOOST)
    x = f32_to_bf16_bits(rng.normal(0.0, 1.0, size=(T, H)).astype(np.float32))
    return logits, x


def workload(name, E=E_GPT_OSS, H=H_GPT_OSS):
    seed, T, act, hot = MOE_WORKLOADS[name]
    logits, x = moe_inputs(seed, T, E=E, H=H, hot=hot)
    return dict(logits=logits, x=x, T=T, act_mode=act, seed=seed)


def dense(seed, N, K):
    """One dense projection: blocks [N, K/32, 16], scales [N, K/32], bias bf16 [N]."""
    rng = np.random.default_rng(seed)
    blocks, scales, bias = _weights(rng, (), N, K)
    return dict(w_blocks=blocks, w_scales=scales, bias=bias)


def dense_bf16_weights(seed, N, K):
    """bf16 bits [N, K] of a dense weight before MXFP4 quantisation: N(0, 0.02)
    with row scales spread over 2^-4 .. 2^4 and about one outlier (x 50) per
    1024 elements, the shape a trained projection's weights take.  Generated
    in row chunks (float32) so the 201k-row lm_head fits in a few GB."""
    rng = np.random.default_rng(seed)
    out = np.empty((N, K), dtype=np.uint16)
    for r0 in range(0, N, 8192):
        r1 = min(N, r0 + 8192)
        scale = np.ldexp(np.float32(0.02), rng.integers(-4, 5, size=(r1 - r0, 1))).astype(np.float32)
        w = rng.standard_normal(size=(r1 - r0, K), dtype=np.float32) * scale
        spike = rng.random(size=(r1 - r0, K), dtype=np.float32) < np.float32(1.0 / 1024)
        w = np.where(spike, w * np.float32(50.0), w)
        out[r0:r1] = f32_to_bf16_bits(w)
    return out


def dense_x(seed, M, K):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32))
