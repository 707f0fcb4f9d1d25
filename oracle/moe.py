"""MoE layer and dense projection computed from their definitions (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain float64 numpy;
numpy's matmul is the only library primitive used for a contraction.

Sources:
  * gpt-oss page, "GPT-OSS-120B Architecture": 128 experts, 4 active per
    token, hidden size 2880; the MoE layer routes each token to 4 of 128.
  * gpt-oss page, "MXFP4 Tensor Structure": expert weights as *_blocks /
    *_scales / *_bias, bias kept in bfloat16.
  * spark-vllm page, "What's Included": the MoE layers are an FP8 x FP4
    grouped GEMM; qkv, o and lm_head are MXFP4 as well.
  * gptoss-spark page, "What produced it, ranked": qkv_proj, o_proj and the
    201k-row lm_head quantized to MXFP4.

Readings where the pages are silent (listed in the design doc):
  * routing: top-k by fp32 logit, descending, ties to the lower expert
    index (-0 == +0); weights = softmax over the k chosen logits;
  * the fused gate_up tensor holds the gate rows first ([0, I)) and the up
    rows second ([I, 2I)); activation h = silu(gate) * up with
    silu(z) = z / (1 + exp(-z)), no clamp;
  * biases are added inside each expert, before the routing weight;
  * FP8 mode quantizes x, and h, each with its own single per-tensor scale
    over the whole call (h rounded to fp32 first);
  * MXFP4-activation mode (the FP4 x FP4 block-scaled contraction the
    spark-vllm page lists as future work, "Performance Optimizations")
    quantizes each 32-element block of every row of x, and of every routed
    row of h (rounded to fp32 first), with the same block rule as the weight
    quantiser (oracle/quant.py);
  * out[t] = sum_k w[t,k] * y[t,k]; the oracle keeps it in float64.
"""

import numpy as np

from .fp8 import e4m3_decode, quant_per_tensor
from .mxfp4 import bf16_bits_to_f64, dequant
from .quant import quantize_mxfp4

ACT_BF16 = 0
ACT_FP8_E4M3 = 1
ACT_MXFP4 = 2


def route_topk(logits, k):
    """Top-k expert ids and softmax-of-k weights per token.

    logits: float32 [T, E].  Returns ids int32 [T, k] (descending logit,
    ties to the lower index) and weights float64 [T, k].
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    if l.ndim != 2 or not 1 <= k <= l.shape[1]:
        raise ValueError("logits must be [T, E] with 1 <= k <= E")
    if np.isnan(l).any():
        raise ValueError("NaN logits are not supported")
    order = np.argsort(-l, axis=1, kind="stable")       # stable: ties keep index order
    ids = order[:, :k].astype(np.int32)
    chosen = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return ids, w


def permute(ids, E):
    """Token-by-expert regrouping of the T*k (token, slot) pairs.

    Pair p = t*k + j.  Returns counts int64 [E], offsets int64 [E+1],
    sorted_pairs int64 [T*k] (pairs grouped by expert, ascending p inside an
    expert) and inv int64 [T*k] (position of pair p in sorted_pairs).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    sorted_pairs = np.argsort(flat, kind="stable")
    inv = np.empty_like(sorted_pairs)
    inv[sorted_pairs] = np.arange(flat.size)
    return counts, offsets, sorted_pairs, inv


def swiglu(g, I):
    """h = silu(gate) * up for g = [gate | up] along the last axis."""
    gate = g[..., :I]
    up = g[..., I:2 * I]
    with np.errstate(over="ignore"):
        silu = gate / (1.0 + np.exp(-gate))
    return silu * up


def _bias(bias_bits, shape):
    if bias_bits is None:
        return np.zeros(shape, dtype=np.float64)
    return bf16_bits_to_f64(bias_bits)


def moe_forward(x_bits, logits, w13_blocks, w13_scales, w13_bias,
                w2_blocks, w2_scales, w2_bias, k=4, act_mode=ACT_BF16):
    """One MoE layer from router logits: route_topk, then moe_forward_routed.

    x_bits   uint16 [T, H]   bfloat16 activations
    logits   float32 [T, E]  router logits
    w13_*    gate_up weights: blocks [E, 2I, H/32, 16], scales [E, 2I, H/32],
             bias bf16 bits [E, 2I] or None
    w2_*     down weights: blocks [E, H, I/32, 16], scales [E, H, I/32],
             bias bf16 bits [E, H] or None
    act_mode ACT_BF16 (activations used as given), ACT_FP8_E4M3
             (x and h each quantized with one per-tensor scale) or
             ACT_MXFP4 (x and h quantized to MXFP4, one E8M0 scale per
             32-element block of each row)
    """
    ids, w = route_topk(logits, k)
    res = moe_forward_routed(x_bits, ids, w, w13_blocks, w13_scales, w13_bias,
                             w2_blocks, w2_scales, w2_bias, act_mode)
    res.update(ids=ids, weights=w)
    return res


def moe_forward_routed(x_bits, ids, w, w13_blocks, w13_scales, w13_bias,
                       w2_blocks, w2_scales, w2_bias, act_mode=ACT_BF16, weight_format=None):
    """One MoE layer for given routing: ids int [T, k], weights [T, k].

    A pair whose id lies outside [0, E) contributes nothing to its token (the
    HIP boundary skips such pairs); in FP8 mode it also takes no part in the
    scale of h.  Returns a dict of float64 results and intermediates.

    weight_format None is MXFP4 (blocks [.., K/32, 16], E8M0 scales);
    ("nvfp4", g13, g2) is NVFP4 (blocks [.., K/16, 8], E4M3 scales, global
    scales g13 of w13 and g2 of w2; gpt-oss page, "The MXFP4 -> NVFP4
    Conversion").
    """
    x = bf16_bits_to_f64(x_bits)
    T, H = x.shape
    E = w13_blocks.shape[0]
    if weight_format is None:
        elems = 32
        dq13 = lambda e: dequant(w13_blocks[e], w13_scales[e])    # noqa: E731
        dq2 = lambda e: dequant(w2_blocks[e], w2_scales[e])       # noqa: E731
    elif weight_format[0] == "nvfp4":
        from .nvfp4 import dequant_nvfp4
        elems = 16
        g13, g2 = weight_format[1], weight_format[2]
        dq13 = lambda e: dequant_nvfp4(w13_blocks[e], w13_scales[e], g13)   # noqa: E731
        dq2 = lambda e: dequant_nvfp4(w2_blocks[e], w2_scales[e], g2)       # noqa: E731
    else:
        raise ValueError("unknown weight format")
    I = w2_blocks.shape[2] * elems
    if w13_blocks.shape[1] != 2 * I or w13_blocks.shape[2] * elems != H:
        raise ValueError("inconsistent weight shapes")
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    k = ids.shape[1]
    valid = (ids >= 0) & (ids < E)
    res = {}

    if act_mode == ACT_FP8_E4M3:
        xc, sx, _ = quant_per_tensor(x)
        a = e4m3_decode(xc) * sx
        res.update(x_codes=xc, x_scale=sx)
    elif act_mode == ACT_MXFP4:
        xb, xs = quantize_mxfp4(x)                           # per token row, 32-element blocks
        a = dequant(xb, xs)
        res.update(x_blocks=xb, x_scales=xs)
    elif act_mode == ACT_BF16:
        a = x
    else:
        raise ValueError("unknown act_mode")

    b1 = _bias(w13_bias, (E, 2 * I))
    b2 = _bias(w2_bias, (E, H))
    h = np.zeros((T, k, I))
    experts = np.unique(ids[valid])
    for e in experts:
        t, j = np.nonzero(ids == e)
        W1 = dq13(e)                                          # [2I, H]
        g = a[t] @ W1.T + b1[e]
        h[t, j] = swiglu(g, I)
    res["h"] = h

    if act_mode == ACT_FP8_E4M3:
        h32 = h.astype(np.float32).astype(np.float64)
        hc, sh, _ = quant_per_tensor(h32[valid])
        hq = np.zeros_like(h32)
        hq[valid] = e4m3_decode(hc) * sh
        res.update(h32=h32, h_codes=hc, h_scale=sh)
    elif act_mode == ACT_MXFP4:
        h32 = h.astype(np.float32).astype(np.float64)
        hb, hs = quantize_mxfp4(h32[valid])                  # [valid pairs, I/32, 16], [.., I/32]
        hq = np.zeros_like(h32)
        hq[valid] = dequant(hb, hs)
        res.update(h32=h32, h_blocks=hb, h_scales=hs)
    else:
        hq = h

    y = np.zeros((T, k, H))
    for e in experts:
        t, j = np.nonzero(ids == e)
        W2 = dq2(e)                                           # [H, I]
        y[t, j] = hq[t, j] @ W2.T + b2[e]
    res["y"] = y
    res["out"] = np.einsum("tk,tkh->th", np.where(valid, w, 0.0), y)
    return res


def linear(x_bits, w_blocks, w_scales, bias_bits=None):
    """Dense MXFP4 projection y = x W^T + b, float64.

    x_bits uint16 [M, K] bf16; w_blocks [N, K/32, 16]; w_scales [N, K/32];
    bias bf16 bits [N] or None.  Returns float64 [M, N].
    """
    x = bf16_bits_to_f64(x_bits)
    W = dequant(w_blocks, w_scales)
    if W.shape[1] != x.shape[1]:
        raise ValueError("K mismatch")
    return x @ W.T + _bias(bias_bits, (W.shape[0],))


def linear_act(x_bits, w_blocks, w_scales, bias_bits=None, act_mode=ACT_BF16):
    """Dense MXFP4 projection with the activation formats of the MoE layer,
    float64.  Returns a dict with out [M, N] and the activation codes.

    Reading (listed in the design doc): at prefill sizes the dense layers take the
    activations the MoE contraction takes -- the spark-vllm page runs the
    MoE layers as FP8 activations times FP4 weights ("What's Included") and
    asks for the dense layers on the same block-scaled MMA ("Performance
    Optimizations"); the FP4 x FP4 form is the one it lists as future work.
      ACT_BF16      out = x W^T + b (linear()).
      ACT_FP8_E4M3  x quantised with one scale over the whole of x
                    (quant_per_tensor): out = s (codes W^T) + b.
      ACT_MXFP4     each 32-element block of each row of x quantised with the
                    weight rule (quantize_mxfp4): out = dequant(xq) W^T + b.
    """
    x = bf16_bits_to_f64(x_bits)
    W = dequant(w_blocks, w_scales)
    if W.shape[1] != x.shape[1]:
        raise ValueError("K mismatch")
    b = _bias(bias_bits, (W.shape[0],))
    res = {}
    if act_mode == ACT_BF16:
        a = x
    elif act_mode == ACT_FP8_E4M3:
        xc, sx, _ = quant_per_tensor(x)
        a = e4m3_decode(xc) * sx
        res.update(x_codes=xc, x_scale=sx)
    elif act_mode == ACT_MXFP4:
        xb, xs = quantize_mxfp4(x)
        a = dequant(xb, xs)
        res.update(x_blocks=xb, x_scales=xs)
    else:
        raise ValueError("unknown act_mode")
    res["a"] = a
    res["out"] = a @ W.T + b
    return res


def linear_rows(x_bits, w_blocks, w_scales, bias_bits, rows):
    """linear() for a subset of output columns (rows of W), float64 [M, len(rows)]."""
    rows = np.asarray(rows)
    x = bf16_bits_to_f64(x_bits)
    W = dequant(w_blocks[rows], w_scales[rows])
    b = _bias(bias_bits, (w_blocks.shape[0],))[rows]
    return x @ W.T + b
