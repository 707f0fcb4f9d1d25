"""Parity tools for the quantised MoE modes (test infrastructure; CPU only).

In the FP8 and MXFP4-activation modes the kernel quantises h, the SwiGLU
output, which it computes in fp32.  An h code is then only unique where no h
within the fp32 error of the computation rounds to another code.  These
helpers

  * bound that error per element from the arithmetic (``h_tolerance``),
  * check every code the kernel wrote against the oracle's code of the
    oracle's h: equal, or else a rounding that an h within the bound takes
    (``fp8_code_mismatch``, ``mx_code_mismatch``), and
  * turn the codes that do differ into a per-output allowance
    (``mismatch_slack``): |w| |W2| |change of the dequantised h|, summed over
    the token's pairs.

Everything here calls only the oracle.
"""

import numpy as np

import oracle
from oracle.quant import block_exponent, e2m1_nearest

U = 2.0 ** -24        # unit roundoff of fp32 (round to nearest)


def gate_up_terms(a, W1, b1, step=32):
    """g = a W1^T + b1 (float64) for activation rows a [m, H] as the
    contraction sees them and W1 [2I, H] dequantised, and R = the sum of |p_j|
    over the partial sums p_j = a[:, :step*j] W1[:, :step*j]^T at every
    step-element boundary j = 1 .. ceil(H/step) (the last one the whole dot
    product), plus |g| and |b1| for the scale and bias roundings: each
    accumulation step rounds once, by at most u/2 of its partial sum."""
    m, H = a.shape
    acc = np.zeros((m, W1.shape[0]))
    R = np.zeros_like(acc)
    for k0 in range(0, H, step):
        acc += a[:, k0:k0 + step] @ W1[:, k0:k0 + step].T
        R += np.abs(acc)
    g = acc + b1
    return g, R + np.abs(g) + np.abs(b1)


def h_tolerance(g, R, I):
    """Bound on |h_kernel - h| per element, h = silu(gate) * up.

    * The gate and up sums: the kernel adds each MFMA step's products (32
      per step in the bf16 form, 128 in the FP4 form: the 32-element
      boundaries include all of them) into an fp32 accumulator, one rounding
      of at most u/2 of the partial sum per step, plus one for the
      activation scale and one for the bias: u R (from gate_up_terms) bounds
      them with a factor two to spare for the MFMA's own adds.
    * SiLU uses the hardware 2^x and reciprocal: exp(-z) is 2^(-z log2 e),
      whose rounded argument gives it a relative error of about
      |z| log2(e) u/2, which reaches silu scaled by e^-z / (1 + e^-z); an ulp
      or two more for each instruction: (1.5 |z| (1 - sigmoid z) + 4) u
      relative.
    * h is rounded to fp32 once: u relative.
    * Below the normal fp32 range the kernel's SiLU loses its value: for z
      below about -87.3 the hardware reciprocal of 1 + e^-z falls under
      2^-126 and is flushed to zero, so there the whole |h| (at most about
      2^-118 |up|) may go; elsewhere h rounds to a multiple of 2^-149 at
      worst: |h| where z < -87, plus 2^-126 |up| + 2^-149 absolute.
    Propagated through h = silu(gate) * up to first order."""
    gate, up = g[..., :I], g[..., I:2 * I]
    tg, tu = U * R[..., :I], U * R[..., I:2 * I]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-gate))
    silu = gate * sig
    dsilu = sig * (1.0 + gate * (1.0 - sig))
    h = silu * up
    tol = np.abs(dsilu) * tg * np.abs(up) + np.abs(silu) * tu
    tol += ((1.5 * np.abs(gate) * (1.0 - sig) + 4.0) * U + U) * np.abs(h)
    tol += np.where(gate < -87.0, np.abs(h), 0.0) + 2.0 ** -126 * np.abs(up) + 2.0 ** -149
    return tol


def activations(res, x_bits, act_mode):
    """The activation rows the gate_up contraction sees, float64 [T, H]."""
    if act_mode == oracle.ACT_FP8_E4M3:
        return oracle.e4m3_decode(res["x_codes"]) * res["x_scale"]
    if act_mode == oracle.ACT_MXFP4:
        return oracle.dequant(res["x_blocks"], res["x_scales"])
    return oracle.bf16_bits_to_f64(x_bits)


def pair_h_tolerance(a, ids, layer, pairs, k):
    """h_tolerance for the listed pairs (p = t*k + j), float64 [len(pairs), I]."""
    I = layer["w2_blocks"].shape[2] * 32
    tol = np.zeros((len(pairs), I))
    exps = ids.reshape(-1)[pairs]
    for e in np.unique(exps):
        sel = np.nonzero(exps == e)[0]
        W1 = oracle.dequant(layer["w13_blocks"][e], layer["w13_scales"][e])
        b1 = (np.zeros(2 * I) if layer["w13_bias"] is None
              else oracle.bf16_bits_to_f64(layer["w13_bias"][e]))
        g, R = gate_up_terms(a[pairs[sel] // k], W1, b1)
        tol[sel] = h_tolerance(g, R, I)
    return tol


def fp32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def fp8_code_mismatch(codes_gpu, s_gpu, h_ref, tol, s_ref):
    """E4M3 codes the kernel wrote (scale s_gpu) against the oracle's codes of
    its h (h_ref, already fp32, scale s_ref).  Every differing code must be
    one that some h' in [h_ref - tol, h_ref + tol] takes under s_gpu (the
    codec is monotone, so the codes of the two ends bound it).  Returns the
    change |s_gpu decode(c_gpu) - s_ref decode(c_ref)| of the dequantised h at
    differing codes (0 elsewhere) and the number of differing codes."""
    c_ref = oracle.e4m3_encode(fp32(h_ref / s_ref))
    diff = codes_gpu != c_ref
    v_gpu = oracle.e4m3_decode(codes_gpu)
    lo = oracle.e4m3_decode(oracle.e4m3_encode(fp32((h_ref - tol) / s_gpu)))
    hi = oracle.e4m3_decode(oracle.e4m3_encode(fp32((h_ref + tol) / s_gpu)))
    bad = diff & ~((v_gpu >= lo) & (v_gpu <= hi))
    assert not bad.any(), "%d FP8 h codes differ beyond the h error bound" % bad.sum()
    delta = np.where(diff, np.abs(v_gpu * s_gpu - oracle.e4m3_decode(c_ref) * s_ref), 0.0)
    return delta, int(diff.sum())


def _mx_values(v, X):
    """v [..., nb, 32] rounded to E2M1 under shared exponents X [..., nb]."""
    sc = np.ldexp(1.0, X)[..., None]
    mag = oracle.E2M1_TABLE[e2m1_nearest(np.abs(v) / sc)] * sc
    return np.where(v < 0, -mag, mag)


def mx_code_mismatch(blocks_gpu, scales_gpu, h_ref, tol):
    """MXFP4 codes of h the kernel wrote (blocks [m, I/32, 16], scale bytes
    [m, I/32]) against the oracle quantiser of h_ref [m, I] (fp32 values).
    A differing block exponent must be the exponent of some amax within the
    bound of the block's amax; a differing element value must be the rounding,
    under the kernel's exponent, of some h' in [h_ref - tol, h_ref + tol].
    Returns |dequant(kernel) - dequant(oracle)| [m, I] and the number of
    differing elements."""
    m, I = h_ref.shape
    rb, rs = oracle.quantize_mxfp4(h_ref)
    got = oracle.dequant(blocks_gpu, scales_gpu)
    ref = oracle.dequant(rb, rs)
    hb = h_ref.reshape(m, I // 32, 32)
    tb = tol.reshape(m, I // 32, 32)
    x_gpu = scales_gpu.astype(np.int64) - 127
    amax_lo = np.max(np.maximum(np.abs(hb) - tb, 0.0), axis=-1)
    amax_hi = np.max(np.abs(hb) + tb, axis=-1)
    x_ok = (x_gpu >= block_exponent(amax_lo)) & (x_gpu <= block_exponent(amax_hi))
    assert x_ok.all(), "%d MXFP4 h block scales differ beyond the h error bound" % (~x_ok).sum()
    lo = _mx_values(hb - tb, x_gpu).reshape(m, I)
    hi = _mx_values(hb + tb, x_gpu).reshape(m, I)
    diff = got != ref
    bad = diff & ~((got >= lo) & (got <= hi))
    assert not bad.any(), "%d MXFP4 h values differ beyond the h error bound" % bad.sum()
    return np.where(diff, np.abs(got - ref), 0.0), int(diff.sum())


def mismatch_slack(delta, pair_tok, pair_exp, pair_w, tokens, w2_of):
    """Per-output allowance of the differing h codes: for each token in
    `tokens`, sum over its pairs of |w| |W2[e]| @ delta.  delta [m, I] holds
    the dequantised-h change per pair, pair_tok / pair_exp / pair_w [m] the
    pair's token, expert and routing weight; w2_of(e) the dequantised W2.
    None when no code differs."""
    pos = {int(t): i for i, t in enumerate(tokens)}
    hit = np.nonzero(delta.any(axis=1))[0]
    slack = None
    for e in np.unique(pair_exp[hit]):
        W2a = np.abs(w2_of(int(e)))
        if slack is None:
            slack = np.zeros((len(tokens), W2a.shape[0]))
        for p in hit[pair_exp[hit] == e]:
            nz = np.nonzero(delta[p])[0]
            slack[pos[int(pair_tok[p])]] += abs(pair_w[p]) * (W2a[:, nz] @ delta[p, nz])
    return slack


def down_combine(hq, pair_tok, pair_exp, pair_w, tokens, w2_of, b2_of):
    """out[t] = sum over the token's pairs of w (W2[e] hq + b2[e]), float64,
    for the tokens listed (rows of hq are pairs)."""
    pos = {int(t): i for i, t in enumerate(tokens)}
    out = None
    for e in np.unique(pair_exp):
        sel = np.nonzero(pair_exp == e)[0]
        W2 = w2_of(int(e))
        y = hq[sel] @ W2.T + b2_of(int(e))
        if out is None:
            out = np.zeros((len(tokens), W2.shape[0]))
        for i, p in enumerate(sel):
            out[pos[int(pair_tok[p])]] += pair_w[p] * y[i]
    return out
