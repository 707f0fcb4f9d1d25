"""Writes the oracle's results for the full-size MoE workloads to tests/golden/.

Calls only ``oracle`` (float64 CPU reference) and ``synth`` (seeded inputs).
For each workload it stores, in <name>.npz:
  tokens    int64 [n]      tokens whose outputs are kept (all if T <= 32, else
                           a seeded sample including the first and last token)
  out       float32 [n, H] oracle output rows of those tokens
FP8 and MXFP4-activation workloads also store
  x_scale, h_scale, h_amax the per-tensor quantisation values
  h_pairs   int64 [m]      a seeded sample of pair indices p = t*k + j
  h_ref     float32 [m, I] the oracle's h (before quantisation) of those pairs
  slack     float32 [n, H] per-output bound on how far the output may move if
                           h codes whose value lies within the stated h error
                           (H_REL_ERR relative + H_ABS_ERR code units) of a
                           rounding boundary are taken as the neighbouring
                           code (MXFP4: also a block whose amax lies that close
                           to a power of two taking the neighbouring shared
                           exponent); both are correct roundings of an h
                           within that error, so the output is not unique there.
FP8 workloads store x_scale, h_scale and h_amax besides.
Run: python tests/golden/make_golden.py [workload ...]
"""

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SAMPLE = 24
H_PAIRS = 16
# Error allowed between a kernel's fp32 h and the float64 h: fp32 accumulation
# over K = 2880 leaves ~1e-6 relative; these bounds carry a wide margin and are
# asserted against the kernel's h on the sampled pairs.
H_REL_ERR = 2e-5
H_ABS_ERR = 1e-4      # in units of the h scale (FP8: the per-tensor scale; MXFP4: the block scale)


def golden_path(name):
    return os.path.join(HERE, "%s.npz" % name)


def code_gap(h32, s):
    """|decoded neighbour code - decoded code| * s for every h element whose
    quotient lies within the stated error of a rounding boundary, else 0."""
    q = (h32 / s).astype(np.float32).astype(np.float64)
    width = H_REL_ERR * 2.1 * np.abs(q) + H_ABS_ERR
    c = oracle.e4m3_decode(oracle.e4m3_encode(q))
    lo = oracle.e4m3_decode(oracle.e4m3_encode(q - width))
    hi = oracle.e4m3_decode(oracle.e4m3_encode(q + width))
    return np.maximum(np.abs(lo - c), np.abs(hi - c)) * s


def _mx_dequant(v, X):
    """Values v [..., nb, 32] rounded to E2M1 with shared exponents X [..., nb]."""
    sc = np.ldexp(1.0, X)[..., None]
    mag = oracle.E2M1_TABLE[oracle.quant.e2m1_nearest(np.abs(v) / sc)] * sc
    return np.where(v < 0, -mag, mag)


def mx_code_gap(h32):
    """Per element of h32 [..., I] (fp32 values held in float64): the largest
    change of its MXFP4-dequantised value when h moves by up to the stated h
    error (H_REL_ERR relative + H_ABS_ERR units of its block scale), with the
    block's shared exponent taken at both ends of its amax's error range."""
    lead, I = h32.shape[:-1], h32.shape[-1]
    hb = np.asarray(h32, dtype=np.float64).reshape(lead + (I // 32, 32))
    amax = np.abs(hb).max(axis=-1)
    X = oracle.quant.block_exponent(amax)
    wa = H_REL_ERR * 2.1 * amax + H_ABS_ERR * np.ldexp(1.0, X)
    width = H_REL_ERR * 2.1 * np.abs(hb) + H_ABS_ERR * np.ldexp(1.0, X)[..., None]
    cur = _mx_dequant(hb, X)
    gap = np.zeros_like(hb)
    for Xc in (oracle.quant.block_exponent(np.maximum(amax - wa, 0.0)), X,
               oracle.quant.block_exponent(amax + wa)):
        for d in (-1.0, 0.0, 1.0):
            gap = np.maximum(gap, np.abs(_mx_dequant(hb + d * width, Xc) - cur))
    return gap.reshape(h32.shape)


def mx_scale_ambiguous(h32):
    """Per 32-element block of h32 [..., I]: True where the shared exponent of
    an h within the stated error may differ from that of h32."""
    lead, I = h32.shape[:-1], h32.shape[-1]
    hb = np.asarray(h32, dtype=np.float64).reshape(lead + (I // 32, 32))
    amax = np.abs(hb).max(axis=-1)
    wa = H_REL_ERR * 2.1 * amax + H_ABS_ERR * np.ldexp(1.0, oracle.quant.block_exponent(amax))
    return (oracle.quant.block_exponent(np.maximum(amax - wa, 0.0))
            != oracle.quant.block_exponent(amax + wa))


def output_slack(h32, ids, w, layer, tokens, gap_fn):
    """slack[ti, :] = sum_j |w[t, j]| |W2[e]| @ gap(h32[t, j]) for t = tokens[ti]."""
    k = ids.shape[1]
    H = layer["w2_blocks"].shape[1]
    slack = np.zeros((len(tokens), H))
    w2_cache = {}
    for ti, t in enumerate(tokens):
        for j in range(k):
            e = int(ids[t, j])
            if not 0 <= e < layer["w2_blocks"].shape[0]:
                continue
            gap = gap_fn(h32[t, j])
            nz = np.nonzero(gap)[0]
            if nz.size:
                if e not in w2_cache:
                    w2_cache[e] = oracle.dequant(layer["w2_blocks"][e], layer["w2_scales"][e])
                slack[ti] += abs(w[t, j]) * (np.abs(w2_cache[e][:, nz]) @ gap[nz])
    return slack


def make(name, layer):
    wl = synth.workload(name)
    t0 = time.time()
    k = synth.TOPK_GPT_OSS
    res = oracle.moe_forward(wl["x"], wl["logits"], **layer, k=k, act_mode=wl["act_mode"])
    T = wl["T"]
    if T <= 32:
        tokens = np.arange(T)
    else:
        rng = np.random.default_rng(7)
        tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, SAMPLE, replace=False)]))
    extra = {}
    if wl["act_mode"] in (synth.ACT_FP8_E4M3, synth.ACT_MXFP4):
        ids, w = res["ids"], res["weights"]
        if wl["act_mode"] == synth.ACT_FP8_E4M3:
            s = res["h_scale"]
            slack = output_slack(res["h32"], ids, w, layer, tokens, lambda h: code_gap(h, s))
        else:
            slack = output_slack(res["h32"], ids, w, layer, tokens, mx_code_gap)
        rng = np.random.default_rng(9)
        pairs = np.sort(rng.choice(T * k, H_PAIRS, replace=False))
        extra = dict(h_pairs=pairs.astype(np.int64),
                     h_ref=res["h"].reshape(T * k, -1)[pairs].astype(np.float32),
                     slack=slack.astype(np.float32), h_rel_err=np.float64(H_REL_ERR),
                     h_abs_err=np.float64(H_ABS_ERR))
        if wl["act_mode"] == synth.ACT_FP8_E4M3:
            extra.update(x_scale=np.float64(res["x_scale"]), h_scale=np.float64(s),
                         h_amax=np.float64(np.max(np.abs(res["h32"]))))
        print("  %s: ambiguous-code slack max %.3g rms(out) %.3g" % (
            name, slack.max(), np.sqrt(np.mean(res["out"][tokens] ** 2))), flush=True)
    np.savez_compressed(golden_path(name), tokens=tokens.astype(np.int64),
                        out=res["out"][tokens].astype(np.float32), **extra)
    print("%s: T=%d, %.1f s" % (name, T, time.time() - t0), flush=True)


def main(names):
    layer = synth.layer()
    for n in names:
        make(n, layer)


if __name__ == "__main__":
    main(sys.argv[1:] or list(synth.MOE_WORKLOADS))
