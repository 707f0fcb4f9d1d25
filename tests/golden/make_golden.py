"""Writes the oracle's results for the full-size MoE workloads to tests/golden/.

Calls only ``oracle`` (float64 CPU reference) and ``synth`` (seeded inputs).
For each workload it stores, in <name>.npz:
  tokens    int64 [n]      tokens whose outputs are kept (all if T <= 32, else
                           a seeded sample including the first and last token)
  out       float32 [n, H] oracle output rows of those tokens
FP8 workloads also store
  x_scale, h_scale, h_amax the per-tensor quantisation values
  h_pairs   int64 [m]      a seeded sample of pair indices p = t*k + j
  h_ref     float32 [m, I] the oracle's h (before quantisation) of those pairs
  slack     float32 [n, H] per-output bound on how far the output may move if
                           h codes whose value lies within the stated h error
                           (H_REL_ERR relative + H_ABS_ERR code units) of an
                           E4M3 rounding boundary are taken as the neighbouring
                           code; both neighbours are correct roundings of an h
                           within that error, so the output is not unique there.
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
H_ABS_ERR = 1e-4      # in units of the h scale (quantised-value units)


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
    if wl["act_mode"] == synth.ACT_FP8_E4M3:
        s = res["h_scale"]
        ids, w = res["ids"], res["weights"]
        H = wl["x"].shape[1]
        slack = np.zeros((len(tokens), H))
        w2_cache = {}
        for ti, t in enumerate(tokens):
            for j in range(k):
                gap = code_gap(res["h32"][t, j], s)
                nz = np.nonzero(gap)[0]
                if nz.size:
                    e = int(ids[t, j])
                    if e not in w2_cache:
                        w2_cache[e] = oracle.dequant(layer["w2_blocks"][e], layer["w2_scales"][e])
                    slack[ti] += abs(w[t, j]) * (np.abs(w2_cache[e][:, nz]) @ gap[nz])
        del w2_cache
        rng = np.random.default_rng(9)
        pairs = np.sort(rng.choice(T * k, H_PAIRS, replace=False))
        extra = dict(x_scale=np.float64(res["x_scale"]), h_scale=np.float64(s),
                     h_amax=np.float64(np.max(np.abs(res["h32"]))), h_pairs=pairs.astype(np.int64),
                     h_ref=res["h"].reshape(T * k, -1)[pairs].astype(np.float32),
                     slack=slack.astype(np.float32), h_rel_err=np.float64(H_REL_ERR),
                     h_abs_err=np.float64(H_ABS_ERR))
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
