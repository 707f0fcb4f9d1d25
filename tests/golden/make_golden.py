"""Writes the oracle's results for the full-size MoE workloads to tests/golden/.

Calls only ``oracle`` (float64 CPU reference), ``synth`` (seeded inputs) and
the test helpers of ``tests/parity.py`` (which call only the oracle).  For
each workload it stores, in <name>.npz:
  tokens    int64 [n]      tokens whose outputs are kept (all if T <= 32, else
                           a seeded sample including the first and last token)
  out       float32 [n, H] oracle output rows of those tokens
FP8 and MXFP4-activation workloads also store, for every pair p = t*k + j of
the sampled tokens (in token order):
  pairs     int64 [n*k]    the pair indices
  h_ref     float32 [n*k, I] the oracle's h of those pairs, rounded to fp32
                           (the value both sides quantise)
  h_tol     float32 [n*k, I] the bound on a kernel's fp32 error in h from
                           parity.h_tolerance (rounded up to fp32)
and FP8 workloads x_scale, h_scale and h_amax (the per-tensor values).
Run: python tests/golden/make_golden.py [workload ...]
"""

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import synth  # noqa: E402
from parity import activations, pair_h_tolerance  # noqa: E402

SAMPLE = 16


def golden_path(name):
    return os.path.join(HERE, "%s.npz" % name)


def make(name, layer):
    wl = synth.workload(name)
    t0 = time.time()
    k = synth.TOPK_GPT_OSS
    act = wl["act_mode"]
    res = oracle.moe_forward(wl["x"], wl["logits"], **layer, k=k, act_mode=act)
    T = wl["T"]
    if T <= 32:
        tokens = np.arange(T)
    else:
        rng = np.random.default_rng(7)
        tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, SAMPLE, replace=False)]))
    extra = {}
    if act in (synth.ACT_FP8_E4M3, synth.ACT_MXFP4):
        pairs = (tokens[:, None] * k + np.arange(k)[None, :]).reshape(-1)
        tol = pair_h_tolerance(activations(res, wl["x"], act), res["ids"], layer, pairs, k)
        tol32 = tol.astype(np.float32)
        tol32 = np.where(tol32.astype(np.float64) < tol, np.nextafter(tol32, np.float32(np.inf)), tol32)
        extra = dict(pairs=pairs.astype(np.int64),
                     h_ref=res["h32"].reshape(T * k, -1)[pairs].astype(np.float32),
                     h_tol=tol32)
        if act == synth.ACT_FP8_E4M3:
            extra.update(x_scale=np.float64(res["x_scale"]), h_scale=np.float64(res["h_scale"]),
                         h_amax=np.float64(np.max(np.abs(res["h32"]))))
        rel = tol / np.maximum(np.abs(res["h32"].reshape(T * k, -1)[pairs]), 1e-30)
        print("  %s: h error bound median %.2e relative" % (name, float(np.median(rel))), flush=True)
    np.savez_compressed(golden_path(name), tokens=tokens.astype(np.int64),
                        out=res["out"][tokens].astype(np.float32), **extra)
    print("%s: T=%d, %.1f s" % (name, T, time.time() - t0), flush=True)


def main(names):
    layer = synth.layer()
    for n in names:
        make(n, layer)


if __name__ == "__main__":
    main(sys.argv[1:] or list(synth.MOE_WORKLOADS))
