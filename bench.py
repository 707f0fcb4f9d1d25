#!/usr/bin/env python3
"""Throughput of the MXFP4 MoE layer on one MI355X, with roofline context.

A step is one pass of the hot path over one batch: router top-k, then the MoE
layer (permutation, [FP8 quantisation of x], gate_up GEMM + SwiGLU, [FP8
quantisation of h], down GEMM, weighted combine), all through the C ABI.
Weights, logits and activations are resident in HBM before timing starts.
Before every timed step a 1 GiB buffer is read through (a reduction) so the
step reads its weights from HBM and not from the 256 MB last-level cache;
each step is bracketed by events on the launch stream and the eviction is
outside them.  (--flush write overwrites the buffer instead, which leaves
dirty lines whose write-back then competes with the timed step.)

The headline line is the 32-token decode batch (hidden 2880, 128 experts,
top-4, bf16 activations).  The same run also measures the 4-token decode,
the FP8 prefill workloads (2048 tokens; 8192 tokens with hot experts), both
decode batches with NVFP4 expert weights, the dense MXFP4 projections
(qkv_proj, o_proj, lm_head at 1 and 4 tokens) and the weight quantiser, and
times the float64 CPU oracle on a bounded sample for the cpu_baseline field.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--primary-only]
                       [--no-cpu-baseline] [--workload NAME]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer GB/s & % HBM roofline (decode 4–32 tok); MXFP4 TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # dense MFMA, bf16
FP8_PEAK_TFLOPS = 5000.0        # dense MFMA, FP8 (the FP8 x FP4 instruction's operand rate)
MXFP4_PEAK_TFLOPS = 10100.0     # dense MFMA, FP4 / FP6
PRIMARY = "moe_decode_t32"
ACT_NAMES = {0: "bf16", 1: "fp8_e4m3", 2: "mxfp4"}
FLUSH_BYTES = 1 << 30
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def expert_bytes(H, I):
    """Bytes of one expert's gate_up and down weights (blocks + scales + bf16 bias)."""
    gate_up = 2 * I * (H // 32) * 17 + 2 * I * 2
    down = H * (I // 32) * 17 + H * 2
    return gate_up, down


def h_bytes_written(pairs, I, act):
    """Bytes of h the gate_up kernel writes: bf16 hi + lo (bf16 activations) or
    fp32 (FP8) = 4 B per element; with MXFP4 activations the epilogue writes
    E2M1 codes and one E8M0 byte per 32 elements = 17/32 B per element."""
    if act == 2:
        return pairs * I * 17 // 32
    return pairs * I * 4


def moe_accounting(ids, T, H, I, act, E=128):
    """Algorithmic bytes and flops of one layer pass and of its gate_up kernel."""
    touched = len(np.unique(ids))
    pairs = ids.size
    gu, dn = expert_bytes(H, I)
    layer_bytes = touched * (gu + dn) + T * H * 2 + T * E * 4 + T * H * 2
    h_bytes = h_bytes_written(pairs, I, act)
    # bf16 x, E4M3 codes, or E2M1 codes + one scale byte per 32 read
    xin = T * H * 2 if act == 0 else T * H if act == 1 else T * H * 17 // 32
    gemm1_bytes = touched * gu + xin + h_bytes
    gemm1_flops = 2.0 * pairs * 2 * I * H
    flops = 2.0 * pairs * (2 * I * H + H * I)
    return dict(touched=touched, pairs=pairs, layer_bytes=layer_bytes, gemm1_bytes=gemm1_bytes,
                gemm1_flops=gemm1_flops, flops=flops)


def issued_peak_tflops(act):
    """Dense peak of the MFMA instructions a quantised layer issues: FP8 mode
    runs gate_up (2/3 of the flops) on the bf16 MFMA with exactly expanded
    operands and down (1/3) on the block-scaled FP8 x FP4 MFMA at the FP8 rate;
    MXFP4 activations run both on the FP4 x FP4 form at the FP4 rate."""
    if act == 2:
        return MXFP4_PEAK_TFLOPS
    if act == 1:
        return 1.0 / ((2.0 / 3.0) / BF16_PEAK_TFLOPS + (1.0 / 3.0) / FP8_PEAK_TFLOPS)
    return BF16_PEAK_TFLOPS


def tflops_fractions(tflops, flops, nbytes, act, ceiling_gbps=None):
    """The four readings of a prefill TFLOP/s figure: raw, against the nominal
    MXFP4 peak, against the peak of the issued MFMA form, and against the
    attainable roofline min(issued peak, AI x HBM) (nominal 8 TB/s, and the
    measured read ceiling when given)."""
    ai = flops / nbytes
    peak = issued_peak_tflops(act)
    out = dict(TFLOPs=tflops, frac_mxfp4_peak=tflops / MXFP4_PEAK_TFLOPS, issued_peak_TFLOPs=peak,
               frac_issued_peak=tflops / peak, flop_per_byte=ai,
               attainable_TFLOPs=min(peak, ai * HBM_PEAK_GBS / 1e3))
    out["frac_attainable"] = tflops / out["attainable_TFLOPs"]
    if ceiling_gbps:
        out["attainable_measured_TFLOPs"] = min(peak, ai * ceiling_gbps / 1e3)
        out["frac_attainable_measured"] = tflops / out["attainable_measured_TFLOPs"]
    return out


def source_digest(files):
    """Digest of the named files under csrc/ (a kernel's source and the headers it
    includes): counter readings taken on other sources are not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_block_scaled_top_amd", "csrc")
    for n in sorted(files):
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode() + f.read())
    return h.hexdigest()[:16]


class Runner:
    def __init__(self, torch, mx, flush_mode="read"):
        self.torch = torch
        self.mx = mx
        self.flush_mode = flush_mode
        self.flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def evict(self, i):
        """Push the layer out of the 256 MB last-level cache and the L2s.  "read"
        streams the 1 GiB buffer through a reduction, leaving clean lines behind;
        "write" overwrites it, which also leaves up to 256 MB of dirty lines that
        are written back while the next step runs."""
        if self.flush_mode == "write":
            self.flush.fill_(float(i))
        else:
            self._sink = self.flush.amax()

    def dev(self, a):
        torch = self.torch
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    def time_steps(self, step, steps, warmup, flush=True, stage_events=False):
        """Per-step event times (ms); optional per-stage times (ms) via the ABI events."""
        torch, mx = self.torch, self.mx
        for _ in range(warmup):
            if flush:
                self.evict(1)
            step(None)
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        evs = None
        if stage_events:
            evs = [[mx.mxfp4_event_create() for _ in range(mx.NUM_STAGES)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush:
                self.evict(i)
            starts[i].record()
            step(evs[i] if evs else None)
            ends[i].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
        stages = None
        if evs:
            stages = {}
            for a in range(mx.NUM_STAGES - 1):
                d = [mx.mxfp4_event_elapsed_ms(ev[a], ev[a + 1]) for ev in evs]
                stages[mx.STAGES[a + 1]] = float(np.mean(d))
            for ev in evs:
                for e in ev:
                    mx.mxfp4_event_destroy(e)
        return ms, stages, wall


def moe_setup(run, Ld, name, synth, prepare=True):
    torch, mx = run.torch, run.mx
    wl = synth.workload(name)
    T, H = wl["x"].shape
    I = synth.H_GPT_OSS
    E, k, act = synth.E_GPT_OSS, synth.TOPK_GPT_OSS, wl["act_mode"]
    logits = run.dev(wl["logits"])
    x = run.dev(wl["x"])
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.mxfp4_moe_workspace_size(T, H, I, E, k, act), dtype=torch.uint8, device="cuda")
    codes = None
    if act != 0 and prepare:
        # the E2M1 codes restaged once for the prefill GEMMs (a load-time step)
        codes = (mx.mxfp4_moe_prepare_code_stream(Ld["w13_blocks"], H, I, 0),
                 mx.mxfp4_moe_prepare_code_stream(Ld["w2_blocks"], H, I, 1))

    def step(events, ready=False, prepared_codes=False):
        # router + layer in one library call (its "permute" stage covers routing too)
        mx.mxfp4_moe_layer(x, logits, k, Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"],
                           Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], act, out=out,
                           topk_ids=ids, topk_weights=w, workspace=ws, events=events,
                           scale_streams_ready=ready, code_streams=codes if prepared_codes else None)

    step(None)
    torch.cuda.synchronize()
    acct = moe_accounting(ids.cpu().numpy(), T, H, I, act)
    return step, acct, wl


def measure_ceiling(run, nbytes=4 << 30, reps=10):
    """Streaming-read ceiling of this device: a buffer of `nbytes` (4 GiB,
    16 times the last-level cache) read once per launch with nontemporal
    register loads and with nontemporal direct-to-LDS copies; mean GB/s of
    `reps` launches after one warm-up each."""
    torch, mx = run.torch, run.mx
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dict(bytes=nbytes)
    for mode, key in ((0, "register_loads_GBps"), (1, "lds_dma_GBps")):
        n = mx.mxfp4_stream_read(buf, mode, sink)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            mx.mxfp4_stream_read(buf, mode, sink)
        b.record()
        torch.cuda.synchronize()
        out[key] = n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
        out["bytes_read"] = n
    out["ceiling_GBps"] = max(out["register_loads_GBps"], out["lds_dma_GBps"])
    del buf
    torch.cuda.empty_cache()
    return out


def graph_replay_times(run, step, steps, warmup):
    """Per-replay times (ms) of `step` captured in a HIP graph."""
    torch = run.torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(None)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(None)
    torch.cuda.synchronize()
    ms, _, _ = run.time_steps(lambda _ev: g.replay(), steps, warmup, flush=True)
    del g
    return ms


def measure_moe(run, Ld, name, synth, steps, warmup, ceiling_gbps=None, prepared_runs=True):
    step, acct, wl = moe_setup(run, Ld, name, synth, prepared_runs)
    ms, stages, wall = run.time_steps(step, steps, warmup, flush=True, stage_events=True)
    ms_plain, _, _ = run.time_steps(step, steps, warmup, flush=True, stage_events=False)
    warm, _, _ = run.time_steps(step, max(steps // 2, 3), 1, flush=False)
    graph_ms = None
    if wl["act_mode"] == 0:
        # the same call captured once in a HIP graph and replayed (the
        # launches of a serving loop); the cache eviction stays outside
        graph_ms = float(np.mean(graph_replay_times(run, step, steps, warmup)))
    prepared = prepared_all = prepared_stages = None
    if wl["act_mode"] != 0 and prepared_runs:
        # the weight scales restaged once (a load-time step for fixed weights):
        # every timed call passes MXFP4_OPT_SCALE_STREAMS_READY
        ms_prep, _, _ = run.time_steps(lambda ev: step(ev, True), steps, warmup, flush=True)
        prepared = float(np.mean(ms_prep))
        # ... and the E2M1 codes too (restaged code streams)
        _, prepared_stages, _ = run.time_steps(lambda ev: step(ev, True, True), steps, warmup, flush=True,
                                               stage_events=True)
        ms_all, _, _ = run.time_steps(lambda ev: step(ev, True, True), steps, warmup, flush=True)
        prepared_all = float(np.mean(ms_all))
    mean = float(np.mean(ms_plain))
    g1 = stages["gemm1"]
    act = wl["act_mode"]
    res = dict(
        tokens=wl["T"], act=ACT_NAMES[act], touched_experts=acct["touched"],
        ms_per_step=mean, ms_p10=float(np.percentile(ms_plain, 10)),
        ms_p50=float(np.median(ms_plain)), ms_p90=float(np.percentile(ms_plain, 90)),
        layer_GBps=acct["layer_bytes"] / mean / 1e6,
        layer_TFLOPs=acct["flops"] / mean / 1e9,
        layer_hbm_frac=acct["layer_bytes"] / mean / 1e6 / HBM_PEAK_GBS,
        warm_ms_per_step=float(np.mean(warm)),
        graph_ms_per_step=graph_ms,
        prepared_scales_ms_per_step=prepared,
        prepared_ms_per_step=prepared_all, prepared_stage_ms=prepared_stages,
        stage_ms=stages, gemm1_ms=g1,
        gemm1_GBps=acct["gemm1_bytes"] / g1 / 1e6,
        gemm1_TFLOPs=acct["gemm1_flops"] / g1 / 1e9,
        algorithmic_bytes=acct["layer_bytes"], gemm1_bytes=acct["gemm1_bytes"],
        flops=acct["flops"], wall_s=wall)
    if ceiling_gbps:
        res["layer_frac_measured_ceiling"] = res["layer_GBps"] / ceiling_gbps
        res["gemm1_frac_measured_ceiling"] = res["gemm1_GBps"] / ceiling_gbps
    if act != 0:
        res["layer_tflops"] = tflops_fractions(res["layer_TFLOPs"], acct["flops"], acct["layer_bytes"], act,
                                               ceiling_gbps)
        if prepared:
            res["layer_tflops_prepared_scales"] = tflops_fractions(
                acct["flops"] / prepared / 1e9, acct["flops"], acct["layer_bytes"], act, ceiling_gbps)
        if prepared_all:
            res["layer_tflops_prepared"] = tflops_fractions(
                acct["flops"] / prepared_all / 1e9, acct["flops"], acct["layer_bytes"], act, ceiling_gbps)
    return res


def nvfp4_expert_bytes(H, I):
    """Bytes of one NVFP4 expert: 16-element blocks of 8 bytes plus one E4M3
    scale byte each, bf16 bias."""
    gate_up = 2 * I * (H // 16) * 9 + 2 * I * 2
    down = H * (I // 16) * 9 + H * 2
    return gate_up, down


def measure_nvfp4(run, synth, steps, warmup, prepared_runs=True):
    """The MoE batches with NVFP4 expert weights: router top-k and the NVFP4
    MoE layer; the decode batches with bf16 activations, the prefill batches
    with E4M3 activations (both GEMMs on the bf16 MFMA with exactly expanded
    operands; also timed with the restaged scale streams kept)."""
    torch, mx = run.torch, run.mx
    L = synth.nvfp4_layer()
    Nd = {k: (run.dev(v) if isinstance(v, np.ndarray) else v) for k, v in L.items()}
    del L
    H = I = synth.H_GPT_OSS
    E, k = synth.E_GPT_OSS, synth.TOPK_GPT_OSS
    res = {}
    nv_codes = None
    for name in ("moe_decode_t4", "moe_decode_t32", "moe_prefill_t2048_fp8", "moe_prefill_t8192_fp8_skewed"):
        wl = synth.workload(name)
        T = wl["T"]
        act = wl["act_mode"]
        logits, x = run.dev(wl["logits"]), run.dev(wl["x"])
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mx.nvfp4_moe_workspace_size(T, H, I, E, k, act), dtype=torch.uint8, device="cuda")

        def step(events, ready=False, codes=None, logits=logits, x=x, ids=ids, w=w, out=out, ws=ws, act=act):
            mx.mxfp4_route_topk(logits, k, topk_ids=ids, topk_weights=w)
            mx.nvfp4_moe_forward(x, ids, w, Nd["w13_blocks"], Nd["w13_scales"], Nd["w13_global"],
                                 Nd["w13_bias"], Nd["w2_blocks"], Nd["w2_scales"], Nd["w2_global"],
                                 Nd["w2_bias"], out=out, workspace=ws, events=events, act_mode=act,
                                 scale_streams_ready=ready, code_streams=codes)

        step(None)
        torch.cuda.synchronize()
        touched = len(np.unique(ids.cpu().numpy()))
        gu, dn = nvfp4_expert_bytes(H, I)
        layer_bytes = touched * (gu + dn) + T * H * 2 + T * E * 4 + T * H * 2
        gemm1_bytes = touched * gu + T * H * (1 if act else 2) + ids.numel() * I * 4
        ms, stages, _ = run.time_steps(step, steps, warmup, flush=True, stage_events=True)
        ms_plain, _, _ = run.time_steps(step, steps, warmup, flush=True)
        mean = float(np.mean(ms_plain))
        flops = 2.0 * ids.numel() * (2 * I * H + H * I)
        r = dict(tokens=T, act=ACT_NAMES[act], touched_experts=touched, ms_per_step=mean,
                 layer_GBps=layer_bytes / mean / 1e6, layer_hbm_frac=layer_bytes / mean / 1e6 / HBM_PEAK_GBS,
                 layer_TFLOPs=flops / mean / 1e9, stage_ms=stages,
                 gemm1_GBps=gemm1_bytes / stages["gemm1"] / 1e6, algorithmic_bytes=layer_bytes)
        if act and prepared_runs:
            ms_prep, _, _ = run.time_steps(lambda ev: step(ev, True), steps, warmup, flush=True)
            r["prepared_scales_ms_per_step"] = float(np.mean(ms_prep))
            if nv_codes is None:
                nv_codes = (mx.mxfp4_moe_prepare_code_stream(Nd["w13_blocks"], H, I, 0),
                            mx.mxfp4_moe_prepare_code_stream(Nd["w2_blocks"], H, I, 1))
            ms_all, _, _ = run.time_steps(lambda ev: step(ev, True, nv_codes), steps, warmup, flush=True)
            r["prepared_ms_per_step"] = float(np.mean(ms_all))
        if act:
            # both GEMMs issue the bf16 MFMA
            r["frac_issued_peak"] = r["layer_TFLOPs"] / BF16_PEAK_TFLOPS
        res[name.replace("moe_", "moe_nvfp4_")] = r
    del Nd
    return res


def measure_dense(run, synth, steps, warmup):
    mx = run.mx
    out = {}
    for name, (N, K) in synth.DENSE_SHAPES.items():
        D = synth.dense(synth.DENSE_SEEDS[name], N, K)
        wb, wsc, b = run.dev(D["w_blocks"]), run.dev(D["w_scales"]), run.dev(D["bias"])
        for M in (1, 4):
            x = run.dev(synth.dense_x(synth.DENSE_X_SEED, M, K))
            y = run.torch.empty((M, N), dtype=run.torch.bfloat16, device="cuda")

            def step(_ev, x=x, y=y, wb=wb, wsc=wsc, b=b):
                mx.mxfp4_linear(x, wb, wsc, b, out=y)

            ms, _, _ = run.time_steps(step, steps, warmup, flush=True)
            nbytes = N * (K // 32) * 17 + 2 * N + M * K * 2 + M * N * 2
            mean = float(np.mean(ms))
            out["%s_m%d" % (name, M)] = dict(N=N, K=K, M=M, ms=mean, GBps=nbytes / mean / 1e6,
                                             hbm_frac=nbytes / mean / 1e6 / HBM_PEAK_GBS,
                                             TFLOPs=2.0 * M * N * K / mean / 1e9, bytes=nbytes)
        del wb, wsc, b
    return out


def dense_prefill_peak_tflops(act):
    """Dense peak of the block-scaled MFMA form a quantised dense projection
    issues: E4M3 x E2M1 at the FP8 rate, E2M1 x E2M1 at the FP4 rate."""
    return MXFP4_PEAK_TFLOPS if act == 2 else FP8_PEAK_TFLOPS


def measure_dense_prefill(run, synth, steps, warmup, tokens=2048):
    """The dense projections at a prefill's token count with quantised
    activations (x quantised inside the call): time per call, TFLOP/s and its
    fraction of the issued form's peak and of min(peak, AI x 8 TB/s)."""
    mx = run.mx
    out = {}
    for name, (N, K) in synth.DENSE_SHAPES.items():
        D = synth.dense(synth.DENSE_SEEDS[name], N, K)
        wb, wsc, b = run.dev(D["w_blocks"]), run.dev(D["w_scales"]), run.dev(D["bias"])
        x = run.dev(synth.dense_x(synth.DENSE_X_SEED + 100, tokens, K))
        y = run.torch.empty((tokens, N), dtype=run.torch.bfloat16, device="cuda")
        for act in (1, 2):
            ws = run.torch.empty(max(mx.mxfp4_linear_workspace_size(tokens, N, K, act), 1),
                                 dtype=run.torch.uint8, device="cuda")

            def step(_ev, x=x, y=y, wb=wb, wsc=wsc, b=b, act=act, ws=ws):
                mx.mxfp4_linear(x, wb, wsc, b, out=y, act_mode=act, workspace=ws)

            ms, _, _ = run.time_steps(step, steps, warmup, flush=True)
            mean = float(np.mean(ms))
            flops = 2.0 * tokens * N * K
            nbytes = N * (K // 32) * 17 + 2 * N + tokens * K * 2 + tokens * N * 2
            tf = flops / mean / 1e9
            peak = dense_prefill_peak_tflops(act)
            attain = min(peak, flops / nbytes * HBM_PEAK_GBS / 1e3)
            out["%s_%s_m%d" % (name, ACT_NAMES[act], tokens)] = dict(
                N=N, K=K, M=tokens, act=ACT_NAMES[act], ms=mean, TFLOPs=tf, issued_peak_TFLOPs=peak,
                frac_issued_peak=tf / peak, flop_per_byte=flops / nbytes, attainable_TFLOPs=attain,
                frac_attainable=tf / attain)
            del ws
        del wb, wsc, b, x, y
    return out


def measure_quantizer(run, synth, steps, warmup):
    """BF16 -> MXFP4 quantisation of the lm_head weight (201,088 x 2880): a stream
    of N*K*2 bytes in and N*K*17/32 bytes out."""
    mx = run.mx
    N, K = synth.DENSE_SHAPES["lm_head"]
    w = run.dev(synth.dense_bf16_weights(50, N, K))
    blocks = run.torch.empty((N, K // 32, 16), dtype=run.torch.uint8, device="cuda")
    scales = run.torch.empty((N, K // 32), dtype=run.torch.uint8, device="cuda")

    def step(_ev):
        mx.mxfp4_quantize_weights(w, blocks, scales)

    ms, _, _ = run.time_steps(step, steps, warmup, flush=True)
    nbytes = N * K * 2 + N * (K // 32) * 17
    mean = float(np.mean(ms))
    del w, blocks, scales
    return dict(N=N, K=K, ms=mean, GBps=nbytes / mean / 1e6, hbm_frac=nbytes / mean / 1e6 / HBM_PEAK_GBS,
                bytes=nbytes)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, budget_tokens=16, runs=3):
    """The float64 oracle on the first `budget_tokens` tokens of the headline batch
    (16 of 32 by default, about 50 experts), on host cores, `runs` timed passes;
    the rate is the median over the passes."""
    import oracle
    threads, blas = 1, "unknown"
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(sorted({"%s %s (%s)" % (i.get("internal_api", "?"), i.get("version", "?"),
                                                 i.get("threading_layer", "?"))
                                 for i in info if i.get("user_api") == "blas"})) or "none found"
    except Exception:
        pass
    L = synth.layer()
    wl = synth.workload(PRIMARY)
    x, logits = wl["x"][:budget_tokens], wl["logits"][:budget_tokens]
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        res = oracle.moe_forward(x, logits, **L, k=synth.TOPK_GPT_OSS, act_mode=wl["act_mode"])
        times.append(time.perf_counter() - t0)
    acct = moe_accounting(res["ids"], budget_tokens, synth.H_GPT_OSS, synth.H_GPT_OSS, 0)
    med = float(np.median(times))
    return dict(value=acct["layer_bytes"] / med / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample="first %d of the %d tokens of the decode batch (%d experts touched), float64 numpy, "
                       "median of %d passes (%s s)" % (budget_tokens, wl["T"], acct["touched"], runs,
                                                       ", ".join("%.2f" % t for t in times)),
                cpu_model=_cpu_model(), nproc=os.cpu_count(), blas=blas, seconds_median=med)


def pmc_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    ent = d.get(kernel)
    if not ent or not ent.get("sources"):
        return None
    try:
        if ent.get("source_digest") != source_digest(ent["sources"]):
            return None
    except OSError:
        return None
    return ent.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=PRIMARY)
    ap.add_argument("--primary-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=("read", "write"), default="read",
                    help="how the 1 GiB cache eviction before each timed step touches its buffer")
    ap.add_argument("--pmc-calibrate", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (3 times), the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only measure the streaming-read ceiling (4 GiB read once per launch, register "
                         "loads and direct-to-LDS copies) and print it")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling measurement")
    ap.add_argument("--no-prepared", action="store_true",
                    help="skip the prefill timings with restaged scales and codes (kernel traces of the "
                         "default path alone)")
    ap.add_argument("--dense-only", action="store_true",
                    help="only measure the dense projections (qkv_proj, o_proj, lm_head at 1 and 4 tokens) "
                         "and print them")
    ap.add_argument("--nvfp4-only", action="store_true",
                    help="only measure the NVFP4 decode layers (4 and 32 tokens) and print them")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (requested %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mxfp4_block_scaled_top_amd as mx
    import synth

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.pmc_calibrate:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 512 << 20, "bytes_written": 512 << 20,
                          "launches": 3}))
        return
    mx.lib()
    run = Runner(torch, mx, args.flush)
    ceiling = None if args.no_ceiling else measure_ceiling(run)
    if ceiling:
        print("bench: read ceiling %.0f GB/s (register loads %.0f, LDS DMA %.0f)"
              % (ceiling["ceiling_GBps"], ceiling["register_loads_GBps"], ceiling["lds_dma_GBps"]),
              file=sys.stderr, flush=True)
    if args.hbm_ceiling:
        print(json.dumps({"hbm_ceiling": ceiling}), flush=True)
        return
    cg = ceiling["ceiling_GBps"] if ceiling else None
    if args.dense_only:
        print(json.dumps({"dense": measure_dense(run, synth, args.steps, args.warmup),
                          "dense_prefill": measure_dense_prefill(run, synth, max(args.steps // 2, 5), 2)}),
              flush=True)
        return
    if args.nvfp4_only:
        print(json.dumps({"nvfp4": measure_nvfp4(run, synth, args.steps, args.warmup, not args.no_prepared)}),
              flush=True)
        return
    L = synth.layer()
    Ld = {k: run.dev(v) for k, v in L.items()}
    del L
    print("bench: layer resident (%.2f GB)" % (sum(t.numel() * t.element_size() for t in Ld.values()) / 1e9),
          file=sys.stderr, flush=True)

    def moe_line(name, r):
        extra = ""
        if r.get("prepared_ms_per_step"):
            extra = " (restaged scales and codes: %.1f us)" % (r["prepared_ms_per_step"] * 1e3)
        return "bench: %s %.1f us/step%s" % (name, r["ms_per_step"] * 1e3, extra)

    prim = measure_moe(run, Ld, args.workload, synth, args.steps, args.warmup, cg, not args.no_prepared)
    print(moe_line(args.workload, prim), file=sys.stderr, flush=True)
    others = {}
    if not args.primary_only:
        for name in synth.MOE_WORKLOADS:
            if name == args.workload:
                continue
            others[name] = measure_moe(run, Ld, name, synth, max(args.steps // 2, 5), 2, cg, not args.no_prepared)
            print(moe_line(name, others[name]), file=sys.stderr, flush=True)
        del Ld
        torch.cuda.empty_cache()
        others.update(measure_nvfp4(run, synth, max(args.steps // 2, 5), 2, not args.no_prepared))
        print("bench: nvfp4 decode %.1f / %.1f us (4 / 32 tokens), prefill %.1f / %.1f us (2048 / 8192 tokens)"
              % (others["moe_nvfp4_decode_t4"]["ms_per_step"] * 1e3,
                 others["moe_nvfp4_decode_t32"]["ms_per_step"] * 1e3,
                 others["moe_nvfp4_prefill_t2048_fp8"]["ms_per_step"] * 1e3,
                 others["moe_nvfp4_prefill_t8192_fp8_skewed"]["ms_per_step"] * 1e3), file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        others["dense"] = measure_dense(run, synth, max(args.steps // 2, 5), 2)
        print("bench: dense set done", file=sys.stderr, flush=True)
        others["dense_prefill"] = measure_dense_prefill(run, synth, max(args.steps // 3, 5), 2)
        print("bench: prefill dense set done", file=sys.stderr, flush=True)
        others["quantize_lm_head"] = measure_quantizer(run, synth, max(args.steps // 3, 5), 2)
        print("bench: quantiser %.1f us" % (others["quantize_lm_head"]["ms"] * 1e3), file=sys.stderr, flush=True)

    fp8 = prim["act"] != "bf16"
    fp4 = prim["act"] == "mxfp4"
    # the FP8 gate_up runs with copy waves while the experts average at most 64
    # rows (tokens * top-k <= 64 * experts)
    cw = fp8 and not fp4 and prim["tokens"] * 4 <= 64 * 128
    kname = ("prefill_gemm_kernel<true, 128, true, false, false>" if fp4 else
             "prefill_gemm_cw_kernel" if cw else
             "prefill_gemm_kernel<true, 128, false, false, false>" if fp8 else "gemv_persist_kernel<0, 12, false, false>")
    if fp8 and prim["tokens"] >= 4096:
        peak = MXFP4_PEAK_TFLOPS if fp4 else FP8_PEAK_TFLOPS
        roof = dict(bound="mfma", achieved=prim["gemm1_TFLOPs"], peak=peak, unit="TFLOP/s",
                    frac=prim["gemm1_TFLOPs"] / peak)
    else:
        roof = dict(bound="hbm", achieved=prim["gemm1_GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=prim["gemm1_GBps"] / HBM_PEAK_GBS)
    roof["kernel"] = kname
    roof["traffic"] = pmc_traffic(kname)
    if cg and roof["unit"] == "GB/s":
        roof["measured_ceiling"] = cg
        roof["frac_measured_ceiling"] = roof["achieved"] / cg
    line = {
        "metric": METRIC,
        "value": prim["layer_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prim["act"],
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": prim["tokens"], "experts": 128, "topk": 4,
                   "hidden": 2880, "intermediate": 2880, "weights": "mxfp4", "act": prim["act"],
                   "parallelism": "none (1 GPU)", "cache_eviction": "%s 1 GiB before each step" % args.flush},
        "hbm_frac": prim["layer_hbm_frac"],
        "hbm_ceiling": ceiling,
        "roofline": roof,
        "detail": prim,
        "workloads": others,
        "source_digest": source_digest(os.listdir(os.path.join(ROOT, "mxfp4_block_scaled_top_amd", "csrc"))),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
