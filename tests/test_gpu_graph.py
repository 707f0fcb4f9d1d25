"""The router + layer call captured in a HIP graph (torch.cuda.CUDAGraph on
ROCm) and replayed.  The forum page ("[SM121] 4 bugs causing ! output +
gpt-oss-120B at 59 tok/s", Part 2) credits graph capture with most of its
decode speed-up.  The library's layer launches kernels only (no memset,
copy or synchronisation), so a capture of one call is the whole layer.

Each replay follows new inputs copied into the captured buffers and some
eager device work, and must give bitwise the output, router ids and weights
of an eager call on the same inputs (the same kernels run)."""

import numpy as np
import pytest

import synth
from helpers import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import mxfp4_block_scaled_top_amd as m
    m.lib()
    return m


def _layer(mx, Ld, x, logits, k, act, out, ids, w, ws):
    return mx.mxfp4_moe_layer(x, logits, k, Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"],
                              Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], act, out=out,
                              topk_ids=ids, topk_weights=w, workspace=ws)


def _replays_match_eager(mx, Ld, E, H, I, T, k, act, seeds):
    dev = dict(dtype=torch.bfloat16, device="cuda")
    x = torch.empty((T, H), **dev)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), **dev)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(mx.mxfp4_moe_workspace_size(T, H, I, E, k, act), dtype=torch.uint8, device="cuda")
    lg0, x0 = synth.moe_inputs(seeds[0], T, E=E, H=H)
    x.copy_(to_dev(x0, torch))
    logits.copy_(to_dev(lg0, torch))
    # warm-up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _layer(mx, Ld, x, logits, k, act, out, ids, w, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _layer(mx, Ld, x, logits, k, act, out, ids, w, ws)
    torch.cuda.synchronize()
    out_e = torch.empty_like(out)
    ids_e = torch.empty_like(ids)
    w_e = torch.empty_like(w)
    ws_e = torch.empty_like(ws)
    for seed in seeds:
        lg, xb = synth.moe_inputs(seed, T, E=E, H=H)
        x.copy_(to_dev(xb, torch))
        logits.copy_(to_dev(lg, torch))
        scratch = torch.randn(1 << 20, device="cuda")      # eager work between replays
        scratch.mul_(2.0).add_(1.0)
        g.replay()
        torch.cuda.synchronize()
        _layer(mx, Ld, x, logits, k, act, out_e, ids_e, w_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_e) and torch.equal(w, w_e), "router outputs differ (seed %d)" % seed
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), "layer output differs (seed %d)" % seed
        assert float(scratch.abs().sum()) > 0
    del g


@pytest.mark.parametrize("T", [4, 32])
def test_decode_layer_replays_in_a_graph(mx, T):
    """The gpt-oss MoE layer at the decode batch sizes (bf16 activations; at 4
    tokens the gate_up kernel routes the batch itself)."""
    L = synth.layer()
    Ld = {k: (None if v is None else to_dev(v, torch)) for k, v in L.items()}
    _replays_match_eager(mx, Ld, synth.E_GPT_OSS, synth.H_GPT_OSS, synth.H_GPT_OSS, T, synth.TOPK_GPT_OSS,
                         synth.ACT_BF16, seeds=[70 + T, 71 + T, 72 + T])


@pytest.mark.parametrize("act", [synth.ACT_FP8_E4M3, synth.ACT_MXFP4])
def test_quantised_layer_replays_in_a_graph(mx, act):
    """A small layer in the quantised modes (per-tensor amax words, the scale
    restaging and the tile list are all rebuilt inside every replay)."""
    E, H, I, T, k = 8, 256, 320, 150, 4
    L = synth.layer(seed=77, E=E, H=H, I=I)
    Ld = {kk: (None if v is None else to_dev(v, torch)) for kk, v in L.items()}
    _replays_match_eager(mx, Ld, E, H, I, T, k, act, seeds=[80, 81, 82])
