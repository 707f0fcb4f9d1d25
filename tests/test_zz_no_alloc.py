"""The allocation-free router + layer entry point (mxfp4_moe_layer_noalloc)
against the workspace entry point (mxfp4_moe_layer), through the C ABI.

The two run the same kernels; the allocation-free one works in the library's
fixed device scratch.  Its outputs (top-k ids, weights and the layer output)
must equal the workspace entry point's bit for bit, on two calls in a row
with the second smaller than the first (the scratch keeps the first call's
contents), in every activation mode that fits the scratch, and at the
headline decode shape.  Sizes beyond the scratch are refused.
"""

import numpy as np
import pytest

import oracle
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


def _dev(L):
    return {k: (None if v is None else to_dev(v, torch)) for k, v in L.items()}


def _both(mx, Ld, x, logits, k, act):
    """One call of each entry point on the same inputs; asserts bitwise equality."""
    T, H = x.shape
    xd, ld = to_dev(x, torch), to_dev(logits, torch)
    args = (Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"])
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((T, k), -5, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    mx.mxfp4_moe_layer_noalloc(xd, ld, k, *args, act, out, ids, w)
    ref_out, ref_ids, ref_w = mx.mxfp4_moe_layer(xd, ld, k, *args, act)
    torch.cuda.synchronize()
    assert torch.equal(ids, ref_ids)
    assert torch.equal(w, ref_w)
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    rid, _ = oracle.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    return out


@pytest.mark.parametrize("act", [synth.ACT_BF16, synth.ACT_FP8_E4M3, synth.ACT_MXFP4])
def test_noalloc_equals_workspace_entry_two_calls(mx, act):
    E, H, I, k = 16, 288, 320, 4
    L = synth.layer(seed=71, E=E, H=H, I=I)
    Ld = _dev(L)
    for T in (40, 5):           # the second call is smaller than the first
        logits, x = synth.moe_inputs(72 + T, T, E=E, H=H)
        _both(mx, Ld, x, logits, k, act)


def test_noalloc_decode_workloads(mx):
    # the gpt-oss MoE shape: 32-token decode batch, then the 4-token one
    Ld = _dev(synth.layer())
    for name in ("moe_decode_t32", "moe_decode_t4"):
        wl = synth.workload(name)
        _both(mx, Ld, wl["x"], wl["logits"], synth.TOPK_GPT_OSS, wl["act_mode"])


def test_noalloc_refuses_sizes_beyond_the_scratch(mx):
    # 400 tokens x top-4 at hidden = intermediate = 2880 need about 37 MB of
    # intermediates, more than the 32 MiB scratch
    E, H, I, T, k = 4, 2880, 2880, 400, 4
    L = synth.layer(seed=81, E=E, H=H, I=I)
    Ld = _dev(L)
    logits, x = synth.moe_inputs(82, T, E=E, H=H)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    assert mx.mxfp4_moe_workspace_size(T, H, I, E, k, synth.ACT_BF16) > (32 << 20)
    with pytest.raises(mx.Mxfp4Error) as ei:
        mx.mxfp4_moe_layer_noalloc(to_dev(x, torch), to_dev(logits, torch), k, Ld["w13_blocks"], Ld["w13_scales"],
                                   Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], synth.ACT_BF16,
                                   out, ids, w)
    assert ei.value.status == 5
    # a size that fits still runs after the refusal
    _both(mx, Ld, x[:60], logits[:60], k, synth.ACT_BF16)
