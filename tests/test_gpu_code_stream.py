"""Restaged E2M1 code streams (mxfp4_moe_prepare_code_stream) through the C ABI.

The stream is a layout of this library, not a step of the method, so the
checks are exact: the prepared bytes equal the documented layout built here
with numpy from the blocks, and the layer given the streams returns bitwise
the output it returns without them (the GEMMs then copy the same codes into
the same LDS places), in the E4M3, MXFP4-activation and NVFP4 prefill modes,
over K tails, ragged n-tiles, both row-tile heights, the copy-wave kernel and
the gpt-oss shape at 2048 tokens.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import bf16_dev_to_f64, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FP8 = synth.ACT_FP8_E4M3
A4 = synth.ACT_MXFP4


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import mxfp4_block_scaled_top_amd as m
    m.lib()
    return m


def _layout(blocks, which, H, I):
    """The stream as the header states it: for expert e, row tile nt and
    128-element step s, 256 rows of four 16-byte slots; slot j of row lr holds
    block 4s + (j ^ ((lr / 2) % 4)) of weight row r(lr) (gate_up: gate row
    min(128 nt + lr % 128, I - 1), plus I for lr >= 128; down: min(256 nt + lr,
    H - 1)), zeros past K."""
    E = blocks.shape[0]
    gu = which == 0
    nout, K = (I, H) if gu else (H, I)
    nb = K // 32
    b = blocks.reshape(E, -1, nb, 16)
    tiles = -(-nout // 128) if gu else -(-nout // 256)
    steps = -(-nb // 4)
    out = np.zeros((E, tiles, steps, 256, 4, 16), np.uint8)
    lr = np.arange(256)
    for nt in range(tiles):
        if gu:
            row = np.where(lr < 128, 0, nout) + np.minimum(nt * 128 + (lr & 127), nout - 1)
        else:
            row = np.minimum(nt * 256 + lr, nout - 1)
        for s in range(steps):
            for j in range(4):
                blk = 4 * s + (j ^ ((lr >> 1) & 3))
                ok = blk < nb
                out[:, nt, s, ok, j, :] = b[:, row[ok], blk[ok], :]
    return out.reshape(-1)


def _streams(mx, Ld, H, I):
    return (mx.mxfp4_moe_prepare_code_stream(Ld["w13_blocks"], H, I, 0),
            mx.mxfp4_moe_prepare_code_stream(Ld["w2_blocks"], H, I, 1))


@pytest.mark.parametrize("E,H,I", [(2, 288, 320), (3, 224, 192), (1, 64, 96)])
def test_stream_bytes_follow_the_layout(mx, E, H, I):
    L = synth.layer(seed=E * 3 + H, E=E, H=H, I=I)
    for which, name in ((0, "w13_blocks"), (1, "w2_blocks")):
        dev = to_dev(L[name], torch)
        got = mx.mxfp4_moe_prepare_code_stream(dev, H, I, which).cpu().numpy()
        ref = _layout(L[name], which, H, I)
        assert got.size == mx.mxfp4_moe_code_stream_size(H, I, E, which) == ref.size
        assert np.array_equal(got, ref), "%s E%d H%d I%d" % (name, E, H, I)


def _mx_pair(mx, L, x, ids, w, act, streams):
    Ld = {k: (None if v is None else to_dev(v, torch)) for k, v in L.items()}
    H, I = x.shape[1], L["w2_blocks"].shape[2] * 32
    args = (to_dev(x, torch), to_dev(ids.astype(np.int32), torch), to_dev(w.astype(np.float32), torch),
            Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"],
            act)
    plain = bf16_dev_to_f64(mx.mxfp4_moe_forward(*args))
    cs = _streams(mx, Ld, H, I) if streams else None
    got = bf16_dev_to_f64(mx.mxfp4_moe_forward(*args, code_streams=cs))
    torch.cuda.synchronize()
    return plain, got


# E, H, I, T, k: K tails of every kind (H/32, I/32 mod 8), ragged n-tiles,
# experts averaging <= 64 rows (copy waves; NVFP4 wide-N units) and more
SHAPES = [
    (8, 288, 320, 37, 4),
    (8, 288, 320, 300, 4),
    (4, 224, 192, 70, 2),
    (1, 256, 160, 9, 1),
    (16, 160, 256, 300, 4),
]


@pytest.mark.parametrize("act", [FP8, A4])
@pytest.mark.parametrize("E,H,I,T,k", SHAPES)
def test_layer_with_streams_is_bitwise_the_layer(mx, E, H, I, T, k, act):
    L = synth.layer(seed=E * 7 + H + act, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 5, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    plain, got = _mx_pair(mx, L, x, ids, w, act, True)
    assert np.isfinite(plain).all()
    assert np.array_equal(plain, got), "E%d H%d I%d T%d k%d act %d" % (E, H, I, T, k, act)


@pytest.mark.parametrize("E,H,I,T,k", [s for s in SHAPES if s[1] >= 160 and s[2] >= 160])
def test_nvfp4_layer_with_streams_is_bitwise_the_layer(mx, E, H, I, T, k):
    L = synth.nvfp4_layer(seed=E * 9 + H, E=E, H=H, I=I)
    Ld = {k_: (to_dev(v, torch) if isinstance(v, np.ndarray) else v) for k_, v in L.items()}
    logits, x = synth.moe_inputs(T + 6, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    args = (to_dev(x, torch), to_dev(ids.astype(np.int32), torch), to_dev(w.astype(np.float32), torch),
            Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_global"], Ld["w13_bias"], Ld["w2_blocks"],
            Ld["w2_scales"], Ld["w2_global"], Ld["w2_bias"])
    plain = bf16_dev_to_f64(mx.nvfp4_moe_forward(*args, act_mode=FP8))
    got = bf16_dev_to_f64(mx.nvfp4_moe_forward(*args, act_mode=FP8, code_streams=_streams(mx, Ld, H, I)))
    torch.cuda.synchronize()
    assert np.isfinite(plain).all()
    assert np.array_equal(plain, got), "nvfp4 E%d H%d I%d T%d k%d" % (E, H, I, T, k)


@pytest.mark.parametrize("name", ["moe_prefill_t2048_fp8", "moe_prefill_t2048_fp4"])
def test_gpt_oss_prefill_with_streams_is_bitwise_the_layer(mx, name):
    L = synth.layer()
    wl = synth.workload(name)
    ids, w = oracle.route_topk(wl["logits"], 4)
    plain, got = _mx_pair(mx, L, wl["x"], ids, w, wl["act_mode"], True)
    assert np.isfinite(plain).all()
    assert np.array_equal(plain, got), name


def test_stream_arguments_are_checked(mx):
    blocks = torch.zeros(2 * 64 * 3 * 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.Mxfp4Error):
        mx.mxfp4_moe_code_stream_size(96, 64, 2, 2)          # which
    with pytest.raises(mx.Mxfp4Error):
        mx.mxfp4_moe_code_stream_size(100, 64, 2, 0)         # H not a multiple of 32
    short = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.Mxfp4Error):
        mx.mxfp4_moe_prepare_code_stream(blocks.view(2, 64, 3, 16), 96, 32, 1, out=short)
