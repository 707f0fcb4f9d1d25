"""GPU edge cases of the codecs and of the E8M0 scale range, against the oracle.

* The FP8 E4M3 codec (``mxfp4_quant_fp8_e4m3``, the codec of the FP8 MoE
  mode) on fp32 inputs placed on and a few ulps either side of every rounding
  midpoint between E4M3 values, both signs, subnormal steps included, and on
  the largest quotient the per-tensor scale can produce (just above 448).
* The BF16 -> MXFP4 quantiser on every finite bf16 pattern, each in blocks
  whose largest element fixes the shared exponent at several offsets from
  the pattern's own binade, and on a block below the exponent clamp.
* MoE layers whose E8M0 scale bytes sit at the ends of the range each mode
  accepts: 0, 1, 253 and 254 with MXFP4 activations; 11, 12, 251 and 252
  with bf16 and FP8 activations, and the dense projection at 11 and 252.

Every expected value comes from the oracle (float64 CPU reference).
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close_rounded, bf16_bits_to_f64, bf16_dev_to_f64, to_dev
from test_gpu_parity import _layer_dev, _mx_act_check, _run_moe, mx  # noqa: F401  (mx: fixture)
from test_oracle_quant import small_block_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- E4M3 codec ----


def _e4m3_midpoint_values():
    """Positive fp32 values on, and up to 64 fp32 steps either side of, every
    midpoint between consecutive finite E4M3 magnitudes (0 .. 448)."""
    mags = np.unique(np.abs(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)       # exact in fp32
    steps = np.arange(-64, 65, dtype=np.int64)
    bits = mids.view(np.uint32).astype(np.int64)[:, None] + steps[None, :]
    return bits.astype(np.uint32).view(np.float32).reshape(-1)


@pytest.mark.parametrize("k", [-40, 0, 20])
def test_quant_fp8_fp32_midpoints_power_of_two_scale(mx, k):
    # one element 448 * 2^k fixes s = 2^k exactly, so every quotient is the
    # planted value itself: on, below and above each rounding midpoint
    v = _e4m3_midpoint_values()
    v = np.concatenate([[448.0], v, -v, [0.0, -0.0]]).astype(np.float32)
    v = (v.astype(np.float64) * 2.0 ** k).astype(np.float32)
    assert np.array_equal(v.astype(np.float64) / 2.0 ** k, np.concatenate(
        [[448.0], _e4m3_midpoint_values(), -_e4m3_midpoint_values(), [0.0, -0.0]]))
    codes, scale, amax = mx.mxfp4_quant_fp8_e4m3(to_dev(v, torch))
    rc, rs, ra = oracle.quant_per_tensor(v.astype(np.float64))
    assert rs == 2.0 ** k and float(scale.item()) == rs and float(amax.item()) == ra
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc)
    assert got[-1] == 0x80 and got[-2] == 0x00          # sign of zero kept


def test_quant_fp8_fp32_near_midpoints_rounded_scale(mx):
    # a scale that is not a power of two: quotients land near the midpoints
    # after the correctly rounded divide
    v = _e4m3_midpoint_values()
    f = np.float32(1.3)
    v = np.concatenate([[448.0], v, -v]).astype(np.float32) * f
    codes, scale, amax = mx.mxfp4_quant_fp8_e4m3(to_dev(v, torch))
    rc, rs, ra = oracle.quant_per_tensor(v.astype(np.float64))
    assert float(scale.item()) == rs and float(amax.item()) == ra
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_fp8_quotient_above_448_saturates(mx):
    # amax values whose scale fp32(amax/448) rounds down, so that the largest
    # quotient fp32(amax/s) is just above 448: the code saturates to 448
    rng = np.random.default_rng(5)
    cand = (448.0 * rng.uniform(1.0, 2.0, 20000)).astype(np.float32).astype(np.float64)
    s = (cand / 448.0).astype(np.float32).astype(np.float64)
    q = (cand / s).astype(np.float32).astype(np.float64)
    picks = cand[q > 448.0][:8]
    assert picks.size == 8
    for a in picks:
        v = np.array([a, -a, a / 3, 1.0, -0.0], dtype=np.float32)
        codes, scale, amax = mx.mxfp4_quant_fp8_e4m3(to_dev(v, torch))
        rc, rs, ra = oracle.quant_per_tensor(v.astype(np.float64))
        assert float(scale.item()) == rs and float(amax.item()) == ra
        got = codes.cpu().numpy()
        assert np.array_equal(got, rc)
        assert got[0] == 0x7E and got[1] == 0xFE


# ------------------------------------------------------- BF16 -> MXFP4 quantiser ----


def _every_bf16_in_pinned_blocks():
    """Blocks of 31 finite bf16 patterns from one binade 2^b (both signs) plus
    one element 2^(b + d) that fixes the block's exponent: d = 0 gives
    quotients in [4, 8) (the pattern's own binade is the block's top binade;
    its element is then 2^b itself), d = 1..4 quotients in [2, 4) down to
    [0.25, 0.5).  Returns bf16 bits [nblocks, 32]."""
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        val = (bits << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(val)
    bits, val = bits[fin].astype(np.uint16), val[fin]
    nz = val != 0
    binade = np.full(val.shape, 0, dtype=np.int64)
    binade[nz] = np.floor(np.log2(np.abs(val[nz]))).astype(np.int64)
    rows = []
    for b in np.unique(binade[nz]):
        members = bits[nz & (binade == b)]
        for d in range(5):
            if b + d > 127:
                continue
            pin = synth.f32_to_bf16_bits(np.array([np.ldexp(1.0, int(b + d))], dtype=np.float32))[0]
            assert bf16_bits_to_f64(pin) == np.ldexp(1.0, int(b + d))
            for i in range(0, members.size, 31):
                chunk = members[i:i + 31]
                row = np.full(32, pin, dtype=np.uint16)
                row[1:1 + chunk.size] = chunk
                rows.append(row)
    zeros = bits[~nz]                              # +0 and -0
    rows.append(np.concatenate([zeros, np.full(30, zeros[0], np.uint16)]))
    return np.stack(rows)


def test_quantize_weights_every_bf16_pattern(mx):
    w = _every_bf16_in_pinned_blocks()
    got_b, got_s = mx.mxfp4_quantize_weights(to_dev(w, torch))
    torch.cuda.synchronize()
    rb, rs = oracle.quantize_mxfp4(bf16_bits_to_f64(w))
    assert np.array_equal(got_s.cpu().numpy(), rs)
    assert np.array_equal(got_b.cpu().numpy(), rb)
    assert w.shape[0] > 10000


def test_quantize_weights_block_below_the_clamp(mx):
    # the hand-worked block with amax 2^-124 (tests/golden/mxfp4_small_block_case.txt)
    v, want, sbyte = small_block_case()
    w = synth.f32_to_bf16_bits(np.stack([v, -v]).astype(np.float32))
    got_b, got_s = mx.mxfp4_quantize_weights(to_dev(w, torch))
    torch.cuda.synchronize()
    codes = oracle.unpack_nibbles(got_b.cpu().numpy())
    assert got_s.cpu().numpy().tolist() == [[sbyte], [sbyte]]
    assert np.array_equal(codes[0, :], want)
    assert np.array_equal(codes[1, :], want ^ 8)


# ------------------------------------------------------- E8M0 scale-byte edges ----


def _scaled_x(x, factors):
    """x (bf16 bits [T, H]) with 32-element block b of every row multiplied by
    factors[b] (powers of two), rounded back to bf16."""
    f = np.repeat(np.asarray(factors, dtype=np.float64), 32)
    return synth.f32_to_bf16_bits((bf16_bits_to_f64(x) * f).astype(np.float32))


def test_mxfp4_act_w13_scale_bytes_0_1_253_254(mx):
    # gate_up weights: K block 0 with scale bytes 0 / 1 (2^-127, 2^-126),
    # K block 1 with 253 / 254 (2^126, 2^127).  x block 0 is scaled up by
    # 2^120 and x block 1 down by 2^-110 (tokens 0-3) or 2^-117 (tokens 4-7:
    # amax below 2^-114, where the activation quantiser's exponent clamp at
    # -116 applies), so every product stays finite and both blocks contribute.
    E, H, I, T, k = 2, 64, 64, 8, 2
    L = synth.layer(seed=301, E=E, H=H, I=I)
    rng = np.random.default_rng(302)
    L["w13_scales"][:, :, 0] = rng.integers(0, 2, size=(E, 2 * I), dtype=np.uint8)
    L["w13_scales"][:, :, 1] = rng.integers(253, 255, size=(E, 2 * I), dtype=np.uint8)
    logits, x = synth.moe_inputs(303, T, E=E, H=H)
    x = np.concatenate([_scaled_x(x[:4], [2.0 ** 120, 2.0 ** -110]),
                        _scaled_x(x[4:], [2.0 ** 120, 2.0 ** -117])])
    ids, w = oracle.route_topk(logits, k)
    _mx_act_check(mx, L, x, ids, w, "w13 scale bytes 0/1/253/254")


def test_mxfp4_act_w2_scale_bytes_0_1(mx):
    # down weights at scale bytes 0 and 1 only and no down bias; gate_up at
    # bytes 133..137 makes h of order 2^24, so the down products (order
    # 2^-103) stay in the normal fp32 range while bytes 0 and 1 decide them
    E, H, I, T, k = 2, 96, 64, 8, 2
    L = synth.layer(seed=311, E=E, H=H, I=I)
    rng = np.random.default_rng(312)
    L["w13_scales"] = rng.integers(133, 138, size=L["w13_scales"].shape, dtype=np.uint8)
    L["w2_scales"] = rng.integers(0, 2, size=L["w2_scales"].shape, dtype=np.uint8)
    L["w2_bias"] = None
    logits, x = synth.moe_inputs(313, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    _mx_act_check(mx, L, x, ids, w, "w2 scale bytes 0/1")


def test_mxfp4_act_w2_scale_bytes_253_254(mx):
    # down weights at scale bytes 253 and 254; the up rows of gate_up use
    # scale bytes 8..12 and no bias, so h is of order 2^-110 and the down
    # products stay finite
    E, H, I, T, k = 2, 96, 64, 8, 2
    L = synth.layer(seed=321, E=E, H=H, I=I)
    rng = np.random.default_rng(322)
    L["w13_scales"][:, I:, :] = rng.integers(8, 13, size=(E, I, H // 32), dtype=np.uint8)
    L["w13_bias"] = None
    L["w2_scales"] = rng.integers(253, 255, size=L["w2_scales"].shape, dtype=np.uint8)
    logits, x = synth.moe_inputs(323, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    _mx_act_check(mx, L, x, ids, w, "w2 scale bytes 253/254")


@pytest.mark.parametrize("act,b0,xexp", [(synth.ACT_BF16, 11, 116), (synth.ACT_FP8_E4M3, 11, 116),
                                         (synth.ACT_BF16, 251, -100), (synth.ACT_FP8_E4M3, 200, -40)])
def test_bf16_fp8_modes_w13_scale_bytes_11_12_251_252(mx, act, b0, xexp):
    # the ends of the byte range these modes accept ([11, 252]) in gate_up:
    # every w13 scale byte b0 / b0 + 1 against x scaled by 2^xexp.  (The FP8
    # mode sums weights times E4M3 codes up to 448 before the per-tensor
    # scale, so its top case stays where those sums fit fp32.)
    E, H, I, T, k = 2, 64, 64, 6, 2
    L = synth.layer(seed=331, E=E, H=H, I=I)
    rng = np.random.default_rng(332)
    L["w13_scales"] = rng.integers(b0, b0 + 2, size=L["w13_scales"].shape, dtype=np.uint8)
    logits, x = synth.moe_inputs(333, T, E=E, H=H)
    x = _scaled_x(x, [2.0 ** xexp, 2.0 ** xexp])
    ids, w = oracle.route_topk(logits, k)
    got = _run_moe(mx, _layer_dev(L), x, ids, w, act)
    ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=act)["out"]
    assert np.all(np.isfinite(ref))
    assert_close_rounded(got, ref, "w13 scale bytes %d/%d act%d" % (b0, b0 + 1, act))


@pytest.mark.parametrize("act", [synth.ACT_BF16, synth.ACT_FP8_E4M3])
def test_bf16_fp8_modes_w2_scale_bytes_11_12(mx, act):
    # down weights at bytes 11 / 12 only and no down bias: outputs of order
    # 2^-110, decided by those bytes alone
    E, H, I, T, k = 2, 96, 64, 6, 2
    L = synth.layer(seed=351, E=E, H=H, I=I)
    rng = np.random.default_rng(352)
    L["w2_scales"] = rng.integers(11, 13, size=L["w2_scales"].shape, dtype=np.uint8)
    L["w2_bias"] = None
    logits, x = synth.moe_inputs(353, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    got = _run_moe(mx, _layer_dev(L), x, ids, w, act)
    ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=act)["out"]
    assert_close_rounded(got, ref, "w2 scale bytes 11/12 act%d" % act)


def test_bf16_mode_w2_scale_bytes_251_252(mx):
    # down rows alternate between bytes 11 / 12 and 251 / 252; the up rows of
    # gate_up take bytes 11..15 and no bias, so h is of order 2^-110 and the
    # 251 / 252 rows stay finite (the 11 / 12 rows leave the down bias alone)
    E, H, I, T, k = 2, 96, 64, 6, 2
    L = synth.layer(seed=341, E=E, H=H, I=I)
    rng = np.random.default_rng(342)
    L["w13_scales"][:, I:, :] = rng.integers(11, 16, size=(E, I, H // 32), dtype=np.uint8)
    L["w13_bias"] = None
    s2 = rng.integers(11, 13, size=L["w2_scales"].shape).astype(np.uint8)
    s2[:, 1::2, :] = rng.integers(251, 253, size=s2[:, 1::2, :].shape, dtype=np.uint8)
    L["w2_scales"] = s2
    logits, x = synth.moe_inputs(343, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    got = _run_moe(mx, _layer_dev(L), x, ids, w, synth.ACT_BF16)
    ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=synth.ACT_BF16)["out"]
    assert np.all(np.isfinite(ref))
    assert_close_rounded(got, ref, "w2 scale bytes 11/12/251/252 bf16")


def test_linear_scale_bytes_11_and_252(mx):
    # the dense projection at the ends of its byte range: a one-hot x picks
    # one column of W, so each output is a single weight times a power of two
    for s, e in ((11, 116), (12, 115), (252, -125), (200, -73)):
        for N in (16, 4096):
            codes = np.zeros((N, 32), np.uint8)
            codes[:, 5] = np.arange(N) % 16
            blocks = (codes[:, 0::2] | (codes[:, 1::2] << 4)).reshape(N, 1, 16).astype(np.uint8)
            scales = np.full((N, 1), s, np.uint8)
            x = np.zeros((1, 32), np.float32)
            x[0, 5] = 2.0 ** e
            xb = synth.f32_to_bf16_bits(x)
            out = mx.mxfp4_linear(to_dev(xb, torch), to_dev(blocks, torch), to_dev(scales, torch))
            torch.cuda.synchronize()
            ref = oracle.linear(xb, blocks, scales)
            assert np.array_equal(bf16_dev_to_f64(out), ref), "byte %d N %d" % (s, N)
