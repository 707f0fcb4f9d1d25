"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bars: top-k ids, permutation and FP8 codes bit-exact; layer outputs within
relative Frobenius error 2e-3 and max |error| 2e-2 * rms(reference).  In the
quantised modes the codes of h are compared with the oracle's codes of its h:
a code may differ only where an h within the fp32 error bound of the kernel's
arithmetic (parity.h_tolerance) rounds to it, and the outputs are then held to
the bar beyond the change those codes alone make (SLACK_MAX bounds it).
"""

import os

import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_close, assert_close_rounded, assert_close_rounded_slack, assert_close_slack,
                     bf16_bits_to_f64, bf16_dev_to_f64, errors, no_constant_rows, to_dev)
from parity import (activations, down_combine, fp8_code_mismatch, mismatch_slack, mx_code_mismatch,
                    pair_h_tolerance)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
# At full and mid size: largest share of h codes that may differ from the
# oracle's (each within the h error bound), and largest allowance they may
# take, as a fraction of the output norm.  One differing E2M1 code moves one
# h element by a whole E2M1 step (up to 2^(X+1)); over the 18 sampled tokens
# of a full-size golden that alone is about 3e-4 of the output norm.
DIFF_MAX = 1e-4
SLACK_MAX = 4e-4


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import mxfp4_block_scaled_top_amd as m
    m.lib()
    return m


def _layer_dev(L):
    return {k: (None if v is None else to_dev(v, torch)) for k, v in L.items()}


def _run_moe(mx, Ld, x_bits, ids, w, act_mode, want_ws=False):
    T = x_bits.shape[0]
    E, twoI = Ld["w13_blocks"].shape[:2]
    H = x_bits.shape[1]
    k = ids.shape[1]
    ws_bytes = mx.mxfp4_moe_workspace_size(T, H, twoI // 2, E, k, act_mode)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = mx.mxfp4_moe_forward(to_dev(x_bits, torch), to_dev(ids.astype(np.int32), torch),
                               to_dev(w.astype(np.float32), torch), Ld["w13_blocks"],
                               Ld["w13_scales"], Ld["w13_bias"], Ld["w2_blocks"],
                               Ld["w2_scales"], Ld["w2_bias"], act_mode, workspace=ws)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)
    if not want_ws:
        return got
    lay = mx.mxfp4_moe_workspace_layout_query(T, H, twoI // 2, E, k, act_mode)
    return got, ws, lay


def _ws_view(ws, lay, key, dtype, count):
    nbytes = np.dtype(dtype).itemsize * count
    return ws[lay[key]:lay[key] + nbytes].cpu().numpy().view(dtype)


def _code_rows_dev(ws, lay, key, rows, row_bytes):
    """Rows of an activation code buffer (x_codes, h_codes) as a device view:
    row_bytes bytes per row at a stride of whole 128-byte lines."""
    ld = -(-row_bytes // 128) * 128
    return ws[lay[key]:lay[key] + rows * ld].view(rows, ld)[:, :row_bytes]


def _code_rows(ws, lay, key, rows, row_bytes):
    return _code_rows_dev(ws, lay, key, rows, row_bytes).cpu().numpy()


def _status(ws, lay):
    return _ws_view(ws, lay, "status", np.int32, 16)


def _f32(bits):
    return float(np.array([bits], dtype=np.int32).view(np.float32)[0])


# ---------------------------------------------------------------- routing ----


@pytest.mark.parametrize("T,E,k", [(1, 128, 4), (7, 128, 4), (300, 128, 4), (33, 64, 1),
                                   (65, 200, 8), (17, 512, 16), (5, 3, 3)])
def test_route_topk_bit_exact(mx, T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    ids, w = mx.mxfp4_route_topk(to_dev(logits, torch), k)
    ref_ids, ref_w = oracle.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


def test_route_topk_ties_and_signed_zero(mx):
    rng = np.random.default_rng(3)
    logits = rng.integers(-2, 3, size=(257, 128)).astype(np.float32)
    logits[0] = 0.0
    logits[1, ::3] = -0.0
    logits[2] = -np.inf
    logits[2, 77] = 1.0
    ids, w = mx.mxfp4_route_topk(to_dev(logits, torch), 4)
    ref_ids, ref_w = oracle.route_topk(logits, 4)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("name", list(synth.MOE_WORKLOADS))
def test_route_topk_workloads(mx, name):
    wl = synth.workload(name)
    ids, w = mx.mxfp4_route_topk(to_dev(wl["logits"], torch), synth.TOPK_GPT_OSS)
    ref_ids, ref_w = oracle.route_topk(wl["logits"], synth.TOPK_GPT_OSS)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


# ---------------------------------------------------------------- fp8 codec ----


@pytest.mark.parametrize("top", [-100, -10, 0, 3, 20, 100])
def test_quant_fp8_exhaustive_bf16(mx, top):
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (bits << 16).view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) < np.float32(2.0 ** top))
    vb = (bits[keep]).astype(np.uint16)
    codes, scale, amax = mx.mxfp4_quant_fp8_e4m3(to_dev(vb, torch))
    rc, rs, ra = oracle.quant_per_tensor(bf16_bits_to_f64(vb))
    assert float(amax.item()) == ra
    assert float(scale.item()) == rs
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("n", [0, 1, 17, 4096, 1000003])
def test_quant_fp8_fp32_ragged(mx, n):
    rng = np.random.default_rng(n)
    v = (rng.standard_cauchy(n) * 3).astype(np.float32)
    codes, scale, amax = mx.mxfp4_quant_fp8_e4m3(to_dev(v, torch))
    rc, rs, ra = oracle.quant_per_tensor(v.astype(np.float64))
    assert float(amax.item()) == ra and float(scale.item()) == rs
    assert np.array_equal(codes.cpu().numpy(), rc)


# -------------------------------------------------------------- permutation ----


@pytest.mark.parametrize("T,E,k,hot", [(25, 16, 4, 0), (1024, 16, 4, 0), (1025, 16, 4, 3),
                                       (5000, 64, 4, 5), (333, 16, 1, 0)])
def test_permutation_bit_exact(mx, T, E, k, hot):
    H = I = 64
    L = synth.layer(seed=5, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(6, T, E=E, H=H, hot=hot)
    ids, w = oracle.route_topk(logits, k)
    for act in (synth.ACT_BF16, synth.ACT_FP8_E4M3):
        got, ws, lay = _run_moe(mx, _layer_dev(L), x, ids, w, act, want_ws=True)
        counts, offsets, sp, inv = oracle.permute(ids, E)
        np_ = T * k
        assert np.array_equal(_ws_view(ws, lay, "expert_offsets", np.int32, E + 1), offsets)
        assert np.array_equal(_ws_view(ws, lay, "sorted_pairs", np.int32, np_), sp)
        assert np.array_equal(_ws_view(ws, lay, "inv_pairs", np.int32, np_), inv)
        bm = 4 if act == synth.ACT_BF16 else 128
        assert _status(ws, lay)[5] == int(np.sum((counts + bm - 1) // bm))
        assert _status(ws, lay)[0] == 0
        # row-tile list: (expert, first row, end row, w) per BM rows of each expert in
        # expert order, w = (index of the expert's first entry) | (its entry count << 16),
        # then expert -1 up to the workspace's bound on the tile count
        ntile = (counts + bm - 1) // bm
        first = np.concatenate([[0], np.cumsum(ntile)[:-1]])
        bound = np_ // bm + min(np_, E) + 1
        assert bound <= 32768
        want = [(e, offsets[e] + b, min(offsets[e] + b + bm, offsets[e + 1]),
                 int(first[e]) | (int(ntile[e]) << 16))
                for e in range(E) for b in range(0, int(counts[e]), bm)]
        want += [(-1, 0, 0, 0)] * (bound - len(want))
        got_tiles = _ws_view(ws, lay, "tiles", np.int32, 4 * bound).reshape(bound, 4)
        assert np.array_equal(got_tiles, np.array(want, dtype=np.int32))


@pytest.mark.parametrize("act", [synth.ACT_BF16, synth.ACT_FP8_E4M3])
def test_multiblock_permutation_bad_ids_and_status_reuse(mx, act):
    # 4400 pairs: the multi-block permutation.  Ids outside [0, E) are skipped
    # and flagged; a second call on the same workspace with clean ids and x
    # halved (a smaller FP8 amax) must start from cleared status words.
    E, H, I, T, k = 16, 64, 64, 1100, 4
    L = synth.layer(seed=41, E=E, H=H, I=I)
    Ld = _layer_dev(L)
    logits, x = synth.moe_inputs(42, T, E=E, H=H, hot=2)
    ids, w = oracle.route_topk(logits, k)
    ids_bad = ids.copy()
    ids_bad[0, 1] = -1
    ids_bad[700, 3] = E + 2
    ids_bad[1099, 0] = -7
    ws = torch.zeros(mx.mxfp4_moe_workspace_size(T, H, I, E, k, act), dtype=torch.uint8, device="cuda")
    lay = mx.mxfp4_moe_workspace_layout_query(T, H, I, E, k, act)

    def call(xb, idb):
        out = mx.mxfp4_moe_forward(to_dev(xb, torch), to_dev(idb.astype(np.int32), torch),
                                   to_dev(w.astype(np.float32), torch), Ld["w13_blocks"], Ld["w13_scales"],
                                   Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], act,
                                   workspace=ws)
        torch.cuda.synchronize()
        return bf16_dev_to_f64(out)

    got = call(x, ids_bad)
    assert _status(ws, lay)[0] & 1
    flat = ids_bad.reshape(-1).astype(np.int64)
    keep = np.nonzero((flat >= 0) & (flat < E))[0]
    _, offsets, sp, inv_kept = oracle.permute(flat[keep].reshape(-1, 1), E)
    want_inv = np.full(T * k, -1, dtype=np.int64)
    want_inv[keep] = inv_kept
    assert np.array_equal(_ws_view(ws, lay, "expert_offsets", np.int32, E + 1), offsets)
    assert np.array_equal(_ws_view(ws, lay, "sorted_pairs", np.int32, keep.size), keep[sp])
    assert np.array_equal(_ws_view(ws, lay, "inv_pairs", np.int32, T * k), want_inv)
    assert_close_rounded(got, oracle.moe_forward_routed(x, ids_bad, w, **L, act_mode=act)["out"], "bad ids")

    # x / 2 exactly (bf16 exponent field minus one; no zeros or subnormals here)
    assert np.all((x & 0x7f80) > 0x80)
    x2 = (x - 0x80).astype(np.uint16)
    got = call(x2, ids)
    assert _status(ws, lay)[0] == 0
    assert_close_rounded(got, oracle.moe_forward_routed(x2, ids, w, **L, act_mode=act)["out"], "reused workspace")


# ------------------------------------------------------------ small layers ----

SMALL = [  # E, H, I, T, k   (H/32 and I/32 give every K tail modulo 4)
    (8, 288, 320, 1, 4),
    (8, 288, 320, 5, 4),
    (8, 288, 320, 37, 4),
    (16, 96, 128, 300, 4),
    (4, 224, 64, 70, 2),
    (1, 64, 96, 9, 1),
    (8, 288, 320, 120, 4),
]


@pytest.mark.parametrize("E,H,I,T,k", SMALL)
@pytest.mark.parametrize("act", [synth.ACT_BF16, synth.ACT_FP8_E4M3])
def test_moe_small_layers(mx, E, H, I, T, k, act):
    L = synth.layer(seed=E * 7 + H, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 11, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    got, ws, lay = _run_moe(mx, _layer_dev(L), x, ids, w, act, want_ws=True)
    ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=act)
    assert_close_rounded(got, ref["out"], "E%d H%d I%d T%d act%d" % (E, H, I, T, act))
    np_ = T * k
    st = _status(ws, lay)
    inv = _ws_view(ws, lay, "inv_pairs", np.int32, np_)
    if act == synth.ACT_FP8_E4M3:
        # x codes are stored in expert-sorted row order: row r is token sp[r] // k
        sp = _ws_view(ws, lay, "sorted_pairs", np.int32, np_)
        nrows = int(_ws_view(ws, lay, "expert_offsets", np.int32, E + 1)[E])
        xc = _code_rows(ws, lay, "x_codes", np_, H)[:nrows]
        assert np.array_equal(xc, ref["x_codes"][sp[:nrows] // k])
        assert _f32(st[3]) == ref["x_scale"]
        h_gpu = _ws_view(ws, lay, "h", np.float32, np_ * I).reshape(np_, I)
        hc_gpu = _code_rows(ws, lay, "h_codes", np_, I)
        # the GPU's codes of h are the oracle codec applied to the GPU's own fp32 h
        rc, rs, ra = oracle.quant_per_tensor(h_gpu.astype(np.float64))
        assert _f32(st[2]) == ra and _f32(st[4]) == rs
        assert np.array_equal(hc_gpu, rc)
        # and h itself matches the oracle's h (sorted rows back to (t, j))
        h_ref = ref["h"].reshape(np_, I)
        rf, _, _ = errors(h_gpu[inv], h_ref)
        assert rf < 1e-4
    else:
        hh = _ws_view(ws, lay, "h", np.uint16, 2 * np_ * I)
        h_gpu = bf16_bits_to_f64(hh[:np_ * I]) + bf16_bits_to_f64(hh[np_ * I:])
        rf, _, _ = errors(h_gpu.reshape(np_, I)[inv], ref["h"].reshape(np_, I))
        assert rf < 1e-5
        # bf16 outputs are the oracle rounded once, up to rare one-ulp flips
        ref_bits = synth.f32_to_bf16_bits(ref["out"].astype(np.float32))
        assert np.mean(got != bf16_bits_to_f64(ref_bits)) < 0.02


def test_moe_edge_cases(mx):
    E, H, I, T, k = 8, 64, 96, 40, 4
    L = synth.layer(seed=77, E=E, H=H, I=I)
    Ld = _layer_dev(L)
    logits, x = synth.moe_inputs(78, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    for act in (synth.ACT_BF16, synth.ACT_FP8_E4M3):
        # every token on the same four experts (one expert spans several tiles)
        ids_hot = np.tile(np.arange(k, dtype=np.int32), (T, 1))
        got = _run_moe(mx, Ld, x, ids_hot, w, act)
        assert_close_rounded(got, oracle.moe_forward_routed(x, ids_hot, w, **L, act_mode=act)["out"], "hot")
        # duplicated expert inside a token, and ids out of range (skipped, flagged)
        ids_bad = ids.copy()
        ids_bad[0, 1] = ids_bad[0, 0]
        ids_bad[3, 2] = -1
        ids_bad[5, 0] = E + 5
        got, ws, lay = _run_moe(mx, Ld, x, ids_bad, w, act, want_ws=True)
        assert _status(ws, lay)[0] & 1
        assert_close_rounded(got, oracle.moe_forward_routed(x, ids_bad, w, **L, act_mode=act)["out"], "bad ids")
        # all-zero activations: outputs come from the biases alone
        x0 = np.zeros_like(x)
        got = _run_moe(mx, Ld, x0, ids, w, act)
        assert_close_rounded(got, oracle.moe_forward_routed(x0, ids, w, **L, act_mode=act)["out"], "zero x")
        # no bias
        Lnb = dict(L, w13_bias=None, w2_bias=None)
        Ldnb = dict(Ld, w13_bias=None, w2_bias=None)
        got = _run_moe(mx, Ldnb, x, ids, w, act)
        assert_close_rounded(got, oracle.moe_forward_routed(x, ids, w, **Lnb, act_mode=act)["out"], "no bias")


def test_moe_wide_scales(mx):
    E, H, I, T, k = 4, 128, 64, 16, 2
    rng = np.random.default_rng(91)
    L = synth.layer(seed=90, E=E, H=H, I=I)
    L["w13_scales"] = rng.integers(100, 155, size=L["w13_scales"].shape, dtype=np.uint8)
    L["w2_scales"] = rng.integers(100, 155, size=L["w2_scales"].shape, dtype=np.uint8)
    logits, x = synth.moe_inputs(92, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    for act in (synth.ACT_BF16, synth.ACT_FP8_E4M3):
        got = _run_moe(mx, _layer_dev(L), x, ids, w, act)
        assert_close_rounded(got, oracle.moe_forward_routed(x, ids, w, **L, act_mode=act)["out"], "scales")


def test_moe_zero_tokens_is_noop(mx):
    L = synth.layer(seed=1, E=4, H=64, I=64)
    Ld = _layer_dev(L)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    w = torch.zeros((0, 2), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_moe_forward(x, ids, w, Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"],
                         Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], 0, out=out,
                         workspace=torch.zeros(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()


def test_moe_deterministic(mx):
    E, H, I, T, k = 16, 96, 128, 300, 4
    L = synth.layer(seed=3, E=E, H=H, I=I)
    Ld = _layer_dev(L)
    logits, x = synth.moe_inputs(4, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    for act in (synth.ACT_BF16, synth.ACT_FP8_E4M3):
        a = _run_moe(mx, Ld, x, ids, w, act)
        b = _run_moe(mx, Ld, x, ids, w, act)
        assert np.array_equal(a, b)


# ------------------------------------------------------------------ dense ----


@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (4, 48, 96), (17, 1040, 288), (33, 64, 4096),
                                   (3, 5120, 2880), (1, 2880, 4096)])
def test_linear_small_and_projection_shapes(mx, M, N, K):
    D = synth.dense(M * 31 + N, N, K)
    x = synth.dense_x(M + K, M, K)
    out = mx.mxfp4_linear(to_dev(x, torch), to_dev(D["w_blocks"], torch), to_dev(D["w_scales"], torch),
                          to_dev(D["bias"], torch))
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)
    ref = oracle.linear(x, D["w_blocks"], D["w_scales"], D["bias"])
    assert_close_rounded(got, ref, "linear %dx%dx%d" % (M, N, K))
    no_constant_rows(got)


@pytest.mark.parametrize("name", ["qkv_proj", "o_proj", "lm_head"])
@pytest.mark.parametrize("M", [1, 4])
def test_linear_dense_set_full_size(mx, name, M):
    N, K = synth.DENSE_SHAPES[name]
    D = synth.dense(synth.DENSE_SEEDS[name], N, K)
    x = synth.dense_x(synth.DENSE_X_SEED, M, K)
    out = mx.mxfp4_linear(to_dev(x, torch), to_dev(D["w_blocks"], torch), to_dev(D["w_scales"], torch),
                          to_dev(D["bias"], torch))
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)
    if N > 8192:   # lm_head: sampled rows, including both ends
        rng = np.random.default_rng(5)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                         rng.choice(N, 2048, replace=False)]))
        ref = oracle.linear_rows(x, D["w_blocks"], D["w_scales"], D["bias"], rows)
        got_s = got[:, rows]
    else:
        ref = oracle.linear(x, D["w_blocks"], D["w_scales"], D["bias"])
        got_s = got
    assert_close(got_s, ref, name)
    no_constant_rows(got)


def test_linear_no_bias_zero_rows(mx):
    D = synth.dense(8, 64, 64)
    x = synth.dense_x(9, 5, 64)
    out = mx.mxfp4_linear(to_dev(x, torch), to_dev(D["w_blocks"], torch), to_dev(D["w_scales"], torch))
    torch.cuda.synchronize()
    assert_close_rounded(bf16_dev_to_f64(out), oracle.linear(x, D["w_blocks"], D["w_scales"]), "no bias")
    empty = mx.mxfp4_linear(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"),
                            to_dev(D["w_blocks"], torch), to_dev(D["w_scales"], torch))
    assert empty.shape == (0, 64)


# ------------------------------------------------- full-size MoE workloads ----


@pytest.fixture(scope="module")
def full_layer():
    L = synth.layer()
    return L, _layer_dev(L)


def _w2_of(L):
    return lambda e: oracle.dequant(L["w2_blocks"][e], L["w2_scales"][e])


def _b2_of(L, H):
    if L["w2_bias"] is None:
        return lambda e: np.zeros(H)
    return lambda e: oracle.bf16_bits_to_f64(L["w2_bias"][e])


def _codes_and_outputs(got_tok, ref_tok, delta, ndiff, hq, pairs, ids, w_gpu, w_ref, tokens, L, what):
    """Shared tail of the quantised-mode checks for the pairs of `tokens`:
    the down projection and combine of the kernel's own h codes (hq, float64)
    against the kernel's output under the plain bar, the allowance of the
    differing codes below SLACK_MAX, and the output against the float64
    layer beyond that allowance (plain bar when no code differs)."""
    k = ids.shape[1]
    H = got_tok.shape[1]
    tok, exp = pairs // k, ids.reshape(-1)[pairs]
    own = down_combine(hq, tok, exp, w_gpu.reshape(-1)[pairs], tokens, _w2_of(L), _b2_of(L, H))
    assert_close_rounded(got_tok, own, what + " (own h codes)")
    slack = mismatch_slack(delta, tok, exp, w_ref.reshape(-1)[pairs], tokens, _w2_of(L))
    ratio = 0.0 if slack is None else np.linalg.norm(slack) / np.linalg.norm(ref_tok)
    rel, mabs, rms = errors(got_tok, ref_tok)
    print("%s: %d of %d h codes differ, |slack|/|out| %.2e, rel Frobenius %.3e, max abs %.3e rms"
          % (what, ndiff, hq.size, ratio, rel, mabs / rms))
    assert ndiff <= DIFF_MAX * hq.size, "%s: %d h codes differ" % (what, ndiff)
    assert ratio <= SLACK_MAX, "%s: allowance of the differing h codes %.2e" % (what, ratio)
    if slack is None:
        assert_close(got_tok, ref_tok, what)
    else:
        assert_close_slack(got_tok, ref_tok, slack, what)


@pytest.mark.parametrize("name", list(synth.MOE_WORKLOADS))
def test_moe_full_size_workloads(mx, full_layer, name):
    path = os.path.join(GOLDEN, "%s.npz" % name)
    gold = np.load(path)
    L, Ld = full_layer
    wl = synth.workload(name)
    act = wl["act_mode"]
    ids_d, w_d = mx.mxfp4_route_topk(to_dev(wl["logits"], torch), synth.TOPK_GPT_OSS)
    ref_ids, ref_w = oracle.route_topk(wl["logits"], synth.TOPK_GPT_OSS)
    assert np.array_equal(ids_d.cpu().numpy(), ref_ids)
    T, H = wl["x"].shape
    I = synth.H_GPT_OSS
    E = synth.E_GPT_OSS
    k = synth.TOPK_GPT_OSS
    ws_bytes = mx.mxfp4_moe_workspace_size(T, H, I, E, k, act)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    out = mx.mxfp4_moe_forward(to_dev(wl["x"], torch), ids_d, w_d, Ld["w13_blocks"], Ld["w13_scales"],
                               Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], act,
                               workspace=ws)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)
    tokens = gold["tokens"]
    ref = gold["out"].astype(np.float64)
    no_constant_rows(got)
    lay = mx.mxfp4_moe_workspace_layout_query(T, H, I, E, k, act)
    st = _status(ws, lay)
    assert st[0] == 0
    if act == synth.ACT_BF16:
        assert_close(got[tokens], ref, name)
        return
    np_ = T * k
    sp = _ws_view(ws, lay, "sorted_pairs", np.int32, np_).astype(np.int64)
    inv = _ws_view(ws, lay, "inv_pairs", np.int32, np_)
    pairs = gold["pairs"]
    rows_np = inv[pairs].astype(np.int64)
    rows = torch.from_numpy(rows_np).cuda()
    h_ref = gold["h_ref"].astype(np.float64)
    tol = gold["h_tol"].astype(np.float64)
    if act == synth.ACT_FP8_E4M3:
        xc_ref, sx, _ = oracle.quant_per_tensor(oracle.bf16_bits_to_f64(wl["x"]))
        assert _f32(st[3]) == sx == float(gold["x_scale"])
        xc = _code_rows(ws, lay, "x_codes", np_, H)
        assert np.array_equal(xc, xc_ref[sp // k])          # every pair routed
        h_t = ws[lay["h"]:lay["h"] + np_ * I * 4].view(torch.float32).view(np_, I)
        # the kernel's fp32 h within the error bound, on every pair of the sampled tokens
        h_gpu = h_t[rows].cpu().numpy().astype(np.float64)
        err = np.abs(h_gpu - h_ref)
        worst = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
        assert np.all(err <= tol), "%s: h beyond the error bound (worst %.2f of it: h %r, kernel %r, bound %r)" % (
            name, float(err[worst] / max(tol[worst], 1e-300)), h_ref[worst], h_gpu[worst], tol[worst])
        print("%s: kernel h error at most %.3f of its bound" % (name, float(np.max(err / np.maximum(tol, 1e-300)))))
        # amax and scale from the GPU's own fp32 h, codes on a sample of rows
        amax = float(h_t.abs().max().item())
        assert _f32(st[2]) == amax
        assert _f32(st[4]) == oracle.fp8.f32_scale(amax)
        assert abs(amax - float(gold["h_amax"])) <= 1e-5 * float(gold["h_amax"])
        srows = np.random.default_rng(1).choice(np_, 512, replace=False)
        h_rows = h_t[torch.from_numpy(srows).cuda()].cpu().numpy().astype(np.float64)
        sh = _f32(st[4])
        rc = oracle.e4m3_encode((h_rows / sh).astype(np.float32).astype(np.float64))
        hc_all = _code_rows_dev(ws, lay, "h_codes", np_, I)
        assert np.array_equal(hc_all[torch.from_numpy(srows).cuda()].cpu().numpy(), rc)
        # codes of every pair of the sampled tokens against the oracle's codes
        c_gpu = hc_all[rows].cpu().numpy()
        delta, ndiff = fp8_code_mismatch(c_gpu, sh, h_ref, tol, float(gold["h_scale"]))
        hq = oracle.e4m3_decode(c_gpu) * sh
    else:
        # x codes of every sorted row (every pair is routed)
        xb = _code_rows(ws, lay, "x_codes", np_, H // 2).reshape(np_, H // 32, 16)
        xs = _step_major(ws, lay, "x_scales", np_, H)
        rb, rs = oracle.quantize_mxfp4(oracle.bf16_bits_to_f64(wl["x"]))
        assert np.array_equal(xs[:, :H // 32], rs[sp // k])
        assert np.array_equal(xb, rb[sp // k])
        del xb, rb
        # h codes of every pair of the sampled tokens against the oracle's
        hb = _code_rows_dev(ws, lay, "h_codes", np_, I // 2).reshape(np_, I // 32, 16)
        hb = hb[rows].cpu().numpy()
        hs = _step_major(ws, lay, "h_scales", np_, I)[rows_np][:, :I // 32]
        delta, ndiff = mx_code_mismatch(hb, hs, h_ref, tol)
        hq = oracle.dequant(hb, hs)
    _codes_and_outputs(got[tokens], ref, delta, ndiff, hq, pairs, ref_ids, w_d.cpu().numpy(), ref_w,
                       tokens, L, name)


@pytest.mark.parametrize("act", [synth.ACT_FP8_E4M3, synth.ACT_MXFP4])
def test_moe_multi_unit_layers(mx, act):
    """gpt-oss expert shapes (H = I = 2880) with 8 experts and 1400 tokens:
    700 rows per expert, so each prefill block takes more than one unit (gate_up
    1104 units, down 576, over 256 blocks).  Every h code, every output, and
    the down projection of the kernel's own codes are checked."""
    E, H, I, T, k = 8, 2880, 2880, 1400, 4
    L = synth.layer(seed=61, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(62, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    got, ws, lay = _run_moe(mx, _layer_dev(L), x, ids, w, act, want_ws=True)
    ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=act)
    np_ = T * k
    inv = _ws_view(ws, lay, "inv_pairs", np.int32, np_).astype(np.int64)
    pairs = np.arange(np_)
    h_ref = ref["h32"].reshape(np_, I)
    tol = pair_h_tolerance(activations(ref, x, act), ids, L, pairs, k)
    if act == synth.ACT_FP8_E4M3:
        h_gpu = _ws_view(ws, lay, "h", np.float32, np_ * I).reshape(np_, I)[inv].astype(np.float64)
        assert np.all(np.abs(h_gpu - h_ref) <= tol)
        sh = _f32(_status(ws, lay)[4])
        c_gpu = _code_rows(ws, lay, "h_codes", np_, I)[inv]
        delta, ndiff = fp8_code_mismatch(c_gpu, sh, h_ref, tol, ref["h_scale"])
        hq = oracle.e4m3_decode(c_gpu) * sh
    else:
        hb = _code_rows(ws, lay, "h_codes", np_, I // 2).reshape(np_, I // 32, 16)[inv]
        hs = _step_major(ws, lay, "h_scales", np_, I)[inv][:, :I // 32]
        delta, ndiff = mx_code_mismatch(hb, hs, h_ref, tol)
        hq = oracle.dequant(hb, hs)
    _codes_and_outputs(got, ref["out"], delta, ndiff, hq, pairs, ids, w.astype(np.float32), w,
                       np.arange(T), L, "multi-unit act%d" % act)


# ------------------------------------- MXFP4 activations (FP4 x FP4 MFMA) ----


def _step_major(ws, lay, key, rows, K):
    """MXFP4 activation scales from the workspace's step-major layout
    [ceil(K/128), rows, 4] as [rows, 4*ceil(K/128)] (blocks past K/32 are pad)."""
    ns = -(-K // 128)
    a = _ws_view(ws, lay, key, np.uint8, ns * rows * 4).reshape(ns, rows, 4)
    return a.transpose(1, 0, 2).reshape(rows, ns * 4)


def _mx_act_check(mx, L, x, ids, w, what):
    """The FP4 x FP4 layer against the oracle, step by step.

    The x codes are unique and compared bit for bit.  The h codes (quantised
    in the gate_up epilogue; no fp32 h is kept) are compared with the oracle
    quantiser of the oracle's h: a code may differ only where an h within the
    kernel's error bound rounds to it.  The output is compared with the
    oracle's down projection and combine of the kernel's own h codes, and end
    to end beyond the change the differing codes make.  Returns the relative
    error against the float64 layer."""
    E = L["w13_blocks"].shape[0]
    T, H = x.shape
    I = L["w2_blocks"].shape[2] * 32
    k = ids.shape[1]
    np_ = T * k
    got, ws, lay = _run_moe(mx, _layer_dev(L), x, ids, w, synth.ACT_MXFP4, want_ws=True)
    ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=synth.ACT_MXFP4)
    sp = _ws_view(ws, lay, "sorted_pairs", np.int32, np_)
    nrows = int(_ws_view(ws, lay, "expert_offsets", np.int32, E + 1)[E])
    pairs = sp[:nrows].astype(np.int64)
    xb = _code_rows(ws, lay, "x_codes", np_, H // 2).reshape(np_, H // 32, 16)[:nrows]
    xs = _step_major(ws, lay, "x_scales", np_, H)[:nrows]
    assert np.array_equal(xb, ref["x_blocks"][pairs // k])
    assert np.array_equal(xs[:, :H // 32], ref["x_scales"][pairs // k])
    assert np.all(xs[:, H // 32:] == 127)
    hb = _code_rows(ws, lay, "h_codes", np_, I // 2).reshape(np_, I // 32, 16)[:nrows]
    hs = _step_major(ws, lay, "h_scales", np_, I)[:nrows]
    assert np.all(hs[:, I // 32:] == 127)
    hs = hs[:, :I // 32]
    tol = pair_h_tolerance(activations(ref, x, synth.ACT_MXFP4), ids, L, pairs, k)
    delta, ndiff = mx_code_mismatch(hb, hs, ref["h32"].reshape(np_, I)[pairs], tol)
    # y = W2 h' + b2 of the kernel's h codes and the weighted combine, float64
    hq = oracle.dequant(hb, hs)
    tok, exp = pairs // k, ids.reshape(-1).astype(np.int64)[pairs]
    wf = w.reshape(-1)[pairs]
    tokens = np.arange(T)
    out_ref = down_combine(hq, tok, exp, wf, tokens, _w2_of(L), _b2_of(L, H)) if nrows else np.zeros((T, H))
    assert_close_rounded(got, out_ref, what)
    # end to end against the float64 layer, beyond the change the differing
    # h codes make
    slack = mismatch_slack(delta, tok, exp, wf, tokens, _w2_of(L))
    if slack is None:
        assert_close_rounded(got, ref["out"], what + " end to end")
    else:
        assert_close_rounded_slack(got, ref["out"], slack, what + " end to end")
    end = errors(got, ref["out"])[0]
    print("%s: end-to-end rel %.3e, %d h codes differ" % (what, end, ndiff))
    return end


def _expected_stream(scales, nout, gateup):
    """The restaged scale stream from its definition: for expert e, n-tile nt,
    K step s and LDS row lr of the unit, the scales of blocks 4s .. 4s+3 of
    the weight row the unit holds in that LDS row (127 past K, and for LDS
    rows past the last weight row)."""
    E, R, nb = scales.shape
    bn = 128 if gateup else 256
    NT, ns = -(-nout // bn), -(-nb // 4)
    lr = np.arange(256)
    out = np.full((E, NT, ns, 256, 4), 127, dtype=np.uint8)
    for nt in range(NT):
        idx = nt * 128 + (lr & 127) if gateup else nt * 256 + lr
        real = idx < nout
        rows = (np.where(lr < 128, 0, nout) if gateup else 0) + np.minimum(idx, nout - 1)
        for s4 in range(ns):
            for j in range(4):
                b = 4 * s4 + j
                if b < nb:
                    out[:, nt, s4, real, j] = scales[:, rows[real], b]
    return out.reshape(-1)


@pytest.mark.parametrize("act", [synth.ACT_FP8_E4M3, synth.ACT_MXFP4])
@pytest.mark.parametrize("E,H,I", [(8, 288, 320), (4, 224, 96), (2, 544, 384), (2, 1056, 1024), (3, 2880, 2880),
                                   (2, 3200, 3328)])
def test_prefill_scale_streams(mx, E, H, I, act):
    L = synth.layer(seed=E + H + I, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(5, 20, E=E, H=H)
    ids, w = oracle.route_topk(logits, 2)
    _, ws, lay = _run_moe(mx, _layer_dev(L), x, ids, w, act, want_ws=True)
    want13 = _expected_stream(L["w13_scales"], I, True)
    want2 = _expected_stream(L["w2_scales"], H, False)
    assert np.array_equal(_ws_view(ws, lay, "w13_scale_stream", np.uint8, want13.size), want13)
    assert np.array_equal(_ws_view(ws, lay, "w2_scale_stream", np.uint8, want2.size), want2)


@pytest.mark.parametrize("act", [synth.ACT_FP8_E4M3, synth.ACT_MXFP4])
def test_scale_streams_ready_reuses_the_workspace(mx, act):
    E, H, I, T, k = 8, 288, 320, 40, 4
    L = synth.layer(seed=91, E=E, H=H, I=I)
    Ld = _layer_dev(L)
    logits, x = synth.moe_inputs(92, T, E=E, H=H)
    xd, ld = to_dev(x, torch), to_dev(logits, torch)
    ws = torch.zeros(mx.mxfp4_moe_workspace_size(T, H, I, E, k, act), dtype=torch.uint8, device="cuda")
    lay = mx.mxfp4_moe_workspace_layout_query(T, H, I, E, k, act)

    def run(ready):
        out = mx.mxfp4_moe_layer(xd, ld, k, Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"], Ld["w2_blocks"],
                                 Ld["w2_scales"], Ld["w2_bias"], act, workspace=ws, scale_streams_ready=ready)[0]
        torch.cuda.synchronize()
        return out.clone()

    first = run(False)
    assert torch.equal(run(True), first)           # the streams left by the first call
    # the flag does skip the restaging: with the streams cleared the result changes
    ws[lay["w13_scale_stream"]:lay["total_bytes"]] = 0
    assert not torch.equal(run(True), first)
    assert torch.equal(run(False), first)          # and a normal call restages them again


@pytest.mark.parametrize("act", [synth.ACT_FP8_E4M3, synth.ACT_MXFP4])
def test_prefill_long_k(mx, act):
    # K = 3200 and 3328 (more than 3072: the scale restage's generic path),
    # 25 and 26 K steps with ragged last steps
    E, H, I, T, k = 2, 3200, 3328, 6, 2
    L = synth.layer(seed=97, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(98, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    if act == synth.ACT_MXFP4:
        _mx_act_check(mx, L, x, ids, w, "long K mxfp4-act")
    else:
        got = _run_moe(mx, _layer_dev(L), x, ids, w, act)
        ref = oracle.moe_forward_routed(x, ids, w, **L, act_mode=act)
        assert_close_rounded(got, ref["out"], "long K fp8")


# MXFP4 activations run K steps of 256 (eight MX blocks): H/32 and I/32 here
# add the tails 5 and 6 modulo 8 and multi-step tails 3, 5, 6, 7 and 0
SMALL_A4 = SMALL + [
    (4, 416, 352, 19, 2),
    (4, 448, 480, 23, 4),
    (4, 512, 160, 7, 2),
    (2, 192, 768, 5, 1),
]


@pytest.mark.parametrize("E,H,I,T,k", SMALL_A4)
def test_mxfp4_act_small_layers(mx, E, H, I, T, k):
    L = synth.layer(seed=E * 13 + H, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 17, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    _mx_act_check(mx, L, x, ids, w, "mxfp4-act E%d H%d I%d T%d" % (E, H, I, T))


def test_mxfp4_act_edge_cases(mx):
    E, H, I, T, k = 8, 64, 96, 40, 4
    L = synth.layer(seed=79, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(80, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    # every token on the same four experts (one expert spans several tiles)
    _mx_act_check(mx, L, x, np.tile(np.arange(k, dtype=np.int32), (T, 1)), w, "hot")
    # duplicated expert inside a token, ids out of range (skipped)
    ids_bad = ids.copy()
    ids_bad[0, 1] = ids_bad[0, 0]
    ids_bad[3, 2] = -1
    ids_bad[5, 0] = E + 5
    _mx_act_check(mx, L, x, ids_bad, w, "bad ids")
    # all-zero activations (every block gets the smallest scale) and no bias
    _mx_act_check(mx, L, np.zeros_like(x), ids, w, "zero x")
    _mx_act_check(mx, dict(L, w13_bias=None, w2_bias=None), x, ids, w, "no bias")
    # a wide spread of magnitudes inside the blocks of x
    xw = synth.f32_to_bf16_bits(oracle.bf16_bits_to_f64(x) * np.exp2(np.random.default_rng(81).integers(
        -20, 20, size=x.shape)))
    _mx_act_check(mx, L, xw, ids, w, "wide x")


# ------------------------------------------------------ weight quantiser ----


def _quant_ref(w_bits):
    return oracle.quantize_mxfp4(bf16_bits_to_f64(w_bits))


def _quant_gpu(mx, w_bits):
    b, s = mx.mxfp4_quantize_weights(to_dev(w_bits, torch))
    torch.cuda.synchronize()
    return b.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("N,K", [(1, 32), (37, 320), (64, 2880), (5, 4096)])
def test_quantize_weights_bit_exact(mx, N, K):
    w = synth.dense_bf16_weights(40 + N, N, K)
    b, s = _quant_gpu(mx, w)
    rb, rs = _quant_ref(w)
    assert np.array_equal(s, rs)
    assert np.array_equal(b, rb)


def test_quantize_weights_ties_signs_and_extremes(mx):
    # rows: exact rounding ties under scale 2^0 (block max 6), zeros and -0,
    # bf16 subnormals, the largest finite bf16, and values just past ties
    rows = []
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    rows.append((ties + [-t for t in ties]) * 2)
    rows.append([0.0] * 16 + [-0.0] * 16)
    rows.append([2.0 ** -133 * (i + 1) for i in range(32)])
    rows.append([3.3895e38 * (1 - 2 * (i % 2)) for i in range(32)])
    rows.append([(t + 2.0 ** -6) for t in ties] * 4)
    rows.append([7.99, 7.0, -6.5] + [0.0] * 29)
    w = synth.f32_to_bf16_bits(np.array(rows, dtype=np.float32))
    b, s = _quant_gpu(mx, w)
    rb, rs = _quant_ref(w)
    assert np.array_equal(s, rs)
    assert np.array_equal(b, rb)


def test_quantize_weights_full_lm_head_sampled(mx):
    # the 201,088 x 2880 lm_head quantised at once; rows sampled for the oracle
    N, K = synth.DENSE_SHAPES["lm_head"]
    w = synth.dense_bf16_weights(50, N, K)
    b, s = _quant_gpu(mx, w)
    rows = np.random.default_rng(51).choice(N, 512, replace=False)
    rows = np.concatenate([rows, [0, N - 1]])
    rb, rs = _quant_ref(w[rows])
    assert np.array_equal(s[rows], rs)
    assert np.array_equal(b[rows], rb)


def test_quantized_weights_feed_the_linear(mx):
    # quantise on the GPU, run the dense projection on the result, compare with
    # the oracle's linear on the oracle's quantisation of the same weights
    N, K, M = 1040, 2880, 4
    w = synth.dense_bf16_weights(52, N, K)
    b, s = mx.mxfp4_quantize_weights(to_dev(w, torch))
    x = synth.dense_x(53, M, K)
    out = mx.mxfp4_linear(to_dev(x, torch), b, s)
    torch.cuda.synchronize()
    rb, rs = _quant_ref(w)
    ref = oracle.linear(x, rb, rs, None)
    assert_close_rounded(bf16_dev_to_f64(out), ref, "quantise -> linear")


# ------------------------------------------------- router + layer in one call ----


@pytest.mark.parametrize("E,H,I,T,k,act", [(8, 288, 320, 37, 4, synth.ACT_BF16),
                                           (8, 288, 320, 37, 4, synth.ACT_FP8_E4M3),
                                           (128, 256, 128, 1025, 4, synth.ACT_BF16),
                                           (128, 256, 128, 64, 4, synth.ACT_BF16),
                                           (128, 256, 128, 65, 4, synth.ACT_BF16),
                                           (512, 64, 64, 64, 4, synth.ACT_BF16),
                                           (16, 96, 128, 300, 2, synth.ACT_FP8_E4M3),
                                           # up to 16 tokens route and permute in one launch
                                           (128, 256, 128, 4, 4, synth.ACT_BF16),
                                           (8, 288, 320, 16, 4, synth.ACT_FP8_E4M3),
                                           (512, 64, 64, 1, 4, synth.ACT_BF16),
                                           (48, 96, 128, 9, 2, synth.ACT_BF16),
                                           (200, 64, 96, 13, 3, synth.ACT_BF16),
                                           # single-wave permutation: <= 128 pairs, <= 128 experts, k <= 16
                                           (128, 256, 128, 32, 4, synth.ACT_BF16),
                                           (128, 256, 128, 31, 4, synth.ACT_FP8_E4M3),
                                           (64, 96, 128, 25, 5, synth.ACT_BF16),
                                           (16, 64, 64, 8, 16, synth.ACT_BF16),
                                           (3, 64, 64, 2, 3, synth.ACT_BF16),
                                           (127, 64, 96, 42, 3, synth.ACT_BF16),
                                           # decode batches: gate_up routes the batch itself
                                           # (T <= 8, T * k <= 128, E <= 128, H >= 160)
                                           (128, 288, 320, 8, 4, synth.ACT_BF16),
                                           (128, 288, 320, 9, 4, synth.ACT_BF16),
                                           (100, 256, 128, 5, 5, synth.ACT_BF16),
                                           (64, 256, 128, 7, 16, synth.ACT_BF16),
                                           (128, 320, 256, 1, 1, synth.ACT_BF16),
                                           (9, 2880, 2880, 3, 4, synth.ACT_BF16)])
def test_moe_layer_equals_route_then_forward(mx, E, H, I, T, k, act):
    L = synth.layer(seed=E + H, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 3, T, E=E, H=H)
    Ld = _layer_dev(L)
    lg, xd = to_dev(logits, torch), to_dev(x, torch)
    ids, w = mx.mxfp4_route_topk(lg, k)
    out_a = mx.mxfp4_moe_forward(xd, ids, w, Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"],
                                 Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], act)
    out_b, ids_b, w_b = mx.mxfp4_moe_layer(xd, lg, k, Ld["w13_blocks"], Ld["w13_scales"], Ld["w13_bias"],
                                           Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"], act)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_b) and torch.equal(w, w_b)
    assert torch.equal(out_a, out_b)
    rid, rw = oracle.route_topk(logits, k)
    assert np.array_equal(ids_b.cpu().numpy(), rid)


@pytest.mark.parametrize("H", [64, 256])
@pytest.mark.parametrize("T,E,k", [(32, 128, 4), (7, 128, 16), (25, 100, 5), (8, 128, 4), (3, 100, 5)])
def test_moe_layer_routing_ties_and_signed_zero(mx, T, E, k, H):
    """Tie-heavy logits (small integers, all-zero rows, -0 next to +0) routed by
    the layer (H = 64: the fused route + permutation launch; H = 256: the
    gate_up kernel routing the batch itself) equal the stand-alone router
    bitwise, and the oracle's choices."""
    rng = np.random.default_rng(T + E)
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    logits[0] = 0.0
    logits[1, ::3] = -0.0
    logits[2, :] = -np.inf
    logits[2, 5] = 1.0
    I = H
    L = synth.layer(seed=9, E=E, H=H, I=I)
    Ld = _layer_dev(L)
    x = synth.f32_to_bf16_bits(rng.normal(size=(T, H)).astype(np.float32))
    lg = to_dev(logits, torch)
    ids, w = mx.mxfp4_route_topk(lg, k)
    _, ids_b, w_b = mx.mxfp4_moe_layer(to_dev(x, torch), lg, k, Ld["w13_blocks"], Ld["w13_scales"],
                                       Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"],
                                       synth.ACT_BF16)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_b) and torch.equal(w, w_b)
    rid, _ = oracle.route_topk(logits, k)
    assert np.array_equal(ids_b.cpu().numpy(), rid)


@pytest.mark.parametrize("name", ["moe_decode_t4", "moe_decode_t32"])
def test_moe_layer_decode_workload_against_golden(mx, full_layer, name):
    wl = synth.workload(name)
    g = np.load(os.path.join(GOLDEN, "%s.npz" % name))
    lg, xd = to_dev(wl["logits"], torch), to_dev(wl["x"], torch)
    Ld = full_layer[1]
    out, ids, _ = mx.mxfp4_moe_layer(xd, lg, synth.TOPK_GPT_OSS, Ld["w13_blocks"], Ld["w13_scales"],
                                     Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"], Ld["w2_bias"],
                                     wl["act_mode"])
    torch.cuda.synchronize()
    rid, _ = oracle.route_topk(wl["logits"], synth.TOPK_GPT_OSS)
    assert np.array_equal(ids.cpu().numpy(), rid)
    got = bf16_dev_to_f64(out)[g["tokens"]]
    assert_close(got, g["out"].astype(np.float64), name + " via moe_layer")


# ------------------------------------------------------------ NVFP4 weights ----


def _nv_dev(L):
    return {k: (to_dev(v, torch) if isinstance(v, np.ndarray) else v) for k, v in L.items()}


def _run_nv(mx, Ld, x_bits, ids, w):
    out = mx.nvfp4_moe_forward(to_dev(x_bits, torch), to_dev(ids.astype(np.int32), torch),
                               to_dev(w.astype(np.float32), torch), Ld["w13_blocks"], Ld["w13_scales"],
                               Ld["w13_global"], Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"],
                               Ld["w2_global"], Ld["w2_bias"])
    torch.cuda.synchronize()
    return out


def _mx_as_nv(blocks, scales):
    """MXFP4 weights as NVFP4 with the same values (power-of-two E4M3 scales)."""
    nb = blocks.shape[-2]
    e = scales.astype(np.int64) - 127
    assert e.min() >= -9 and e.max() <= 8
    # 2^-6 .. 2^8 are E4M3 normals (mantissa 0); 2^-9 .. 2^-7 are the
    # subnormal codes 1, 2, 4 (m * 2^-9)
    codes = np.where(e >= -6, (e + 7) << 3, 1 << np.clip(e + 9, 0, 2)).astype(np.uint8)
    return (np.ascontiguousarray(blocks.reshape(blocks.shape[:-2] + (2 * nb, 8))),
            np.ascontiguousarray(np.repeat(codes, 2, axis=-1)))


# NVFP4 runs where 160 <= H, I <= 3072; H/32 and I/32 still give every K tail
# modulo 4, and the largest case fills the kernel's twelve chunk groups
NV_SMALL = [  # E, H, I, T, k
    (8, 288, 320, 1, 4),
    (8, 288, 320, 5, 4),
    (8, 288, 320, 37, 4),
    (16, 160, 256, 300, 4),
    (4, 224, 192, 70, 2),
    (1, 256, 160, 9, 1),
    (2, 3072, 3072, 3, 2),
]


@pytest.mark.parametrize("E,H,I,T,k", [(8, 288, 320, 37, 4), (16, 160, 256, 300, 4), (4, 224, 192, 70, 2)])
def test_nvfp4_equals_mxfp4_for_power_of_two_scales(mx, E, H, I, T, k):
    # the same weight values in both formats give bitwise the same layer
    L = synth.layer(seed=E * 5 + H, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 1, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    ref = _run_moe(mx, _layer_dev(L), x, ids, w, synth.ACT_BF16)
    n13, m13 = _mx_as_nv(L["w13_blocks"], L["w13_scales"])
    n2, m2 = _mx_as_nv(L["w2_blocks"], L["w2_scales"])
    Nd = _nv_dev(dict(w13_blocks=n13, w13_scales=m13, w13_global=1.0, w13_bias=L["w13_bias"],
                      w2_blocks=n2, w2_scales=m2, w2_global=1.0, w2_bias=L["w2_bias"]))
    got = bf16_dev_to_f64(_run_nv(mx, Nd, x, ids, w))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("E,H,I,T,k", NV_SMALL)
def test_nvfp4_small_layers(mx, E, H, I, T, k):
    L = synth.nvfp4_layer(seed=E * 11 + H, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 5, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    got = bf16_dev_to_f64(_run_nv(mx, _nv_dev(L), x, ids, w))
    ref = oracle.moe_forward_routed(x, ids, w, L["w13_blocks"], L["w13_scales"], L["w13_bias"],
                                    L["w2_blocks"], L["w2_scales"], L["w2_bias"],
                                    weight_format=("nvfp4", L["w13_global"], L["w2_global"]))
    assert_close_rounded(got, ref["out"], "nvfp4 E%d H%d I%d T%d" % (E, H, I, T))


def test_nvfp4_decode_wide_activation_range(mx):
    """The NVFP4 decode kernels multiply f16 operands: each m-tile column of
    bf16 activations is scaled by its own power of two into f16.  Tokens
    2^50 apart in magnitude (beyond f16's range on both sides, several in one
    m-tile) and a token with outliers 2^12 above its other values must meet
    the layer bar against the oracle."""
    E, H, I, T, k = 4, 288, 320, 8, 4
    L = synth.nvfp4_layer(seed=412, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(411, T, E=E, H=H)
    xf = oracle.bf16_bits_to_f64(x) * 2.0 ** np.array([20, -30, 0, 12, -12, 5, 0, -20])[:, None]
    xf[2, ::37] *= 2.0 ** 12
    x = synth.f32_to_bf16_bits(xf.astype(np.float32))
    ids, w = oracle.route_topk(logits, k)
    got = bf16_dev_to_f64(_run_nv(mx, _nv_dev(L), x, ids, w))
    ref = oracle.moe_forward_routed(x, ids, w, L["w13_blocks"], L["w13_scales"], L["w13_bias"],
                                    L["w2_blocks"], L["w2_scales"], L["w2_bias"],
                                    weight_format=("nvfp4", L["w13_global"], L["w2_global"]))
    for t in range(T):   # per token: their magnitudes differ by up to 2^100
        assert_close_rounded(got[t:t + 1], ref["out"][t:t + 1], "nvfp4 wide range, token %d" % t)


@pytest.mark.parametrize("T", [4, 32])
def test_nvfp4_decode_full_size_sampled(mx, T):
    # gpt-oss-120b MoE shape with NVFP4 weights; the oracle on 4 sampled tokens
    L = synth.nvfp4_layer()
    logits, x = synth.moe_inputs(40 + T, T)
    ids, w = oracle.route_topk(logits, synth.TOPK_GPT_OSS)
    got = bf16_dev_to_f64(_run_nv(mx, _nv_dev(L), x, ids, w))
    no_constant_rows(got)
    toks = np.random.default_rng(T).choice(T, min(T, 4), replace=False)
    ref = oracle.moe_forward_routed(x[toks], ids[toks], w[toks], L["w13_blocks"], L["w13_scales"],
                                    L["w13_bias"], L["w2_blocks"], L["w2_scales"], L["w2_bias"],
                                    weight_format=("nvfp4", L["w13_global"], L["w2_global"]))
    assert_close(got[toks], ref["out"], "nvfp4 decode T%d" % T)


def test_nvfp4_rejects_small_shapes_and_bad_globals(mx):
    L = synth.nvfp4_layer(seed=3, E=4, H=160, I=160)
    Ld = _nv_dev(L)
    logits, x = synth.moe_inputs(1, 4, E=4, H=160)
    ids, w = oracle.route_topk(logits, 2)
    bad = dict(L, w13_global=float("inf"))
    with pytest.raises(mx.Mxfp4Error):
        _run_nv(mx, _nv_dev(bad), x, ids, w)
    S = synth.nvfp4_layer(seed=3, E=4, H=128, I=160)
    _, xs = synth.moe_inputs(1, 4, E=4, H=128)
    with pytest.raises(mx.Mxfp4Error):
        _run_nv(mx, _nv_dev(S), xs, ids, w)
    out = _run_nv(mx, Ld, x, ids, w)
    assert out.shape == (4, 160)
