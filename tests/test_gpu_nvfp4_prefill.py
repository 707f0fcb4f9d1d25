"""GPU parity of the MoE layer with NVFP4 expert weights and E4M3 activations
(the prefill GEMMs), through the C ABI, against the float64 oracle.

Both GEMMs expand the E4M3 codes and the NVFP4 weights (E2M1 x E4M3 block
scale) exactly to bf16 and run the bf16 MFMA with fp32 sums; the global
scale joins the per-tensor activation scale in the epilogue.  Checks, as for
the MXFP4 FP8 mode: the x codes and scale bit-exact; h close to the oracle's
h (fp32 arithmetic only); the GPU's h codes equal to the oracle codec applied
to the GPU's own h; the output equal, to the layer bar, to the down GEMM and
combine computed by the oracle from those codes; and, against the oracle's
own h, differing h codes only where an h within the kernel's fp32 error
bound takes them.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close_rounded, bf16_dev_to_f64, errors, no_constant_rows, to_dev
from parity import down_combine, fp32, fp8_code_mismatch, gate_up_terms, h_tolerance
from test_gpu_parity import _code_rows, _f32, _layer_dev, _mx_as_nv, _nv_dev, _run_moe, _run_nv, _status, _ws_view

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FP8 = synth.ACT_FP8_E4M3


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import mxfp4_block_scaled_top_amd as m
    m.lib()
    return m


def _run(mx, Ld, x, ids, w, ready=False, ws=None):
    T, H = x.shape
    E, twoI = Ld["w13_blocks"].shape[:2]
    k = ids.shape[1]
    if ws is None:
        ws = torch.zeros(mx.nvfp4_moe_workspace_size(T, H, twoI // 2, E, k, FP8), dtype=torch.uint8,
                         device="cuda")
    out = mx.nvfp4_moe_forward(to_dev(x, torch), to_dev(ids.astype(np.int32), torch),
                               to_dev(w.astype(np.float32), torch), Ld["w13_blocks"], Ld["w13_scales"],
                               Ld["w13_global"], Ld["w13_bias"], Ld["w2_blocks"], Ld["w2_scales"],
                               Ld["w2_global"], Ld["w2_bias"], act_mode=FP8, workspace=ws,
                               scale_streams_ready=ready)
    torch.cuda.synchronize()
    lay = mx.mxfp4_moe_workspace_layout_query(T, H, twoI // 2, E, k, FP8)
    return bf16_dev_to_f64(out), ws, lay


def _dq(L, which, e):
    g = L["w13_global"] if which == 13 else L["w2_global"]
    return oracle.dequant_nvfp4(L["w%d_blocks" % which][e], L["w%d_scales" % which][e], g)


def _bias(L, which, e, n):
    b = L["w%d_bias" % which]
    return np.zeros(n) if b is None else oracle.bf16_bits_to_f64(b[e])


def _check(mx, L, x, ids, w, what, tokens=None, ready=False):
    """The layer against the oracle on `tokens` (all if None).  The x and h
    scales are the batch's, so the reference h is formed here from the
    batch's x codes (the oracle's gate_up terms and SwiGLU)."""
    T, H = x.shape
    k = ids.shape[1]
    I = L["w2_blocks"].shape[2] * 16
    got, ws, lay = _run(mx, _nv_dev(L), x, ids, w)
    if ready:   # the same call again with the restaged scale streams kept
        got2, _, _ = _run(mx, _nv_dev(L), x, ids, w, ready=True, ws=ws)
        assert np.array_equal(got, got2)
    no_constant_rows(got)
    all_tokens = tokens is None
    tokens = np.arange(T) if all_tokens else np.asarray(tokens)
    np_ = T * k
    st = _status(ws, lay)
    inv = _ws_view(ws, lay, "inv_pairs", np.int32, np_)
    # x codes (sorted rows) and the scale over the whole batch
    xc_all, xs_all, _ = oracle.quant_per_tensor(oracle.bf16_bits_to_f64(x))
    assert _f32(st[3]) == xs_all
    xc = _code_rows(ws, lay, "x_codes", np_, H)
    rows = inv.reshape(T, k)[tokens].reshape(-1)
    assert np.array_equal(xc[rows], np.repeat(xc_all[tokens], k, axis=0))
    # the GPU's h codes are the codec on its own fp32 h, amax over all pairs
    h_gpu = _ws_view(ws, lay, "h", np.float32, np_ * I).reshape(np_, I).astype(np.float64)
    hc_gpu = _code_rows(ws, lay, "h_codes", np_, I)
    s_h = _f32(st[4])
    rc, rs, ra = oracle.quant_per_tensor(h_gpu)
    assert _f32(st[2]) == ra and s_h == rs
    assert np.array_equal(hc_gpu, rc)
    # h of the listed tokens' pairs ((token, slot) order) against the oracle
    a = (oracle.e4m3_decode(xc_all) * xs_all)[tokens]
    pair_e = ids[tokens].reshape(-1)
    h_ref = np.zeros((len(pair_e), I))
    tol = np.zeros_like(h_ref)
    for e in np.unique(pair_e):
        sel = np.nonzero(pair_e == e)[0]
        g, R = gate_up_terms(a[sel // k], _dq(L, 13, int(e)), _bias(L, 13, int(e), 2 * I))
        h_ref[sel] = oracle.moe.swiglu(g, I)
        tol[sel] = h_tolerance(g, R, I)
    rf, _, _ = errors(h_gpu[rows], h_ref)
    print("%s: h rel Frobenius %.2e" % (what, rf))
    assert rf < 1e-5
    # codes that differ from the codec on the oracle's h: only within its bound
    _, ndiff = fp8_code_mismatch(hc_gpu[rows], s_h, fp32(h_ref), tol, s_h)
    print("%s: %d of %d h codes differ from the oracle's" % (what, ndiff, h_ref.size))
    assert ndiff <= max(2, 1e-4 * h_ref.size)
    # output = down + combine of the GPU's own codes, to the layer bar
    hq = oracle.e4m3_decode(hc_gpu[rows]) * s_h
    own = down_combine(hq, np.repeat(tokens, k), pair_e, w[tokens].reshape(-1), tokens,
                       lambda e: _dq(L, 2, e), lambda e: _bias(L, 2, e, H))
    assert_close_rounded(got[tokens], own, what + " (own h codes)")
    if all_tokens and ndiff == 0:
        ref = oracle.moe_forward_routed(x, ids, w, L["w13_blocks"], L["w13_scales"], L["w13_bias"],
                                        L["w2_blocks"], L["w2_scales"], L["w2_bias"], act_mode=FP8,
                                        weight_format=("nvfp4", L["w13_global"], L["w2_global"]))
        assert_close_rounded(got, ref["out"], what + " (oracle)")
    return got


# every K tail modulo 4 (H/32, I/32), one expert, k = 1, a token count past
# one 128-row tile per expert; no lower limit on H, I with E4M3 activations.
# Experts averaging at most 64 rows take 64-row tiles (all but the 300- and
# 150-token cases; at 120 tokens some experts span two tiles).
NV_FP8_SMALL = [  # E, H, I, T, k
    (8, 288, 320, 1, 4),
    (8, 288, 320, 37, 4),
    (16, 96, 128, 300, 4),
    (4, 224, 64, 70, 2),
    (1, 64, 96, 9, 1),
    (2, 3200, 1024, 150, 2),
    (8, 288, 320, 120, 4),
]


@pytest.mark.parametrize("E,H,I,T,k", NV_FP8_SMALL)
def test_nvfp4_fp8_small_layers(mx, E, H, I, T, k):
    L = synth.nvfp4_layer(seed=E * 13 + H, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 19, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    _check(mx, L, x, ids, w, "nvfp4 fp8 E%d H%d I%d T%d k%d" % (E, H, I, T, k), ready=(T == 300))


@pytest.mark.parametrize("E,H,I,T,k", [(8, 288, 320, 37, 4), (16, 96, 128, 300, 4)])
def test_nvfp4_fp8_gate_up_equals_mxfp4_for_power_of_two_scales(mx, E, H, I, T, k):
    """With power-of-two block scales and global 1 the NVFP4 weights hold the
    MXFP4 values; the gate_up operands are then the same bf16 numbers in the
    same MFMA order: bitwise the same h (the down GEMMs differ: MXFP4 takes
    the block-scaled FP8 x FP4 instruction)."""
    L = synth.layer(seed=E * 5 + H + 1, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(T + 2, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    _, ws_mx, lay = _run_moe(mx, _layer_dev(L), x, ids, w, FP8, want_ws=True)
    n13, m13 = _mx_as_nv(L["w13_blocks"], L["w13_scales"])
    n2, m2 = _mx_as_nv(L["w2_blocks"], L["w2_scales"])
    Nd = _nv_dev(dict(w13_blocks=n13, w13_scales=m13, w13_global=1.0, w13_bias=L["w13_bias"],
                      w2_blocks=n2, w2_scales=m2, w2_global=1.0, w2_bias=L["w2_bias"]))
    _, ws_nv, _ = _run(mx, Nd, x, ids, w)
    np_ = T * k
    for key, n in (("x_codes", H), ("h_codes", I)):
        assert np.array_equal(_code_rows(ws_mx, lay, key, np_, n), _code_rows(ws_nv, lay, key, np_, n)), key
    assert np.array_equal(_ws_view(ws_mx, lay, "h", np.float32, np_ * I), _ws_view(ws_nv, lay, "h", np.float32, np_ * I))
    assert np.array_equal(_status(ws_mx, lay)[:5], _status(ws_nv, lay)[:5])


def test_nvfp4_fp8_wide_n_units_multi_unit(mx):
    """gpt-oss widths with the experts averaging 50 rows: the wide-N units
    (64 rows x two n-tiles), about 750 gate_up units over the 256 blocks, so
    the copier steps into further units; every token checked."""
    E, H, I, T, k = 48, 2880, 2880, 600, 4
    L = synth.nvfp4_layer(seed=421, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(422, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    _check(mx, L, x, ids, w, "nvfp4 fp8 wide-N E%d T%d" % (E, T))


@pytest.mark.parametrize("T", [2048])
def test_nvfp4_fp8_prefill_full_size_sampled(mx, T):
    """The gpt-oss-120b MoE shape with NVFP4 weights at a 2048-token prefill;
    the oracle on 16 sampled tokens."""
    L = synth.nvfp4_layer()
    logits, x = synth.moe_inputs(90 + T, T)
    ids, w = oracle.route_topk(logits, synth.TOPK_GPT_OSS)
    toks = np.sort(np.random.default_rng(T + 1).choice(T, 16, replace=False))
    _check(mx, L, x, ids, w, "nvfp4 fp8 T%d" % T, tokens=toks)


def _every_scale_code(L, seed):
    """L with its block scales drawn from every finite E4M3 code (both signs,
    zero and the subnormals m * 2^-9 included), each code at least once per
    tensor; the kernels decode the scales with the hardware conversion."""
    rng = np.random.default_rng(seed)
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    out = dict(L)
    for key in ("w13_scales", "w2_scales"):
        sc = rng.choice(codes, size=L[key].shape).astype(np.uint8)
        sc.reshape(-1)[:codes.size] = rng.permutation(codes)
        out[key] = sc
    return out


def test_nvfp4_every_finite_scale_code(mx):
    """Both NVFP4 paths (bf16 activations: the decode GEMV; E4M3 activations:
    the prefill GEMMs) with every finite E4M3 block-scale code."""
    E, H, I, T, k = 8, 288, 320, 37, 4
    L = _every_scale_code(synth.nvfp4_layer(seed=401, E=E, H=H, I=I), 402)
    logits, x = synth.moe_inputs(403, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, k)
    got = bf16_dev_to_f64(_run_nv(mx, _nv_dev(L), x, ids, w))
    no_constant_rows(got)
    ref = oracle.moe_forward_routed(x, ids, w, L["w13_blocks"], L["w13_scales"], L["w13_bias"],
                                    L["w2_blocks"], L["w2_scales"], L["w2_bias"],
                                    weight_format=("nvfp4", L["w13_global"], L["w2_global"]))
    assert_close_rounded(got, ref["out"], "nvfp4 bf16, every scale code")
    _check(mx, L, x, ids, w, "nvfp4 fp8, every scale code")
