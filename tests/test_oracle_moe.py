"""Pins for the oracle's routing, permutation, MoE layer and dense linear.

The MoE layer and the dense linear are checked against a pure-Python brute
force written from the definitions on tiny shapes: every weight is decoded
from its nibble and scale bits with exact rationals, contractions are exact
(fractions.Fraction), only silu/exp are float64.  Routing is checked against
a full sort, permutation against explicit loops.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle.moe import ACT_BF16, ACT_FP8_E4M3, ACT_MXFP4

# ----------------------------------------------------------------- brute force


def _bf_e2m1(code):
    s = -1 if code & 8 else 1
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return s * mag


def _bf_weight(blocks, scales, n, kk):
    byte = int(blocks[n, kk // 32, (kk % 32) // 2])
    code = (byte >> 4) if kk % 2 else (byte & 15)
    return _bf_e2m1(code) * Fraction(2) ** (int(scales[n, kk // 32]) - 127)


def _bf_bf16(bits):
    return Fraction(struct.unpack(">f", struct.pack(">I", int(bits) << 16))[0])


def _bf_rn_f32(fr):
    if fr == 0:
        return Fraction(0)
    s = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * ulp


def _bf_e4m3_values():
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            vals.append((v, m))
    return vals


E4M3_VALS = _bf_e4m3_values()


def _bf_fp8_round(q):
    """Nearest E4M3 value (ties to even mantissa), saturating; returns Fraction."""
    a = abs(q)
    best = None
    for v, m in E4M3_VALS:
        d = abs(a - v)
        if best is None or d < best[0] or (d == best[0] and m % 2 == 0 and best[2] % 2 == 1):
            best = (d, v, m)
    return best[1] if q >= 0 else -best[1]


def _bf_quant(values):
    """Per-tensor FP8: returns list of dequantized Fractions."""
    amax = max(abs(v) for v in values)
    s = Fraction(1) if amax == 0 else _bf_rn_f32(amax / 448)
    return [_bf_fp8_round(_bf_rn_f32(v / s)) * s for v in values]


E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def _bf_floor_log2(a):
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _bf_mx_quant(values):
    """MXFP4 of one row (length a multiple of 32), block by block: shared
    exponent floor(log2 amax) - 2 clamped to [-116, 125], each |v| / 2^X to the
    nearest E2M1 magnitude (a tie to the even code, past 6 to 6), sign kept.
    Returns the dequantized Fractions."""
    out = []
    for b0 in range(0, len(values), 32):
        blk = values[b0:b0 + 32]
        amax = max(abs(v) for v in blk)
        X = -116 if amax == 0 else min(max(_bf_floor_log2(amax) - 2, -116), 125)
        sc = Fraction(2) ** X
        for v in blk:
            q = abs(v) / sc
            best = None
            for c, m in enumerate(E2M1_MAGS):
                d = abs(q - m)
                if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                    best = (d, c)
            mag = E2M1_MAGS[best[1]] * sc
            out.append(-mag if v < 0 else mag)
    return out


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _bf_moe(x_bits, logits, L, k, act_mode, routes=None):
    """Exact-rational MoE layer.  `routes`, if given, is the routing itself:
    routes[t] = [(expert id, weight), ...] for the k slots of token t; ids
    outside [0, E) name no expert, so their slot is left out altogether (no h,
    no part in the FP8 h scale, nothing added to the output)."""
    T, H = x_bits.shape
    E = L["w13_blocks"].shape[0]
    I = L["w2_blocks"].shape[2] * 32
    x = [[_bf_bf16(x_bits[t, i]) for i in range(H)] for t in range(T)]
    if act_mode == ACT_FP8_E4M3:
        flat = _bf_quant([v for row in x for v in row])
        x = [flat[t * H:(t + 1) * H] for t in range(T)]
    elif act_mode == ACT_MXFP4:
        x = [_bf_mx_quant(row) for row in x]
    if routes is None:
        routes = []
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
            z = [math.exp(float(logits[t, e]) - float(logits[t, order[0]])) for e in order]
            routes.append([(e, zi / sum(z)) for e, zi in zip(order, z)])
    hs = {}
    for t in range(T):
        for j, (e, _) in enumerate(routes[t]):
            if not 0 <= e < E:
                continue
            g = []
            for n in range(2 * I):
                acc = sum(_bf_weight(L["w13_blocks"][e], L["w13_scales"][e], n, kk) * x[t][kk]
                          for kk in range(H))
                g.append(acc + _bf_bf16(L["w13_bias"][e, n]))
            hs[t, j] = [_silu(float(g[i])) * float(g[I + i]) for i in range(I)]
    if act_mode == ACT_FP8_E4M3:
        keys = sorted(hs)
        flat = _bf_quant([_bf_rn_f32(Fraction(v)) for key in keys for v in hs[key]])
        hs = {key: flat[i * I:(i + 1) * I] for i, key in enumerate(keys)}
    elif act_mode == ACT_MXFP4:
        hs = {key: _bf_mx_quant([_bf_rn_f32(Fraction(v)) for v in val]) for key, val in hs.items()}
    else:
        hs = {key: [Fraction(v) for v in val] for key, val in hs.items()}
    out = np.zeros((T, H))
    for t in range(T):
        for j, (e, w) in enumerate(routes[t]):
            if not 0 <= e < E:
                continue
            for n in range(H):
                acc = sum(_bf_weight(L["w2_blocks"][e], L["w2_scales"][e], n, kk) * hs[t, j][kk]
                          for kk in range(I))
                out[t, n] += w * float(acc + _bf_bf16(L["w2_bias"][e, n]))
    return out


def _tiny(E=4, H=64, I=64, T=3, seed=9):
    L = synth.layer(seed=seed, E=E, H=H, I=I)
    logits, x = synth.moe_inputs(seed + 1, T, E=E, H=H)
    return L, logits, x


# --------------------------------------------------------------------- routing


def test_route_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(4)
    logits = rng.integers(-3, 4, size=(64, 16)).astype(np.float32)   # many ties
    logits[0, :] = 0.0
    logits[1, ::2] = -0.0                                            # -0 ties +0
    ids, w = oracle.route_topk(logits, 4)
    for t in range(64):
        want = sorted(range(16), key=lambda e: (-float(logits[t, e]), e))[:4]
        assert list(ids[t]) == want
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.allclose(w[0], 0.25)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_route_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(8)
    logits = rng.normal(size=(20, 128)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 4)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)
    assert np.all(np.diff(np.take_along_axis(logits, ids.astype(np.int64), axis=1), axis=1) <= 0)
    ids1, w1 = oracle.route_topk(logits, 1)
    assert np.array_equal(ids1[:, 0], np.argmax(logits, axis=1)) and np.all(w1 == 1.0)
    with pytest.raises(ValueError):
        oracle.route_topk(np.array([[np.nan, 1.0]], dtype=np.float32), 1)


def test_permute_matches_loops():
    rng = np.random.default_rng(12)
    T, k, E = 37, 4, 16
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sp, inv = oracle.permute(ids, E)
    want = []
    for e in range(E):
        want += [t * k + j for t in range(T) for j in range(k) if ids[t, j] == e]
        assert counts[e] == sum(1 for v in ids.ravel() if v == e)
    assert list(sp) == want
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(sp[inv], np.arange(T * k))


# -------------------------------------------------------------- moe and linear


@pytest.mark.parametrize("act_mode", [ACT_BF16, ACT_FP8_E4M3, ACT_MXFP4])
def test_moe_forward_matches_exact_brute_force(act_mode):
    L, logits, x = _tiny()
    res = oracle.moe_forward(x, logits, **L, k=2, act_mode=act_mode)
    bf = _bf_moe(x, logits, L, 2, act_mode)
    scale = np.sqrt(np.mean(bf ** 2))
    assert np.max(np.abs(res["out"] - bf)) <= 1e-12 * scale * 64


@pytest.mark.parametrize("act_mode", [ACT_BF16, ACT_FP8_E4M3, ACT_MXFP4])
def test_moe_forward_skips_out_of_range_ids_brute_force(act_mode):
    # ids -1, E and E+3 name no expert: the brute force leaves those slots out
    # (no h, no part in the FP8 h scale, nothing added to the output).  An id of
    # -1 read as the last expert (numpy's negative index) would add that
    # expert's output and, in FP8 mode, its h to the scale.
    L, logits, x = _tiny(T=4)
    E = L["w13_blocks"].shape[0]
    ids = np.array([[0, -1], [E, 2], [3, 1], [E + 3, -1]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.625, 0.375], [0.9, 0.1]])
    res = oracle.moe_forward_routed(x, ids, w, **L, act_mode=act_mode)
    routes = [[(int(e), float(wi)) for e, wi in zip(ids[t], w[t])] for t in range(4)]
    bf = _bf_moe(x, logits, L, 2, act_mode, routes=routes)
    scale = np.sqrt(np.mean(bf ** 2))
    assert np.max(np.abs(res["out"] - bf)) <= 1e-12 * scale * 64
    assert np.all(res["out"][3] == 0.0)             # both slots of token 3 skipped
    # the skipped slots carry no h, and the FP8 h scale is the one of the valid
    # pairs alone (against the same layer with the bad slots given expert E-1)
    assert np.all(res["h"][ids < 0] == 0.0) and np.all(res["h"][ids >= E] == 0.0)
    if act_mode == ACT_FP8_E4M3:
        valid = (ids >= 0) & (ids < E)
        amax = np.max(np.abs(res["h32"][valid]))
        assert res["h_scale"] == oracle.fp8.f32_scale(amax)
        alt = oracle.moe_forward_routed(x, np.where(valid, ids, E - 1), w, **L, act_mode=act_mode)
        assert not np.array_equal(alt["out"], res["out"])


def test_mxfp4_activation_mode_passes_representable_x_unchanged():
    # x made of MXFP4 values: quantising it again changes nothing, so the
    # gate_up outputs (and h) equal those of the bf16 mode exactly; the
    # down inputs do differ (h itself is not representable)
    E, H, I, T = 4, 96, 64, 6
    L = synth.layer(seed=41, E=E, H=H, I=I)
    rng = np.random.default_rng(42)
    xb = rng.integers(0, 256, size=(T, H // 32, 16), dtype=np.uint8)
    xs = rng.integers(120, 131, size=(T, H // 32), dtype=np.uint8)
    x = synth.f32_to_bf16_bits(oracle.dequant(xb, xs).astype(np.float32))
    logits, _ = synth.moe_inputs(43, T, E=E, H=H)
    ids, w = oracle.route_topk(logits, 2)
    mx = oracle.moe_forward_routed(x, ids, w, **L, act_mode=ACT_MXFP4)
    bf = oracle.moe_forward_routed(x, ids, w, **L, act_mode=ACT_BF16)
    assert np.array_equal(mx["h"], bf["h"])
    assert np.array_equal(oracle.dequant(mx["x_blocks"], mx["x_scales"]), oracle.bf16_bits_to_f64(x))
    assert not np.array_equal(mx["out"], bf["out"])


def test_swiglu_takes_silu_of_the_gate_half():
    # gate rows come first in the fused gate_up output; silu is applied to them only
    g = np.zeros(4)
    g[:2] = [1.0, -2.0]
    g[2:] = [3.0, 0.5]
    h = oracle.swiglu(g, 2)
    assert np.allclose(h, [_silu(1.0) * 3.0, _silu(-2.0) * 0.5], rtol=1e-15)
    assert not np.allclose(h, [_silu(3.0) * 1.0, _silu(0.5) * -2.0])


def test_moe_identical_experts_equal_single_expert():
    E, H, I, T = 6, 64, 96, 5
    L1 = synth.layer(seed=21, E=1, H=H, I=I)
    LE = {key: np.repeat(v, E, axis=0) for key, v in L1.items()}
    logits, x = synth.moe_inputs(22, T, E=E, H=H)
    outE = oracle.moe_forward(x, logits, **LE, k=4)["out"]
    out1 = oracle.moe_forward(x, np.zeros((T, 1), np.float32), **L1, k=1)["out"]
    assert np.allclose(outE, out1, rtol=1e-12, atol=1e-12)


def test_moe_e1_k1_reduces_to_dense_linear():
    H, I, T = 64, 64, 4
    L = synth.layer(seed=31, E=1, H=H, I=I)
    _, x = synth.moe_inputs(32, T, E=1, H=H)
    out = oracle.moe_forward(x, np.zeros((T, 1), np.float32), **L, k=1)["out"]
    g = oracle.linear(x, L["w13_blocks"][0], L["w13_scales"][0], L["w13_bias"][0])
    h = oracle.swiglu(g, I)
    W2 = oracle.dequant(L["w2_blocks"][0], L["w2_scales"][0])
    want = h @ W2.T + oracle.bf16_bits_to_f64(L["w2_bias"][0])
    assert np.allclose(out, want, rtol=1e-13, atol=1e-13)


def test_moe_token_permutation_equivariance():
    L, logits, x = _tiny(T=6)
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = oracle.moe_forward(x, logits, **L, k=2)["out"]
    b = oracle.moe_forward(x[perm], logits[perm], **L, k=2)["out"]
    assert np.allclose(a[perm], b, rtol=1e-13, atol=1e-13)


def test_linear_matches_exact_brute_force():
    N, K, M = 24, 96, 3
    D = synth.dense(41, N, K)
    x = synth.dense_x(42, M, K)
    got = oracle.linear(x, D["w_blocks"], D["w_scales"], D["bias"])
    for m in range(M):
        for n in range(N):
            acc = sum(_bf_weight(D["w_blocks"], D["w_scales"], n, kk) * _bf_bf16(x[m, kk])
                      for kk in range(K))
            want = float(acc + _bf_bf16(D["bias"][n]))
            assert abs(got[m, n] - want) <= 1e-13 * max(1.0, abs(want))
    rows = np.array([5, 0, 23])
    assert np.array_equal(oracle.linear_rows(x, D["w_blocks"], D["w_scales"], D["bias"], rows),
                          got[:, rows])


@pytest.mark.parametrize("act_mode", [ACT_FP8_E4M3, ACT_MXFP4])
def test_linear_act_matches_exact_brute_force(act_mode):
    """The quantised-activation dense projection against the brute force:
    per-tensor FP8 over all of x, or MXFP4 per 32-element block of each row,
    then the exact contraction and the bias."""
    N, K, M = 16, 96, 3
    D = synth.dense(43, N, K)
    x = synth.dense_x(44, M, K)
    res = oracle.moe.linear_act(x, D["w_blocks"], D["w_scales"], D["bias"], act_mode)
    vals = [_bf_bf16(v) for v in x.reshape(-1)]
    if act_mode == ACT_FP8_E4M3:
        q = _bf_quant(vals)                    # one scale over the whole of x
        a = [q[m * K:(m + 1) * K] for m in range(M)]
    else:
        a = [_bf_mx_quant(vals[m * K:(m + 1) * K]) for m in range(M)]
    for m in range(M):
        for kk in range(K):
            assert res["a"][m, kk] == float(a[m][kk])
        for n in range(N):
            acc = sum(_bf_weight(D["w_blocks"], D["w_scales"], n, kk) * a[m][kk] for kk in range(K))
            want = float(acc + _bf_bf16(D["bias"][n]))
            assert abs(res["out"][m, n] - want) <= 1e-13 * max(1.0, abs(want))


def test_linear_act_fp8_scale_spans_all_rows():
    """FP8 activations take one scale over the whole of x: a large element in
    row 0 changes the codes of the other rows; MXFP4 blocks do not see it."""
    N, K, M = 16, 64, 3
    D = synth.dense(45, N, K)
    x = synth.dense_x(46, M, K)
    big = x.copy()
    big[0, 5] = np.uint16(0x4700)                # bf16 32768.0
    f0 = oracle.moe.linear_act(x, D["w_blocks"], D["w_scales"], None, ACT_FP8_E4M3)
    f1 = oracle.moe.linear_act(big, D["w_blocks"], D["w_scales"], None, ACT_FP8_E4M3)
    assert f1["x_scale"] == np.float32(32768.0 / 448)
    assert not np.array_equal(f0["x_codes"][1:], f1["x_codes"][1:])
    m0 = oracle.moe.linear_act(x, D["w_blocks"], D["w_scales"], None, ACT_MXFP4)
    m1 = oracle.moe.linear_act(big, D["w_blocks"], D["w_scales"], None, ACT_MXFP4)
    assert np.array_equal(m0["out"][1:], m1["out"][1:])
    assert np.array_equal(m0["x_blocks"][0, 1:], m1["x_blocks"][0, 1:])


def test_linear_act_reduces_to_linear_on_representable_x():
    """Activations the quantisers represent exactly leave the projection as
    the plain definition: bf16 values k * 2^j with |k| <= 6 on a per-tensor
    maximum of 448 * 2^-3 (FP8), and E2M1 values times 2^X with a block
    maximum of 6 * 2^X (MXFP4)."""
    N, K, M = 32, 128, 4
    D = synth.dense(47, N, K)
    rng = np.random.default_rng(48)

    def bf16(v):
        return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)

    e4 = np.array([0, 0.25, 0.5, 1, 1.5, 2, 3, 4, 6, 56, 448], dtype=np.float64) / 8
    xf = rng.choice(e4, size=(M, K)) * rng.choice([-1, 1], size=(M, K))
    xf[0, 0] = 448 / 8
    x = bf16(xf)
    ref = oracle.linear(x, D["w_blocks"], D["w_scales"], D["bias"])
    got = oracle.moe.linear_act(x, D["w_blocks"], D["w_scales"], D["bias"], ACT_FP8_E4M3)
    assert got["x_scale"] == np.float32(1 / 8)
    assert np.array_equal(got["out"], ref)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    xm = rng.choice(mags, size=(M, K)) * rng.choice([-1, 1], size=(M, K))
    X = rng.integers(-20, 20, size=(M, K // 32))
    xm = xm.reshape(M, K // 32, 32)
    xm[:, :, 7] = 6.0
    xm = (xm * np.exp2(X)[:, :, None]).reshape(M, K)
    x = bf16(xm)
    ref = oracle.linear(x, D["w_blocks"], D["w_scales"], D["bias"])
    got = oracle.moe.linear_act(x, D["w_blocks"], D["w_scales"], D["bias"], ACT_MXFP4)
    assert np.array_equal(got["x_scales"], (X + 127).astype(np.uint8))
    assert np.array_equal(got["out"], ref)


def test_linear_act_power_of_two_scaling_of_x():
    """Scaling x by 2^j (in range) keeps every FP8 code and MXFP4 code, moves
    the scales by j, and scales the bias-free output by exactly 2^j."""
    N, K, M = 16, 64, 3
    D = synth.dense(49, N, K)
    x = synth.dense_x(50, M, K)
    x2 = (x.astype(np.uint32) + (3 << 7)).astype(np.uint16)   # bf16 exponent + 3 (no zeros in x)
    assert np.all((x & 0x7f80) != 0)
    for mode in (ACT_FP8_E4M3, ACT_MXFP4):
        r1 = oracle.moe.linear_act(x, D["w_blocks"], D["w_scales"], None, mode)
        r2 = oracle.moe.linear_act(x2, D["w_blocks"], D["w_scales"], None, mode)
        assert np.array_equal(r2["out"], 8 * r1["out"])
        if mode == ACT_FP8_E4M3:
            assert np.array_equal(r1["x_codes"], r2["x_codes"]) and r2["x_scale"] == 8 * r1["x_scale"]
        else:
            assert np.array_equal(r1["x_blocks"], r2["x_blocks"])
            assert np.array_equal(r2["x_scales"].astype(int), r1["x_scales"].astype(int) + 3)


def test_one_bf16_rounding_fits_the_tolerance_but_two_do_not():
    """Error budget behind the 'one rounding at the end' design: rounding a
    Gaussian output to bf16 once costs about 1.7e-3 relative Frobenius error,
    under the 2e-3 bar; an extra bf16 rounding of an intermediate does not fit."""
    rng = np.random.default_rng(1)
    ref = rng.normal(size=200000)
    r1 = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    e1 = np.linalg.norm(r1 - ref) / np.linalg.norm(ref)
    assert 1.4e-3 < e1 < 2e-3
    noise = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((ref + 1e-3).astype(np.float32)))
    e2 = np.linalg.norm((noise - 1e-3) - ref) / np.linalg.norm(ref)
    both = np.sqrt(e1 ** 2 + e2 ** 2)
    assert both > 2e-3
