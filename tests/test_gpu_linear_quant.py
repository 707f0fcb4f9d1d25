"""GPU parity of the dense projection with quantised activations (FP8 E4M3
per tensor, or MXFP4 per 32-element block), through the C ABI, against the
float64 oracle (oracle.moe.linear_act).

The activation codes are a deterministic function of x on both sides, so the
outputs differ only by the kernel's fp32 arithmetic: the block-scaled MFMA's
internal sums (about 2.4e-5 of the sum of |products| per 128 elements,
measured), the fp32 adds across K steps, the scale and the bias, and the final
bf16 rounding.  Bars: the layer bar beyond each output's bf16 rounding
interval (assert_close_rounded), and per output a distance beyond that
interval of at most MFMA_REL times the sum of |a_k w_k| plus a few fp32 ulps
of the output.
"""

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close_rounded, bf16_dev_to_f64, bf16_rounding_interval, no_constant_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ACT_FP8, ACT_MX = synth.ACT_FP8_E4M3, synth.ACT_MXFP4
# twice the measured internal error of the block-scaled MFMA, plus 24 fp32
# adds (one per K step at K = 2880) of u = 2^-24 each
MFMA_REL = 4.8e-5 + 24 * 2.0 ** -24


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import mxfp4_block_scaled_top_amd as m
    m.lib()
    return m


def _check(got, res, W, b, what):
    """got: bf16 outputs as float64; res: oracle.moe.linear_act result for the
    same weight rows W (dequantised, float64) and bias b."""
    ref = res["out"]
    lo, hi = bf16_rounding_interval(got)
    dist = np.maximum(np.maximum(lo - ref, ref - hi), 0.0)
    S = np.abs(res["a"]) @ np.abs(W).T + np.abs(b)
    bound = MFMA_REL * S + 4 * 2.0 ** -24 * np.abs(ref)
    ratio = float(np.max(dist / np.maximum(bound, 1e-300)))
    print("%s: max (distance beyond rounding) / bound = %.3f" % (what, ratio))
    assert np.all(dist <= bound), "%s: %d outputs beyond the MFMA error bound (worst ratio %.2f)" % (
        what, int(np.sum(dist > bound)), ratio)
    assert_close_rounded(got, ref, what)


def _run(mx, x, D, act, rows=None, workspace=None):
    out = mx.mxfp4_linear(to_dev(x, torch), to_dev(D["w_blocks"], torch), to_dev(D["w_scales"], torch),
                          to_dev(D["bias"], torch) if D.get("bias") is not None else None,
                          act_mode=act, workspace=workspace)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(out)


def _oracle(x, D, act, rows=None):
    wb, ws, b = D["w_blocks"], D["w_scales"], D.get("bias")
    if rows is not None:
        wb, ws, b = wb[rows], ws[rows], (b[rows] if b is not None else None)
    res = oracle.moe.linear_act(x, wb, ws, b, act)
    W = oracle.dequant(wb, ws)
    bias = oracle.bf16_bits_to_f64(b) if b is not None else np.zeros(W.shape[0])
    return res, W, bias


# one row tile and a ragged one, one and two n-tiles (256 weight rows each)
# with a 16-row remainder, K of one step, ragged steps, the gpt-oss widths and
# K above 3072 (the scale restaging's byte path)
@pytest.mark.parametrize("act", [ACT_FP8, ACT_MX])
@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (5, 272, 160), (130, 304, 288), (257, 48, 2880),
                                   (64, 2880, 4096), (200, 5120, 2880)])
def test_linear_quantised_shapes(mx, act, M, N, K):
    D = synth.dense(M * 7 + N + K, N, K)
    x = synth.dense_x(M + 3 * K, M, K)
    got = _run(mx, x, D, act)
    res, W, b = _oracle(x, D, act)
    _check(got, res, W, b, "linear act %d %dx%dx%d" % (act, M, N, K))
    no_constant_rows(got)


@pytest.mark.parametrize("act", [ACT_FP8, ACT_MX])
@pytest.mark.parametrize("name", ["qkv_proj", "o_proj", "lm_head"])
def test_linear_quantised_prefill_dense_set(mx, act, name):
    """The gpt-oss projections at a prefill of 2048 tokens (lm_head: 512
    tokens, 2080 sampled weight rows including both ends)."""
    N, K = synth.DENSE_SHAPES[name]
    M = 512 if name == "lm_head" else 2048
    D = synth.dense(synth.DENSE_SEEDS[name], N, K)
    x = synth.dense_x(synth.DENSE_X_SEED + 100, M, K)
    got = _run(mx, x, D, act)
    rows = None
    if N > 8192:
        rng = np.random.default_rng(6)
        rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                         rng.choice(N, 2048, replace=False)]))
        got = got[:, rows]
    res, W, b = _oracle(x, D, act, rows)
    _check(got, res, W, b, "%s act %d, %d tokens" % (name, act, M))
    no_constant_rows(got)


def test_linear_quantised_zero_x_gives_bias_and_empty_m(mx):
    D = synth.dense(60, 272, 160)
    x = np.zeros((9, 160), dtype=np.uint16)
    for act in (ACT_FP8, ACT_MX):
        got = _run(mx, x, D, act)
        assert np.array_equal(got, np.broadcast_to(oracle.bf16_bits_to_f64(D["bias"]), got.shape))
        out = mx.mxfp4_linear(torch.zeros((0, 160), dtype=torch.bfloat16, device="cuda"),
                              to_dev(D["w_blocks"], torch), to_dev(D["w_scales"], torch), act_mode=act)
        assert out.shape == (0, 272)


def test_linear_quantised_repeatable_and_workspace_reused(mx):
    """Two calls give the same bits, also when one workspace serves a larger
    and then a smaller call; and no bias."""
    for act in (ACT_FP8, ACT_MX):
        need = mx.mxfp4_linear_workspace_size(300, 304, 2880, act)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        D = synth.dense(61, 304, 2880)
        D = dict(w_blocks=D["w_blocks"], w_scales=D["w_scales"], bias=None)
        xa = synth.dense_x(62, 300, 2880)
        xb = synth.dense_x(63, 37, 2880)
        a1 = _run(mx, xa, D, act, workspace=ws)
        b1 = _run(mx, xb, D, act, workspace=ws)
        a2 = _run(mx, xa, D, act)
        assert np.array_equal(a1, a2)
        res, W, b = _oracle(xb, D, act)
        _check(b1, res, W, b, "reused workspace act %d" % act)
