"""Shared helpers of the test-suite (device transfer, tolerance checks)."""

import numpy as np

REL_FRO_TOL = 2e-3        # relative Frobenius error bound of layer outputs
MAX_ABS_TOL = 2e-2        # max |error| bound, as a fraction of rms(reference)


def to_dev(a, torch):
    """numpy -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def bf16_dev_to_f64(t):
    """bf16 device tensor -> float64 numpy (exact)."""
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    rel_fro = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    max_abs = np.max(np.abs(d)) if d.size else 0.0
    return rel_fro, max_abs, rms


def assert_close(got, ref, what=""):
    rel_fro, max_abs, rms = errors(got, ref)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    assert rel_fro <= REL_FRO_TOL, "%s: rel Frobenius %.3e > %.1e" % (what, rel_fro, REL_FRO_TOL)
    assert max_abs <= MAX_ABS_TOL * rms, "%s: max abs %.3e > %.1e * rms %.3e" % (
        what, max_abs, MAX_ABS_TOL, rms)
    return rel_fro, max_abs / max(rms, 1e-300)


def bf16_rounding_interval(v):
    """Interval [lo, hi] of reals that round (to nearest) to each bf16 value v:
    half the spacing above, and half the spacing below, which is half as wide
    when |v| is a power of two."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    half = np.ldexp(1.0, (e - 8).astype(np.int64))
    pow2 = a == np.ldexp(1.0, e.astype(np.int64))
    toward0 = np.where(pow2, half / 2, half)
    away = half
    lo = np.where(v >= 0, v - toward0, v - away)
    hi = np.where(v >= 0, v + away, v + toward0)
    return lo, hi


def assert_close_rounded(got, ref, what=""):
    """The same bar applied to the value the bf16 output was rounded from.

    A bf16 output g stands for every real in [g - u, g + u] (u = half its
    spacing); the distance from the reference to that interval must meet the
    relative-Frobenius and max-abs bounds.  Used where outputs are few or
    heavy-tailed, so that the final rounding alone, which no kernel can avoid,
    would already exceed the max-abs bound.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    lo, hi = bf16_rounding_interval(got)
    dist = np.maximum(np.maximum(lo - ref, ref - hi), 0.0)
    rms = np.sqrt(np.mean(ref ** 2))
    rel_fro = np.linalg.norm(dist) / max(np.linalg.norm(ref), 1e-300)
    assert rel_fro <= REL_FRO_TOL, "%s: rel Frobenius beyond rounding %.3e" % (what, rel_fro)
    assert dist.max() <= MAX_ABS_TOL * rms, "%s: max abs beyond rounding %.3e > %.1e * rms %.3e" % (
        what, dist.max(), MAX_ABS_TOL, rms)
    return rel_fro, dist.max() / max(rms, 1e-300)


def assert_close_slack(got, ref, slack, what=""):
    """The bar with a per-output allowance `slack` for outputs that are not
    unique (see tests/golden/make_golden.py): the distance beyond the slack
    must meet the relative-Frobenius and max-abs bounds."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    dist = np.maximum(np.abs(got - ref) - np.asarray(slack, dtype=np.float64), 0.0)
    rms = np.sqrt(np.mean(ref ** 2))
    rel_fro = np.linalg.norm(dist) / max(np.linalg.norm(ref), 1e-300)
    assert rel_fro <= REL_FRO_TOL, "%s: rel Frobenius beyond slack %.3e" % (what, rel_fro)
    assert dist.max() <= MAX_ABS_TOL * rms, "%s: max abs beyond slack %.3e > %.1e * rms %.3e" % (
        what, dist.max(), MAX_ABS_TOL, rms)
    return rel_fro, dist.max() / max(rms, 1e-300)


def assert_close_rounded_slack(got, ref, slack, what=""):
    """assert_close_rounded with the per-output allowance of assert_close_slack:
    the distance from the reference to each bf16 output's rounding interval,
    less the slack, must meet the bounds."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    lo, hi = bf16_rounding_interval(got)
    dist = np.maximum(np.maximum(lo - ref, ref - hi), 0.0)
    dist = np.maximum(dist - np.asarray(slack, dtype=np.float64), 0.0)
    rms = np.sqrt(np.mean(ref ** 2))
    rel_fro = np.linalg.norm(dist) / max(np.linalg.norm(ref), 1e-300)
    assert rel_fro <= REL_FRO_TOL, "%s: rel Frobenius beyond rounding and slack %.3e" % (what, rel_fro)
    assert dist.max() <= MAX_ABS_TOL * rms, "%s: max abs beyond rounding and slack %.3e > %.1e * rms %.3e" % (
        what, dist.max(), MAX_ABS_TOL, rms)
    return rel_fro, dist.max() / max(rms, 1e-300)


def no_constant_rows(out):
    """Broken FP4 kernels were reported to emit rows made of one repeated value
    (forum page, bug 1); a healthy layer output never does at these sizes."""
    out = np.asarray(out)
    if out.shape[1] > 1:
        assert not np.any(np.all(out == out[:, :1], axis=1)), "constant output row"
