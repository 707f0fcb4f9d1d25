"""FP8 E4M3 activation codec with one per-tensor scale (oracle; test only).

The pages run the MoE contraction as FP8 activations times FP4 weights
(spark-vllm page, "What's Included" / full MXFP4 stack: the MoE layers are an
FP8xFP4 grouped GEMM) and list full-scale activation quantization as open
work ("Numerical Accuracy"); they do not define the codec.  The format is
the OCP 8-bit floating point E4M3 encoding: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, subnormals at exponent field 0, no infinities,
S.1111.111 is NaN, largest finite magnitude 448.  The per-tensor scale is
amax/448, which names this variant (the FNUZ variant tops out at 240).

Readings where the pages are silent (each listed in the design doc):
  * scale s = fp32(amax / 448) with the quotient correctly rounded;
    amax == 0 gives s = 1;
  * the value coded is q = fp32(v / s), a correctly rounded fp32 divide
    (not a multiply by 1/s);
  * q -> code rounds to nearest, ties to even mantissa, and saturates to
    +-448 ("satfinite"); the sign of zero is kept (-0 -> 0x80).

Both roundings to fp32 are done by computing the quotient in float64 and
casting: for a quotient of two 24-bit numbers an intermediate of at least
2*24+2 bits makes the double rounding innocuous, and float64 has 53.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7


def e4m3_decode(code):
    """E4M3 code(s) (uint8) -> float64, from the bit fields."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = np.ldexp(m.astype(np.float64), 1 - E4M3_BIAS - 3)          # m * 2^-9
    nrm = np.ldexp(1.0 + m / 8.0, e - E4M3_BIAS)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(q):
    """Values q (float64 holding fp32 numbers, no NaN) -> E4M3 codes uint8.

    Round to nearest, ties to even mantissa, saturate to the largest finite
    magnitude, keep the sign of zero.
    """
    q = np.asarray(q, dtype=np.float64)
    if np.isnan(q).any():
        raise ValueError("NaN has no satfinite E4M3 code here")
    sign = np.signbit(q).astype(np.uint8)
    a = np.abs(q)
    # binade exponent of a (a = f * 2**ex with f in [0.5, 1)), floored at the
    # smallest normal binade 2^-6 so that subnormals share its step 2^-9
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, 1 - E4M3_BIAS)
    step = np.ldexp(1.0, e - 3)
    n = np.rint(a / step)                 # exact scaling; rint is half-to-even
    v = np.minimum(n * step, E4M3_MAX)    # rounded magnitude, saturated

    # magnitude -> fields
    _, ex2 = np.frexp(v)
    ev = ex2.astype(np.int64) - 1
    normal = v >= 2.0 ** (1 - E4M3_BIAS)
    field = np.where(normal, ev + E4M3_BIAS, 0)
    mant_n = np.ldexp(v, -np.where(normal, ev, 0)) * 8.0 - 8.0
    mant_s = np.ldexp(v, 9)
    mant = np.where(normal, mant_n, mant_s)
    mant = mant.astype(np.int64)
    code = (sign.astype(np.int64) << 7) | (field << 3) | mant
    return code.astype(np.uint8)


def f32_scale(amax):
    """s = fp32(amax / 448) (correctly rounded), amax == 0 -> 1."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    return float(np.float32(amax / E4M3_MAX))


def quant_per_tensor(v):
    """Per-tensor FP8 quantization of fp32-representable values v.

    Returns (codes uint8 same shape, scale s as a float holding an fp32,
    amax).  Dequantized value = e4m3_decode(code) * s.
    """
    v = np.asarray(v, dtype=np.float64)
    if v.size and not np.array_equal(v, v.astype(np.float32).astype(np.float64)):
        raise ValueError("quant_per_tensor expects fp32-representable input")
    amax = float(np.max(np.abs(v))) if v.size else 0.0
    s = f32_scale(amax)
    q = (v / s).astype(np.float32).astype(np.float64)
    return e4m3_encode(q), s, amax
