"""CPU oracle for the MXFP4 block-scaled MoE layer and dense projections.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library; the two meet only through the seeded input
arrays of ``synth``.

Everything is plain numpy in float64 (fp32 only where a step is defined in
fp32: the fp8 scale and the value divided by it).  Each function cites the
passage of the source pages it follows; "gpt-oss page" means the blog post
"GPT-OSS-120B on DGX Spark: From MXFP4 to NVFP4 - A Deep-Dive Benchmark",
"spark-vllm page" the README "GPT-OSS-120B with MXFP4 on DGX Spark
(SM121/GB10)" and "gptoss-spark page" the landing page "gptoss-spark".

Pins (see tests/test_oracle_*.py):
  * e2m1 / e8m0 / unpack / dequant: closed forms against the value set the
    gpt-oss page prints, nibble round trips, exact powers of two;
  * fp8 e4m3: exhaustive nearest-code search over all bf16 inputs;
  * route_topk: brute-force full sort;
  * quantize_mxfp4: hand-derived rounding cases (tests/golden), exact round
    trips of representable blocks, the scale rule's closed form, the error
    bound of round-to-nearest;
  * dequant_nvfp4: reduces to the MXFP4 dequant when the scales are powers
    of two shared by block pairs and the global scale is 1; the E4M3 scale
    grid (8 mantissa steps per binade, range) against the gpt-oss page's
    MXFP4/NVFP4 property table;
  * moe_forward / linear: exact rational (fractions.Fraction) brute force on
    tiny shapes (all three activation modes; the MXFP4-activation brute force
    has its own block quantiser), reductions E=1/k=1 to the dense linear,
    identical experts, MXFP4-representable activations passing through the
    MXFP4-activation mode unchanged.
  Values at the full layer shapes are "parity unpinned" by the pages: they
  print no output of any layer; only the functions above are pinned.
"""

from . import fp8, moe, mxfp4, nvfp4, quant  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode, quant_per_tensor  # noqa: F401
from .moe import (ACT_BF16, ACT_FP8_E4M3, ACT_MXFP4, linear, linear_rows,  # noqa: F401
                  moe_forward, moe_forward_routed, permute, route_topk,
                  swiglu)
from .mxfp4 import (E2M1_TABLE, bf16_bits_to_f64, dequant,  # noqa: F401
                    e2m1_value, e8m0_scale, pack_nibbles, unpack_nibbles)
from .nvfp4 import dequant_nvfp4, unpack_nibbles16  # noqa: F401
from .quant import quantize_mxfp4  # noqa: F401

__all__ = [
    "fp8", "moe", "mxfp4", "e4m3_decode", "e4m3_encode", "quant_per_tensor",
    "ACT_BF16", "ACT_FP8_E4M3", "ACT_MXFP4", "linear", "linear_rows", "moe_forward", "moe_forward_routed", "permute", "route_topk", "swiglu", "E2M1_TABLE",
    "bf16_bits_to_f64", "dequant", "e2m1_value", "e8m0_scale",
    "pack_nibbles", "unpack_nibbles", "quant", "quantize_mxfp4", "nvfp4", "dequant_nvfp4",
    "unpack_nibbles16",
]
