"""Plain CPU oracle for layerwise QK-Norm.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. It
shares no code with the HIP library (no kernels, headers, helpers, tables or
constants); the only thing both sides consume is the seeded input data.

What it computes, and where that comes from
-------------------------------------------
Source: "SwiftQK: Fast and Communication-Efficient Tensor Parallelism for
Query-Key Normalization" (Kim, Han, Kim; arXiv 2608.09160v1), the arXiv HTML
page of the paper.

* RMS-Norm, Eq. 1 (the equation body is missing from the page text; the
  reading used everywhere here is ``y = x * gamma / sqrt(sum(x**2)/H + eps)``,
  with eps inside the square root and H the full projected width).
* Phase A: each shard contributes the plain sum of squares of its columns; the
  global statistic is the sum of those partial sums.
* Phase B and the final scaling: the shard is multiplied by gamma and then by
  the global RMS factor.
* Introduction: headwise QK-Norm (an extension beyond the layerwise path)
  computes an independent factor per attention head: Eq. 1 applied to every
  head vector with H = head_dim.
* Fig. 2(b): the precision study compares against an FP64 RMSNorm over the
  full vector, which is what this oracle is (every step in float64).

All arithmetic is float64. bf16 and FP8 E4M3 inputs are decoded exactly;
bf16 and FP8 outputs are rounded once, from the float64 result, to the nearest
representable value (ties to even; FP8 saturates to +-448). With FP8 rows,
gamma is bf16 (Fig. 2(b) evaluates FP8-E4M3 activations with FP32
accumulation; the weight format is not stated, bf16 is the reading taken).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
invariants, a library special case (``torch.nn.functional.rms_norm`` in fp64),
exact rational brute force and the hand-worked examples in ``tests/golden/``.
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits  # noqa: F401
from .fp8 import f64_to_fp8_bits, fp8_bits_to_f64  # noqa: F401
from .qknorm import (  # noqa: F401
    decode_input,
    shard_sum_of_squares,
    combine_partials,
    rms_denominator,
    scale_rows,
    layerwise_rmsnorm,
    apply_with_stats,
    qknorm_fused,
    qknorm_partial_stats,
    qknorm_apply_with_stats,
    headwise_rmsnorm,
    qknorm_headwise,
)
