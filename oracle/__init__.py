"""CPU oracle for the quantized Mixture-of-Experts grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants) and it imports
nothing from ``quantized_moe_grouped_top_amd``.

What it computes, in the order the hot path runs:

* ``formats``   - exact decode/encode of the number formats: OCP e4m3 (E4M3FN),
                  e8m0 power-of-two scales, bf16 round-to-nearest-even, int8.
* ``moe``       - top-k routing, block alignment, activation and weight
                  quantization (fp8 per tensor, int8 per channel, MXFP8 per 32),
                  the grouped GEMM with its scale / router-weight epilogue, and
                  the per-token combine.

Everything is plain numpy.  Floating-point work runs in float64 except where a
step rounds to float32 on purpose because the method defines that rounding
(the quantization scales and the scaled values handed to the fp8 encoder, the
combine, the bf16 output), so that both sides take every integer decision
(a quantized code, an expert choice) in the same precision.

Every function cites the passage of the source pages it follows; readings of
what the pages leave open are stated where they are made.  The pages are:

* "Tianxing/moe quantization" (ROCm Triton pull request): FP8_W8A8 and
  INT8_W8A16 benchmark tables over (M, K, N, E, top_k).
* "Enabling MOE Quantization using linear decomposition" (pytorch/ao pull
  request), Summary: the grouped GEMM as a sequence of per-expert linear ops.
* "[PyTorch] Let GroupedLinear accept MXFP8 input and gradient"
  (TransformerEngine pull request): MXFP8 data + e8m0 scales and the padding of
  each expert's rowwise scales to 128 rows.
* "INT8 quantization support" (AutoAWQ issue): int8 weights used with 16-bit
  activations.

Parity status of every function is listed in the pins of ``tests/``; the
page-1 throughput tables pin only the flop/byte accounting, never outputs.
"""

from . import formats, moe  # noqa: F401
