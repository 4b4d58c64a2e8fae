"""Parity tolerances of the GPU tests against the fp64 oracle.

Outputs (the stated bar): fp32 inputs max |gpu - ref| <= 1e-5; bf16 inputs
(and an fp8 cache, whose values widen exactly to bf16) |gpu - ref| <=
2e-2 + 1e-2 |ref| elementwise.

Log-sum-exp (an extra fp32 output the pages do not define, so its bound is
derived from the kernels' arithmetic): the bf16 kernels round every softmax
weight to bfloat16 before it enters the matrix cores and normalise with the
sum of those same rounded weights, so that the output is an exact convex
combination of the value rows it multiplies.  Rounding to nearest in
bfloat16 (8 significant bits) moves each weight by at most 2^-8 of itself,
so the normaliser by at most 2^-8 of the true one and its log by at most
ln(1 + 2^-8) = 3.90e-3; the fp32 score and accumulation errors add orders of
magnitude less.  Hence atol 4e-3 (plus rtol 1e-4) for the bf16 and fp8
kernels.  The fp32 kernel keeps fp32 weights: atol 1e-5.
"""

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL = 1e-5
LSE_ATOL = 4e-3       # bf16 / fp8 kernels: ln(1 + 2^-8) rounded up
LSE_ATOL_F32 = 1e-5
