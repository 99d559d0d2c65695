"""CPU oracle for the block-scaled FP4 MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The library path
(the HIP kernels behind the C ABI and its Python binding) never calls it and
shares no code with it.

Plain float64 numpy, written from the model cards on block_scaled_fp4_nvfp4
and from the definitions of the E2M1, E4M3 and UE8M0 number formats:
  formats  - exact codecs of E2M1, E4M3 (FN), UE8M0 and bfloat16
  quant    - NVFP4 / MXFP4 quantizers with the per-block 4/6 scale choice,
             MXFP8 and block-FP8 quantizers, dequantizers
  moe      - top-k permutation and the routed-expert FFN
             (dequantize-then-matmul in float64)

Every function cites the card passage it follows.  Where the cards are
silent the reading adopted is stated at the function.  All functions have
pins in tests/ that do not reuse this code.
"""
