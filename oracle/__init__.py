"""Plain CPU oracle for block-scaled quantize-then-GEMM (MXFP8, MXFP4, NVFP4).

TEST INFRASTRUCTURE ONLY. This package is imported by the tests, by the
smoke check in ``__graft_entry__`` and by the ``cpu_baseline`` leg of
``bench.py``; nothing on the product path may import, call or execute it.
It shares no code with the HIP library: it works on bf16 bit patterns with
float64 / exact arithmetic, one obvious step at a time.

Sources (the pages this follows):
  * lightly-train README "DINOv3 + EoMT on RTX 5090", section 2 (number
    formats table): MXFP8 = E4M3 elements with a UE8M0 scale per 1x32,
    MXFP4 = E2M1 elements with a UE8M0 scale per 1x32, NVFP4 = E2M1 elements
    with an E4M3 scale per 1x16 plus an fp32 per-tensor scale.
  * same README, section 5.5 (how the FP4 path works): all GEMMs are TN
    (both operands K-major); the weight-gradient GEMM needs a copy
    quantized along the token axis and stored transposed.
  * "2x, not 16x: the real ledger of BF16 mixed precision", section 2
    (format table: bf16 = 8 exponent bits, 7 mantissa bits) and section 5.4
    (the largest E4M3 value is 448).

Where the pages are silent (shared-exponent formula, rounding, saturation,
sign of zero, nibble order, layouts, NVFP4 scale arithmetic) the oracle
takes one stated reading; each is listed in the module that applies it.

Modules:
  formats   bf16 decode/round, E4M3 and E2M1 grids, RNE+saturate encoders
  quantize  block amax, shared exponent / block scale, element codes,
            packing, row and transposed (column) axis, dequantization
  gemm      exact dequantized float64 GEMM, the error scale S, acceptance
"""
