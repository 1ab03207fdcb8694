"""CPU oracle for the quantized-weight linear projection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this package: only the test suite, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP library (no kernels, no
headers, no tables, no helpers) and imports nothing from it.

The oracle is plain and slow on purpose: every format is decoded from its bit
definition into float64 (exact for every format here), every rounding step is
written out from the definition of round-to-nearest-even, sums run in float64
(integer group sums in int64) and no step is blocked, fused or reordered beyond
what the definition says.

Sources (the web pages this method is described on; cited by title and
section in every function):

  [MXFP8 card]      "Qwen3.8-27B "MXFP8-CRACK" — NInfer artifact", section
                    "How it was built" (MXFP8 packing, UE8M0 scale; MLX affine).
  [FP8 card]        "Qwen3.8-27B EfficientThink-Uncensored FP8 for NInfer",
                    introduction and "Conversion and verification" (block-wise
                    to per-row re-encode, error bound, FP8-activation routes).
  [NVFP4 card]      "Qwen3.8-27B-NVIDIA-NVFP4-NInferV3", "What is in the file"
                    and "How it was created" (row-scale FP8 e4m3fn, grouped
                    formats with FP16 scales, on-the-fly dequantization,
                    head re-encode, BF16 gate projections).
  [RTX5080 card]    "Qwen3.8-27B for NInfer — RTX 5080 16 GB, true 128K +
                    Vision", "Quantization profile" (Q3/Q4/Q5 G64 with FP16
                    scales), "At a glance" (prefill chunk 1792).
  [int8 card]       "Qwen3.8-27B, NInfer int8-prefill artifact for the RTX
                    4090", "What changes" (W8A8 prefill, 129-token threshold,
                    BF16 decode route) and "Measurements".

Parity status per function is listed in ``PARITY`` below; every function is
pinned by tests under ``tests/test_oracle_*.py`` against closed forms, exact
rational arithmetic, invariants or library routines, except where it says
"parity unpinned".
"""

from . import formats, method  # noqa: F401

PARITY = {
    "formats.e4m3_decode": "pinned: closed form for all 256 codes; torch float8_e4m3fn",
    "formats.ue8m0_decode": "pinned: closed form 2^(b-127)",
    "formats.bf16_decode": "pinned: closed form; torch bfloat16 view",
    "formats.f16_decode": "pinned: closed form; numpy float16 view",
    "formats.round_rne": "pinned: Fraction brute force; torch/numpy casts",
    "method.decode_mxfp8": "pinned: closed form, Fraction brute force",
    "method.decode_mlx_affine_int8": "pinned: hand values, ties and a single-rounding case, "
                                     "Fraction brute force with an independent rounding, NaN/Inf",
    "method.reencode_block128_to_row": "pinned: shared-scale invariant, max-code invariant, "
                                       "per-element half-ulp bound, Fraction brute force",
    "method.encode_fp8row": "pinned: as the re-encode (same row encoder)",
    "method.quantize_act_int8_g64": "pinned: closed-form ties, amax->127, Fraction brute force",
    "method.gemv_fp8row": "pinned: one-hot rows, Fraction brute force",
    "method.gemv_qgroup": "pinned: one-hot rows, Fraction brute force",
    "method.unpack_qbits": "pinned: hand-packed streams, bit-by-bit brute force with Python integers, "
                           "equality with the Q4 nibble layout at b = 4",
    "method.linear_qbits_g64": "pinned: route composition, group sums by integer brute force",
    "method.gemm_w8a8_g64": "pinned: int brute force, power-of-two exact case",
    "method.quantize_act_fp8_row": "parity unpinned with respect to the pages (they do not "
                                   "describe the FP8 activation quantizer); pinned to its own "
                                   "stated reading by Fraction brute force",
    "method.gemm_fp8row": "parity unpinned with respect to the pages (same reason); "
                          "pinned to its reading by Fraction brute force",
    "method.route": "pinned: the 129-token threshold; the A8 decode flag below it",
    "method.linear_q4g64": "pinned: route composition, group sums by nibble brute force",
    "method.linear_w8g64 (A8 decode)": "parity unpinned with respect to the pages (they name the A8 decode "
                                       "variant without details); pinned to its reading, the W8A8 "
                                       "arithmetic at decode sizes, by route composition and the W8A8 pins",
}
