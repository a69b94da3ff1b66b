"""CPU oracle for the block-scaled FP8 mixture-of-experts expert layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, tables or
constants with the HIP library under ``block_fp8_mixture_amd/``.

The oracle is deliberately plain and slow: numpy, fp64 wherever the pages
leave precision open, exact integer arithmetic for the FP8 codec, and one
BLAS matmul per 128-wide K block as the only library primitive in the GEMM.

Sources (three web pages, cited by title and section):

* vLLM PR #59128 "Skip padded work in block-FP8 DeepGemmExperts" --
  Purpose; SM100 on B200; SM90 on H200.
* vLLM PR #65794 (per-layer activation-scale format, fused SiLU+quant) --
  Overview; Claims; Details (fused-kernel and sorted-A bullets).
* vLLM PR #59128's description names FP4 weights (prefix sums on SM10.x);
  their format is read as OCP MXFP4 (``fp_formats``).
* TensorRT-LLM PR #21250 "Triton FP8-activation MoE for decode-sized
  batches on Hopper" -- description; rounding-fix commit message (the
  ``reciprocal`` rounding convention); review comments on expert-parallel
  ids and block-scale order.

Pins (tests/test_oracle_*.py) tie every function here to something other
than itself: closed forms, exhaustive codec checks, exact rational
arithmetic, high-precision SiLU, brute force on tiny inputs. Every function
is pinned; none is "parity unpinned". The clamp variants of the SwiGLU are
pinned only against their own defining formula plus invariants, because the
pages name the variants without giving a formula (see ``moe.swiglu``).
"""

from .fp_formats import (E4M3_MAX, bf16_bits_to_f64, bf16_from_f64, e2m1_decode,
                         e4m3_decode, e4m3_encode, e8m0_decode, fp4_unpack)
from .quant import (ROUNDINGS, SCALE_FMTS, group_scales, quantize_groups,
                    reciprocal_multiplier, scales_to_f64)
from .align import align, align_batched
from .moe import (ACTS, MX_BLOCK, WEIGHT_FMTS, combine, forward, gemm_rows_mxfp4,
                  grouped_gemm, mxfp4_dequant, silu_mul_quant, swiglu, token_forward,
                  unquantized_reference)

__all__ = [
    "E4M3_MAX", "bf16_bits_to_f64", "bf16_from_f64", "e2m1_decode", "e4m3_decode",
    "e4m3_encode", "e8m0_decode", "fp4_unpack", "MX_BLOCK", "WEIGHT_FMTS", "gemm_rows_mxfp4",
    "mxfp4_dequant", "ROUNDINGS", "SCALE_FMTS", "group_scales", "quantize_groups",
    "reciprocal_multiplier",
    "scales_to_f64", "align", "align_batched", "ACTS", "combine", "forward", "grouped_gemm",
    "silu_mul_quant", "swiglu", "token_forward", "unquantized_reference",
]
