"""Block-scaled FP8 mixture-of-experts expert layer for AMD MI355X (gfx950).

Thin Python binding over ``libmoefp8.so`` (the C ABI declared in
``include/moe_fp8.h``). Every function here marshals torch tensors into
pointers and sizes and calls the library function of the same name; all
arithmetic runs in the library's HIP kernels. Output tensors are allocated
with torch when the caller does not pass them. Work is enqueued on torch's
current stream and nothing synchronizes.

The library must be built (``python -m block_fp8_mixture_amd.build``); if it
is missing, importing the binding's functions raises -- there is no fallback.
"""

from ._binding import (ACTS, DECODE_LIMITS, GEMM_TILES, NOALLOC_SCRATCH_BYTES, ROUNDINGS, SCALE_FMTS,
                       WEIGHT_FMTS, MoeError,
                       decode_layer_applies, library_path, load_library, moe_act_quant,
                       moe_align, moe_align_batched, moe_barrier_spin_limit, moe_barrier_timeouts, moe_fc1_decode,
                       moe_forward, moe_forward_noalloc, moe_grouped_gemm_fp8,
                       moe_grouped_gemm_fp8_masked, moe_grouped_gemm_mxfp4, moe_silu_mul_quant_masked, moe_min_row_cap, moe_silu_mul_quant,
                       moe_status_string, moe_topk_combine, moe_workspace_bytes,
                       moe_workspace_plan)

__all__ = [
    "ACTS", "DECODE_LIMITS", "GEMM_TILES", "NOALLOC_SCRATCH_BYTES", "ROUNDINGS", "SCALE_FMTS",
    "WEIGHT_FMTS", "MoeError", "decode_layer_applies",
    "library_path", "load_library", "moe_act_quant", "moe_align", "moe_align_batched", "moe_barrier_spin_limit",
    "moe_barrier_timeouts", "moe_fc1_decode", "moe_forward", "moe_forward_noalloc",
    "moe_grouped_gemm_fp8", "moe_grouped_gemm_fp8_masked", "moe_grouped_gemm_mxfp4",
    "moe_silu_mul_quant_masked",
    "moe_min_row_cap", "moe_silu_mul_quant", "moe_status_string", "moe_topk_combine",
    "moe_workspace_bytes", "moe_workspace_plan",
]
