"""Seeded synthetic inputs for the FP8 expert layer.

This module is shared by the oracle tests, the GPU tests and the benchmark,
and holds none of the layer's own arithmetic: it draws activations, router
logits and weights, turns logits into top-k routing (the router is upstream
of the layer), and produces FP8 weight checkpoints (and MXFP4 ones, drawn
directly as codes and scale bytes). Weight quantization here
stands in for the checkpoint producer; it uses torch's float8_e4m3fn cast, a
library routine, and never the layer's activation quantizer.

Workloads (sizes from the pages' benchmarks and tests):

* ``tiny``    -- 4 experts, hidden 256, intermediate 128, top-2, 8 tokens,
  16 rows of capacity per expert (TensorRT-LLM PR #21250, Test Coverage:
  1 to 24 tokens, small shapes).
* ``decode``  -- 288 experts, top-8, hidden 4096, intermediate 512, 1 and 4
  tokens (TensorRT-LLM PR #21250, Performance).
* ``padded``  -- 32 experts, hidden 7168, intermediate 2048, top-8, a
  512-token workspace with 16 live tokens (vLLM PR #59128, SM100 on B200).
* ``full``    -- same shape, 4096 of 4096 tokens live (same section).
* ``sweep``   -- 256 experts, hidden 6144, intermediate 256, top-8,
  M = 1 ... 4096 tokens with Zipf-skewed routing (vLLM PR #65794,
  Validation, GLM-5.3 TP8 shape table).
"""

from .configs import CONFIGS, Workload, get
from .gen import (ExpertWeights, ExpertWeightsMxfp4, make_routing, make_tokens,
                  make_workload, quantize_weight_blocks)

__all__ = ["CONFIGS", "Workload", "get", "ExpertWeights", "ExpertWeightsMxfp4", "make_routing",
           "make_tokens", "make_workload", "quantize_weight_blocks"]
