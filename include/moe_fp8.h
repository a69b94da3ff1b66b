/*
 * moe_fp8.h -- C ABI of the block-scaled FP8 mixture-of-experts expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (vLLM PR #59128 "Skip padded work in block-FP8 DeepGemmExperts",
 * Purpose and SM100-on-B200 sections; TensorRT-LLM PR #21250 "Triton
 * FP8-activation MoE for decode-sized batches on Hopper", description):
 *
 *   moe_align          top-k routing -> per-expert contiguous rows, prefix-sum endpoints
 *   moe_act_quant      BF16 tokens -> FP8 E4M3 codes + one scale per 1x128 group
 *   moe_grouped_gemm_fp8  FP8 x FP8 grouped GEMM with 128x128 fp32 weight block
 *                      scales, visiting only tiles that hold live rows
 *   moe_silu_mul_quant SiLU(gate) * up, quantized to FP8 the same way (FC2 input)
 *   moe_topk_combine   top-k weighted sum of the expert outputs back to tokens, BF16
 *   moe_forward        all of the above on one stream
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device (or managed) memory owned by the
 *   caller. The library never allocates, frees or synchronizes; all work is
 *   enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *   call returns without waiting. Every call is capturable into a HIP graph.
 * - Arguments are validated on the host before anything is enqueued. On any
 *   error nothing is launched and nothing is written. A launch failure
 *   reported by the HIP runtime returns MOE_ERR_HIP.
 * - Matrices are row-major and densely packed unless stated otherwise.
 *   BF16 values are passed as uint16_t bit patterns; FP8 values are OCP E4M3
 *   ("E4M3FN": bias 7, max 448, no infinities) bytes.
 * - Activation scales are stored group-major: scale of row r, 128-wide group
 *   g lives at index g * ld + r, where ld is the row capacity of that buffer.
 *   MOE_SCALE_FP32 and MOE_SCALE_FP32_POW2 store float; MOE_SCALE_UE8M0
 *   stores one uint8_t biased exponent (scale = 2^(byte - 127)).
 * - The live token count may live on the device (`t_live_dev`, one int32),
 *   so a captured graph can replay with a different count. It is clamped to
 *   [0, t_cap]; NULL means t_cap.
 * - "Untouched": rows past the last expert endpoint, pad rows inside an
 *   expert segment (except row_to_pair, which marks them -1), and output rows
 *   of tokens t >= t_live are never written (vLLM PR #59128, SM100 on B200:
 *   untouched gaps; SM90 on H200: unused output capacity left untouched).
 */
#ifndef MOE_FP8_H_
#define MOE_FP8_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad size, null pointer, unknown enum value */
  MOE_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
  MOE_ERR_CAPACITY = 3,    /* row_cap (or a workspace) too small */
  MOE_ERR_HIP = 4          /* the HIP runtime reported an error */
} moe_status;

/* Activation scale formats (vLLM PR #59128, Purpose: packed UE8M0 on one
 * architecture, plain or power-of-two-rounded fp32 on the other; vLLM PR
 * #65794, Overview). Power-of-two rounding rounds up. */
typedef enum {
  MOE_SCALE_FP32 = 0,
  MOE_SCALE_FP32_POW2 = 1,
  MOE_SCALE_UE8M0 = 2
} moe_scale_fmt;

/* Rounding conventions of the FP8 quantizers.
 *   MOE_ROUND_DIVIDE      scale = max(fl32(amax / 448), fl32(1 / (448*512))),
 *                         codes from fl32(x / scale) (vLLM PR #65794, Details);
 *                         the SwiGLU output is quantized from float32.
 *   MOE_ROUND_RECIPROCAL  the fused CUTLASS op's convention that TensorRT-LLM
 *                         PR #21250 follows (rounding-fix commit message):
 *                         inv = fl32(448 / max(amax, 2^-9)), stored scale
 *                         fl32(1 / inv), codes from fl32(x * inv) (with a
 *                         power-of-two format: the stored scale rounded up to
 *                         a power of two, and x divided by it exactly); the
 *                         SwiGLU output is rounded to BF16 before it is
 *                         quantized. The 2^-9 floor (where the divide rule's
 *                         floor starts to bind) is this library's reading.
 * The grouped GEMM accumulates sa * sw * dot in fp32 either way; the review of
 * TensorRT-LLM PR #21250 (block-scale order) notes that forming sa * sw first
 * is that op's order, and the GEMM results match either convention within the
 * GEMM tolerance. */
typedef enum {
  MOE_ROUND_DIVIDE = 0,
  MOE_ROUND_RECIPROCAL = 1
} moe_rounding;

/* Gated activations (TensorRT-LLM PR #21250, Test Coverage: no clamp, clamp,
 * clamp after SiLU; vLLM PR #65794, Details: clamp_limit). With limit L:
 *   SWIGLU                   y = silu(g) * u
 *   SWIGLU_CLAMP             y = silu(min(g, L)) * clamp(u, -L, L)
 *   SWIGLU_CLAMP_AFTER_SILU  y = min(silu(g), L) * clamp(u, -L, L)          */
/* Expert weight formats.
 *   MOE_WEIGHT_E4M3   FP8 E4M3 codes [E, rows, cols] with float32 scales per
 *                     128x128 block [E, rows/128, cols/128] (vLLM PR #59128,
 *                     Purpose; TensorRT-LLM PR #21250, description).
 *   MOE_WEIGHT_MXFP4  FP4 weights (vLLM PR #59128's description names them;
 *                     the pages give no format, read here as OCP MXFP4):
 *                     E2M1 codes packed two per byte, [E, rows, cols/2], the
 *                     even column in the low nibble (magnitudes 0, 0.5, 1,
 *                     1.5, 2, 3, 4, 6; bit 3 the sign), and one E8M0 scale
 *                     byte b (2^(b-127); 255 is NaN) per 32 consecutive
 *                     columns, [E, rows, cols/32]. */
typedef enum {
  MOE_WEIGHT_E4M3 = 0,
  MOE_WEIGHT_MXFP4 = 1
} moe_weight_fmt;

typedef enum {
  MOE_ACT_SWIGLU = 0,
  MOE_ACT_SWIGLU_CLAMP = 1,
  MOE_ACT_SWIGLU_CLAMP_AFTER_SILU = 2
} moe_act;

/* Smallest row capacity that holds any routing of t_cap tokens with top-k:
 * with P = t_cap * topk pairs and n = min(num_experts, P) experts in use,
 * align_rows * floor((P + n * (align_rows - 1)) / align_rows). Returns -1 if
 * the arguments are invalid or the value overflows int32. */
int32_t moe_min_row_cap(int32_t t_cap, int32_t topk, int32_t num_experts, int32_t align_rows);

/* Routing alignment (vLLM PR #59128, Purpose: a shared permutation helper
 * produces the expert endpoints both GEMMs and the activation quantization
 * consume; TensorRT-LLM PR #21250, sequence diagram: padded expert blocks and
 * sorted token ids; review comment on expert parallelism: ids outside the
 * local range are dropped).
 *
 *   topk_ids      device int32 [t_cap, topk]; local ids id - expert_start
 *                 outside [0, num_experts) are dropped (their pair maps to
 *                 row -1)
 *   expert_start  the first expert this caller owns (expert parallelism:
 *                 TensorRT-LLM PR #21250, For MoE owners and review comment:
 *                 pairs of other ranks' experts are dropped, not clamped);
 *                 0 without expert parallelism
 *   t_live_dev    device int32 scalar or NULL (see conventions)
 *   align_rows    >= 1; each expert's row count is rounded up to a multiple
 *   row_cap       rows available; must be >= moe_min_row_cap(...)
 * Outputs (device int32):
 *   expert_counts [num_experts]      live pairs per expert
 *   expert_offsets[num_experts + 1]  exclusive prefix sum of the rounded-up
 *                                    counts; segment e = [off[e], off[e+1])
 *   row_to_pair   [row_cap]  pair index p = t*topk + k of each live row, in
 *                            ascending p within a segment; -1 on pad rows;
 *                            rows >= off[E] untouched
 *   pair_to_row   [t_cap*topk]  row of each pair of a live token, -1 when
 *                            dropped; entries of tokens >= t_live untouched
 * Errors: INVALID_ARG (sizes, null pointers), CAPACITY (row_cap too small). */
moe_status moe_align(const int32_t* topk_ids, int32_t t_cap, const int32_t* t_live_dev,
                     int32_t topk, int32_t num_experts, int32_t expert_start, int32_t align_rows,
                     int32_t row_cap, int32_t* expert_counts, int32_t* expert_offsets,
                     int32_t* row_to_pair, int32_t* pair_to_row, void* stream);

/* Routing into the batched masked-M layout (vLLM PR #65794, Details, batched
 * experts: a fixed capacity per expert with a per-expert valid count, the
 * layout persistent_masked_m_silu_mul_quant consumes): expert e owns rows
 * [e*expert_cap, (e+1)*expert_cap), the first masked_m[e] of which hold its
 * pairs in ascending pair order. Pairs ranked at or past the capacity are
 * dropped (pair_to_row -1) and counted: the pages leave the overflow open,
 * and this library's reading is to drop and report it.
 *
 *   topk_ids, t_cap, t_live_dev, topk, expert_start  as moe_align
 *   expert_cap    rows per expert, >= 1; num_experts * expert_cap <= 2^30
 * Outputs (device int32):
 *   masked_m      [num_experts]  min(pairs of expert e, expert_cap)
 *   row_to_pair   [num_experts * expert_cap]  pair of each live row; rows
 *                 past masked_m[e] of each expert untouched
 *   pair_to_row   [t_cap*topk]  as moe_align (-1 also for overflow)
 *   overflow      one int32 or NULL: the number of pairs dropped for capacity
 * Errors: INVALID_ARG, UNSUPPORTED (num_experts above 1024). */
moe_status moe_align_batched(const int32_t* topk_ids, int32_t t_cap, const int32_t* t_live_dev,
                             int32_t topk, int32_t num_experts, int32_t expert_start,
                             int32_t expert_cap, int32_t* masked_m, int32_t* row_to_pair,
                             int32_t* pair_to_row, int32_t* overflow, void* stream);

/* Per-1x128 FP8 E4M3 activation quantization of the live tokens (vLLM PR
 * #65794, Details: scale = max(amax / 448, 1 / (448 * 512)), then x / scale,
 * both IEEE float32 divisions, round to nearest even, saturating at 448;
 * TensorRT-LLM PR #21250, description: per-1x128 activation quantization).
 * Tokens are quantized once each; the FC1 GEMM gathers them through
 * row_to_pair, so routed copies are never materialized.
 *
 *   x     device BF16 [t_cap, hidden]
 *   xq    device uint8 [t_cap, hidden]; rows t >= t_live untouched
 *   xs    device scales [hidden/128][t_cap] (float or uint8, per `fmt`)
 *   rounding  the quantizer's convention (moe_rounding)
 * Errors: INVALID_ARG (hidden not a positive multiple of 128, null pointers,
 * unknown fmt or rounding). */
moe_status moe_act_quant(const uint16_t* x, int32_t t_cap, const int32_t* t_live_dev,
                         int32_t hidden, moe_scale_fmt fmt, moe_rounding rounding, uint8_t* xq,
                         void* xs, void* stream);

/* Grouped FP8 x FP8 GEMM with per-block scales, over the live rows of every
 * expert segment only (vLLM PR #59128, Purpose and SM90-on-H200: both grouped
 * GEMMs skip unused whole tiles through the prefix-sum endpoints; TensorRT-LLM
 * PR #21250, description: FP8 x FP8 GEMMs with 128x128 weight scales whose
 * grid covers only the expert blocks the batch occupies).
 *
 * For every expert e and live row r in [off[e], off[e] + counts[e]):
 *   C[r, n] = bf16( sum_kb sa[kb, ar] * ws[e, n/128, kb] * sum_{j<128} A[ar, kb*128+j] * W[e, n, kb*128+j] )
 * with ar = a_row_map ? a_row_map[r] / a_row_div : r, accumulated in fp32
 * and rounded to nearest even BF16.
 *
 *   a           device uint8 [a_rows, k]
 *   a_scales    device [k/128][a_rows] in format `fmt`
 *   a_row_map   device int32 [row_cap] or NULL (identity); entries read only
 *               for live rows; must satisfy 0 <= a_row_map[r]/a_row_div < a_rows
 *   w           device uint8 [num_experts, n, k]; w_scales float [num_experts, n/128, k/128]
 *   expert_counts/expert_offsets  as produced by moe_align (device)
 *   max_rows_per_expert  host-side bound on any counts[e] (0 = row_cap); it
 *               only selects which kernels are launched, never the result
 *   c           device BF16 [row_cap, n]; only live rows written
 *   tiles_visited  device int32 or NULL; when given, the number of
 *               (row tile, column tile) pairs computed is ADDED to it
 * Errors: INVALID_ARG (n or k not positive multiples of 128, null pointers,
 * a_row_div < 1, unknown fmt); UNSUPPORTED (num_experts above 1024, k above
 * 32768, a_rows * k or n * k at or above 2^32). */
moe_status moe_grouped_gemm_fp8(const uint8_t* a, const void* a_scales, moe_scale_fmt fmt,
                                int32_t a_rows, const int32_t* a_row_map, int32_t a_row_div,
                                const uint8_t* w, const float* w_scales,
                                const int32_t* expert_counts, const int32_t* expert_offsets,
                                int32_t num_experts, int32_t row_cap, int32_t max_rows_per_expert,
                                int32_t n, int32_t k, uint16_t* c, int32_t* tiles_visited,
                                void* stream);

/* moe_grouped_gemm_fp8 on the batched masked-M layout (see moe_align_batched;
 * vLLM PR #65794, Details, batched experts): expert e's live rows are
 * [e*expert_cap, e*expert_cap + min(masked_m[e], expert_cap)), and C is
 * [num_experts * expert_cap, n]; rows past the mask are untouched. Other
 * arguments and errors as moe_grouped_gemm_fp8, whose kernels it runs. */
moe_status moe_grouped_gemm_fp8_masked(const uint8_t* a, const void* a_scales, moe_scale_fmt fmt,
                                       int32_t a_rows, const int32_t* a_row_map, int32_t a_row_div,
                                       const uint8_t* w, const float* w_scales,
                                       const int32_t* masked_m, int32_t num_experts,
                                       int32_t expert_cap, int32_t n, int32_t k, uint16_t* c,
                                       int32_t* tiles_visited, void* stream);

/* Grouped GEMM with FP8 E4M3 activations and MXFP4 weights (vLLM PR #59128,
 * description: FP4 weights on the same prefix-sum expert endpoints; the
 * format is MOE_WEIGHT_MXFP4's). For every expert e and live row r:
 *   C[r, n] = bf16( sum_kb sa[kb, ar] * sum_{j<128} A[ar, kb*128+j] * w(e, n, kb*128+j) )
 *   w(e, n, k) = e2m1(code of column k of row n) * 2^(w_scales[e, n, k/32] - 127)
 * with ar as in moe_grouped_gemm_fp8, accumulated in fp32 (the weight scales
 * applied inside the matrix cores, the activation scale once per 128-wide
 * block; with UE8M0 activation scales the matrix cores apply both) and
 * rounded to nearest even BF16.
 *
 *   a, a_scales, fmt, a_rows, a_row_map, a_row_div   as moe_grouped_gemm_fp8
 *   w          device uint8 [num_experts, n, k/2] packed E2M1 codes
 *   w_scales   device uint8 [num_experts, n, k/32] E8M0 bytes
 *   expert_cap 0: the aligned layout, expert_counts/expert_offsets as
 *              moe_align produces them; > 0: the batched masked-M layout
 *              (expert_counts is masked_m, expert_offsets is not read, expert
 *              e's rows start at e*expert_cap, row_cap = num_experts*expert_cap)
 *   max_rows_per_expert  host-side bound on any counts[e] (0 = row_cap); it
 *              only selects which kernels are launched, never the result
 *   c          device BF16 [row_cap, n]; only live rows written
 * Errors: INVALID_ARG (n or k not positive multiples of 128, null pointers,
 * a_row_div < 1, unknown fmt, a_rows < 1 with rows to compute, a batched
 * row_cap other than num_experts*expert_cap, max_rows_per_expert < 0); UNSUPPORTED (num_experts above
 * 1024, a_rows * k or n * k at or above 2^32). */
moe_status moe_grouped_gemm_mxfp4(const uint8_t* a, const void* a_scales, moe_scale_fmt fmt,
                                  int32_t a_rows, const int32_t* a_row_map, int32_t a_row_div,
                                  const uint8_t* w, const uint8_t* w_scales,
                                  const int32_t* expert_counts, const int32_t* expert_offsets,
                                  int32_t expert_cap, int32_t num_experts, int32_t row_cap,
                                  int32_t max_rows_per_expert, int32_t n, int32_t k, uint16_t* c,
                                  void* stream);

/* Row-tile heights of the two GEMM kernels, for interpreting tiles_visited:
 * experts with at most MOE_GEMM_STREAM_MAX_ROWS live rows are computed by
 * the weight-streaming kernel in row tiles of MOE_GEMM_STREAM_TILE_M, larger
 * ones by the MFMA-tiled kernel in row tiles of MOE_GEMM_TILED_TILE_M; column
 * tiles are MOE_GEMM_COL_TILE wide in both. */
#define MOE_GEMM_STREAM_TILE_M 16
#define MOE_GEMM_STREAM_MAX_ROWS 64
#define MOE_GEMM_TILED_TILE_M 256
#define MOE_GEMM_COL_TILE 128

/* Fused SiLU(gate) * up + 1x128 FP8 quantization of the FC2 input, over live
 * rows only (vLLM PR #59128, Purpose: the fused activation quantization
 * consumes the live expert endpoints; vLLM PR #65794, Details: fp32
 * SiLU * up without an intermediate BF16 rounding, then the quantization
 * rule above, with use_ue8m0 and clamp_limit options).
 * Gate is columns [0, inter) of each row, up is [inter, 2*inter). SiLU and
 * the product are evaluated in double precision and rounded once to float.
 *
 *   gate_up  device BF16 [row_cap, 2*inter]
 *   hq       device uint8 [row_cap, inter]; hs device [inter/128][row_cap]
 *   clamp_limit  used by the clamp variants; must be > 0 there
 *   rounding  moe_rounding; MOE_ROUND_RECIPROCAL rounds SiLU(gate)*up to BF16
 *             before quantizing it
 * Errors: INVALID_ARG (also when row_cap * inter / 128 exceeds 2^31 - 1). */
moe_status moe_silu_mul_quant(const uint16_t* gate_up, int32_t inter,
                              const int32_t* expert_counts, const int32_t* expert_offsets,
                              int32_t num_experts, int32_t row_cap, moe_act act,
                              float clamp_limit, moe_scale_fmt fmt, moe_rounding rounding,
                              uint8_t* hq, void* hs, void* stream);

/* moe_silu_mul_quant on the batched masked-M layout (vLLM PR #65794,
 * Details: persistent_masked_m_silu_mul_quant): gate_up is
 * [num_experts * expert_cap, 2*inter], hq [num_experts * expert_cap, inter],
 * hs [inter/128][num_experts * expert_cap]; only the first masked_m[e] rows
 * of each expert are read and written. Errors as moe_silu_mul_quant. */
moe_status moe_silu_mul_quant_masked(const uint16_t* gate_up, int32_t inter,
                                     const int32_t* masked_m, int32_t num_experts,
                                     int32_t expert_cap, moe_act act, float clamp_limit,
                                     moe_scale_fmt fmt, moe_rounding rounding, uint8_t* hq,
                                     void* hs, void* stream);

/* Top-k weighted unpermute/sum (TensorRT-LLM PR #21250, rounding-fix commit:
 * the routing weights scale the BF16 expert outputs in fp32 in the top-k sum,
 * not the FC2 accumulators). For each live token t:
 *   out[t, :] = bf16( sum over k ascending with pair_to_row[t*topk+k] in
 *                     [0, row_cap) of topk_w[t, k] * y[row, :] )
 * accumulated in fp32; a token with no valid pair gets zeros.
 *
 *   y        device BF16 [row_cap, hidden]; pair_to_row device int32 [t_cap*topk]
 *   topk_w   device float [t_cap, topk]
 *   out      device BF16 [t_cap, hidden]; rows t >= t_live untouched
 * Errors: INVALID_ARG. */
moe_status moe_topk_combine(const uint16_t* y, int32_t row_cap, const int32_t* pair_to_row,
                            const float* topk_w, int32_t t_cap, const int32_t* t_live_dev,
                            int32_t topk, int32_t hidden, uint16_t* out, void* stream);

/* ---- whole layer ---------------------------------------------------------- */

typedef struct {
  int32_t num_experts;
  int32_t hidden;       /* H, multiple of 128 */
  int32_t inter;        /* I, multiple of 128 */
  int32_t topk;
  int32_t t_cap;        /* token capacity */
  int32_t align_rows;   /* per-expert row alignment, >= 1 */
  int32_t row_cap;      /* 0 = moe_min_row_cap(t_cap, topk, num_experts, align_rows) */
  moe_scale_fmt scale_fmt;
  moe_act act;
  float clamp_limit;
  moe_rounding rounding; /* quantizer convention of both activation quantizations */
  int32_t expert_start;  /* first expert owned (local id = id - expert_start), see moe_align */
  int32_t expert_cap;    /* 0: the aligned layout; > 0: the batched masked-M layout with this
                            many rows per expert (row_cap is then 0 or num_experts *
                            expert_cap, align_rows is unused, and the decode path's
                            fused schedules do not apply) */
  moe_weight_fmt weight_fmt; /* format of w1/w2 and their scales. MXFP4 weights take the
                                one-launch decode layer where it applies and H and I are
                                multiples of 256 (a weight stage is two 128-wide K blocks),
                                otherwise the general six-launch schedule with
                                moe_grouped_gemm_mxfp4 as both GEMMs; the decode path's
                                other fused schedules and moe_fc1_decode are FP8-only */
} moe_problem;

typedef struct {
  const uint16_t* x;          /* BF16 [t_cap, H] */
  const int32_t* topk_ids;    /* [t_cap, topk] */
  const float* topk_w;        /* [t_cap, topk] */
  const int32_t* t_live_dev;  /* scalar or NULL */
  const uint8_t* w1;          /* [E, 2I, H] (MXFP4: [E, 2I, H/2]): gate rows [0, I), up rows [I, 2I) */
  const void* w1_scales;      /* float [E, 2I/128, H/128] (MXFP4: E8M0 bytes [E, 2I, H/32]) */
  const uint8_t* w2;          /* [E, H, I] (MXFP4: [E, H, I/2]) */
  const void* w2_scales;      /* float [E, H/128, I/128] (MXFP4: E8M0 bytes [E, H, I/32]) */
  uint16_t* out;              /* BF16 [t_cap, H]; rows >= t_live untouched */
} moe_tensors;

/* Byte offsets of the intermediates inside the forward workspace (each
 * 256-byte aligned), so callers and tests can inspect them. */
typedef struct {
  size_t expert_counts;  /* int32 [E] */
  size_t expert_offsets; /* int32 [E+1] */
  size_t row_to_pair;    /* int32 [row_cap] */
  size_t pair_to_row;    /* int32 [t_cap*topk] */
  size_t xq;             /* uint8 [t_cap, H] */
  size_t xs;             /* scales [H/128][t_cap] */
  size_t c1;             /* BF16 [row_cap, 2I] */
  size_t hq;             /* uint8 [row_cap, I] */
  size_t hs;             /* scales [I/128][row_cap] */
  size_t y;              /* BF16 [row_cap, H] */
  size_t act;            /* fp32 [row_cap, I] SiLU(gate)*up before quantization; laid out
                            only on the decode path (t_cap*topk <= 64 and the quantized
                            FC2 input rows fit 24 KiB of LDS), else equal to status */
  size_t status;         /* int32 [1024] per-launch outcome of the one-launch decode
                            layer's grid barrier: every launch of that path writes slot b
                            for each of its workgroups b < grid (one per CU): 0 = the
                            barrier opened, 1 = a wait gave up (see moe_barrier_timeouts)
                            and workgroup b wrote NaN (0x7FC0) to its output columns
                            16*(b + grid*j) .. +15 of the live tokens instead of computing
                            them. Other paths do not write it. */
  size_t overflow;       /* int32: pairs dropped for capacity (batched layout only) */
  size_t total;          /* bytes required */
  int32_t row_cap;       /* effective row capacity */
} moe_workspace_layout;

/* Fills `layout` for problem `p`. Errors: INVALID_ARG, CAPACITY, UNSUPPORTED
 * (num_experts above 1024, or a GEMM shape beyond moe_grouped_gemm_fp8's
 * limits). */
moe_status moe_workspace_plan(const moe_problem* p, moe_workspace_layout* layout);

/* Bytes of workspace moe_forward needs for `p` (0 if `p` is invalid). */
size_t moe_workspace_bytes(const moe_problem* p);

/* Limits of moe_forward's decode path and of its one-launch form, on
 * P = t_cap*topk routed pairs of capacity: the decode path needs
 * P <= MOE_DECODE_MAX_PAIRS, P*(I+16) <= MOE_DECODE_FC2_ROW_BYTES and
 * P*I/128 <= MOE_DECODE_FC2_MAX_SCALES (the quantized FC2 input rows in
 * LDS); the one launch also needs t_cap*(H+16) <= MOE_DECODE_LAYER_TOKEN_BYTES,
 * t_cap*H/128 <= MOE_DECODE_LAYER_MAX_SCALES (all tokens' codes and scales in
 * LDS) and H a multiple of 16 (with MXFP4 weights H and I multiples of 256,
 * and the decode path is then the one launch alone). moe_fc1_decode's token
 * limits are 24576 bytes and 256 scales. */
#define MOE_DECODE_MAX_PAIRS 64
#define MOE_DECODE_FC2_ROW_BYTES 24576
#define MOE_DECODE_FC2_MAX_SCALES 256
#define MOE_DECODE_LAYER_TOKEN_BYTES 61440
#define MOE_DECODE_LAYER_MAX_SCALES 512

/* The whole expert layer: align -> act_quant -> FC1 -> silu_mul_quant -> FC2
 * -> topk_combine, enqueued on one stream with no host synchronization
 * (vLLM PR #59128, SM100 on B200: the full-expert benchmark scope; the layer
 * replays inside a captured graph with the token count on the device).
 * On the decode path (see moe_workspace_layout.act) the launches are fewer
 * (TensorRT-LLM PR #21250, description: at decode sizes each launch's fixed
 * cost counts). Within the one-launch limits above (MOE_DECODE_LAYER_*),
 * the layer is ONE launch: one workgroup per CU runs routing, activation
 * quantization and FC1 with SiLU(gate)*up, meets the others at a barrier
 * across the grid, then runs FC2 with the top-k combine for its output
 * columns (beyond moe_fc1_decode's token limits, with a 4-deep instead of a
 * 6-deep weight ring per wave). That launch needs all its workgroups
 * resident at once and keeps its barrier epochs in device globals, so on
 * that path moe_forward drops thread safety across overlapping calls: calls
 * on one device must not overlap in time (one stream, or ordered streams),
 * and the GPU should not be shared with work that holds CUs for long. A
 * barrier wait that gives up never hangs the launch; it is reported in the
 * workspace's status slots and as NaN output columns (see
 * moe_barrier_timeouts). Every other path keeps no state between calls.
 * Otherwise the decode path takes two or three
 * launches: [align + act_quant, then FC1 with SiLU(gate)*up] or the fused
 * FC1 of moe_fc1_decode, then FC2 with the top-k combine. The workspace then
 * holds the same alignment, codes and scales, bit for bit, and FC1/FC2 rows
 * within the GEMM tolerance.
 * `workspace` is device memory of at least moe_workspace_bytes(p) bytes, laid
 * out as moe_workspace_plan describes; its prior contents do not matter.
 * Errors: INVALID_ARG, CAPACITY (workspace or row_cap too small), HIP. */
moe_status moe_forward(const moe_problem* p, const moe_tensors* t, void* workspace,
                       size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * layer as moe_forward computes it, with the workspace taken from a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library instead of a
 * caller buffer. The array exists once per device (its address is looked up
 * on the first call on that device, with that device current) and is held
 * until the process ends. Nothing is allocated or freed by any call.
 * The caller still passes all inputs and `t->out`. The workspace layout is
 * moe_workspace_plan's; the array keeps the last call's contents, and since
 * moe_forward does not depend on prior workspace contents nothing needs
 * clearing. Every call on one device shares that device's array, so calls on
 * one device that overlap in time (different streams without ordering, or
 * several host threads) race and give wrong results; order them.
 * Errors: as moe_forward, and CAPACITY when moe_workspace_bytes(p) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB: every decode-sized problem of the
 * one-launch path, the tiny layer, and general-path layers up to about
 * 64 tokens of the 256-expert sweep shape), HIP if the array's address
 * cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES 67108864
moe_status moe_forward_noalloc(const moe_problem* p, const moe_tensors* t, void* stream);

/* The first launch of moe_forward's decode path, on its own: routing
 * alignment, activation quantization and FC1 with SiLU(gate)*up in one
 * kernel (vLLM PR #59128, Purpose; vLLM PR #65794, Details; TensorRT-LLM
 * PR #21250, For MoE owners). It exists so that the kernel can be timed and
 * tested alone. It applies when the problem takes the decode path
 * (moe_workspace_layout.act laid out) and all t_cap tokens' codes fit 24 KiB
 * of LDS at a row stride of H+16 bytes, with t_cap*H/128 <= 256.
 * It writes, bit for bit as moe_align and moe_act_quant would:
 * expert_counts, expert_offsets, row_to_pair, pair_to_row, xq and xs. It
 * also writes c1 for the live rows and act (fp32 SiLU(gate)*up). The arguments
 * are those of moe_forward: t->w2, t->w2_scales, t->topk_w and t->out are
 * not read. FP8 weights only (UNSUPPORTED for MXFP4).
 * Errors: UNSUPPORTED (not such a problem), INVALID_ARG, CAPACITY, HIP. */
moe_status moe_fc1_decode(const moe_problem* p, const moe_tensors* t, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Number of waits at the grid barrier of moe_forward's one-launch decode
 * path that gave up on the current device since the library was loaded
 * (sticky). A wait gives up after about two seconds without the other
 * workgroups, which only happens when some of them could not become resident
 * (CUs held by other work). The launch then still finishes: every workgroup
 * that gave up, or whose release carried the failure mark, writes NaN to its
 * output columns and 1 to its slot of moe_workspace_layout.status, so the
 * failure is visible in that launch's own outputs without a host poll. This
 * call reads device memory synchronously.
 * Errors: INVALID_ARG (count NULL), HIP. */
moe_status moe_barrier_timeouts(uint32_t* count);

/* Sets how many polls (about a microsecond each) a wait at the one-launch
 * decode layer's grid barrier makes before it gives up, for launches enqueued
 * after the call, process-wide; returns the previous value. Default 2^21.
 * A negative value makes every wait give up at once: a host-forced timeout,
 * so that tests can exercise the failure report above while every kernel
 * still exits normally. Not thread-safe against concurrent launches. */
int32_t moe_barrier_spin_limit(int32_t polls);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H_ */
