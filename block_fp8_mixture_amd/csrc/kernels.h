// Host-side launchers of the gfx950 kernels (internal to libmoefp8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;     // LDS tables in align and the GEMM schedulers
constexpr int kStreamTileM = 16;      // row tile of the weight-streaming GEMM
constexpr int kStreamMaxRows = 64;    // experts with at most this many rows stream
constexpr int kTiledTileM = 256;      // row tile of the MFMA-tiled GEMM
constexpr int kColTile = 128;         // column tile (= weight block rows)

hipError_t launch_align(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                        int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                        int32_t* row_to_pair, int32_t* pair_to_row, hipStream_t stream);

// moe_align and moe_act_quant of one layer in a single launch.
hipError_t launch_prep(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                       int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                       int32_t* row_to_pair, int32_t* pair_to_row, const uint16_t* x, int hidden,
                       int fmt, uint8_t* xq, void* xs, hipStream_t stream);

hipError_t launch_act_quant(const uint16_t* x, int t_cap, const int32_t* t_live_dev, int hidden,
                            int fmt, uint8_t* xq, void* xs, hipStream_t stream);

hipError_t launch_silu_mul_quant(const uint16_t* gate_up, int inter, const int32_t* counts,
                                 const int32_t* offsets, int num_experts, int row_cap, int act,
                                 float clamp_limit, int fmt, uint8_t* hq, void* hs,
                                 hipStream_t stream);

hipError_t launch_topk_combine(const uint16_t* y, int row_cap, const int32_t* pair_to_row,
                               const float* topk_w, int t_cap, const int32_t* t_live_dev,
                               int topk, int hidden, uint16_t* out, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a;
  const void* a_scales;
  int fmt;
  int a_rows;             // leading dimension of a_scales
  const int32_t* a_row_map;
  int a_row_div;
  const uint8_t* w;
  const float* w_scales;
  const int32_t* counts;
  const int32_t* offsets;
  int num_experts;
  int row_cap;
  int max_rows_per_expert;  // host bound on counts[e]
  int max_live_experts;     // host bound on experts with rows
  int n;
  int k;
  uint16_t* c;
  int32_t* tiles_visited;
};

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t stream);

int device_cu_count();

}  // namespace moe
