// Top-k weighted unpermute/sum back to token order, BF16 out.
//
// TensorRT-LLM PR #21250 (rounding-fix commit): the routing weights scale the
// BF16 expert outputs in fp32 inside the top-k sum, not the FC2 accumulators.
// Terms are added in ascending k; dropped pairs (row -1) contribute nothing.
//
// Each lane owns 8 consecutive columns of one token (16-byte loads of every
// routed row, one 16-byte store), so a row is read with fully coalesced
// 1 KiB-per-wave accesses.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 128;
constexpr int kCols = kThreads * 8;  // output columns per block
constexpr int kKChunk = 8;           // top-k rows whose loads are in flight together

// Block b computes columns [cb * kCols, cb * kCols + kCols) of token t, with
// t = b / n_cb and cb = b % n_cb;
// each thread owns 8 columns. The token's row indices and weights are read
// by every thread (the same addresses, served once by the cache) without
// waiting for the live-token count, and the 8 rows of a k-chunk are loaded
// before any is accumulated, so the kernel waits for about three memory
// round trips in all. Accumulation is in ascending k with fp32 FMAs.
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int row_cap, const int32_t* __restrict__ pair_to_row,
    const float* __restrict__ topk_w, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int hidden, uint16_t* __restrict__ out) {
  const int n_cb = (hidden + kCols - 1) / kCols;
  const int t = blockIdx.x / n_cb;
  const int c = (blockIdx.x % n_cb) * kCols + threadIdx.x * 8;
  if (c >= hidden) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int k0 = 0; k0 < topk; k0 += kKChunk) {
    int rows[kKChunk];
    float wts[kKChunk];
#pragma unroll
    for (int j = 0; j < kKChunk; ++j) {
      const int k = k0 + j < topk ? k0 + j : topk - 1;
      rows[j] = pair_to_row[static_cast<int64_t>(t) * topk + k];
      wts[j] = topk_w[static_cast<int64_t>(t) * topk + k];
    }
    uint4 raw[kKChunk];
#pragma unroll
    for (int j = 0; j < kKChunk; ++j) {
      const bool ok = k0 + j < topk && static_cast<unsigned>(rows[j]) < static_cast<unsigned>(row_cap);
      raw[j] = ok ? *reinterpret_cast<const uint4*>(y + static_cast<int64_t>(rows[j]) * hidden + c)
                  : uint4{0, 0, 0, 0};
      if (!ok) wts[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kKChunk; ++j) {
      if (k0 + j >= topk || static_cast<unsigned>(rows[j]) >= static_cast<unsigned>(row_cap)) continue;
      const uint32_t w4[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wts[j], bf16_to_f32(w4[i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wts[j], bf16_to_f32(w4[i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  if (t >= clamp_live(t_live_dev, t_cap)) return;
  uint4 o;
  o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
  o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * hidden + c) = o;
}

}  // namespace

hipError_t launch_topk_combine(const uint16_t* y, int row_cap, const int32_t* pair_to_row,
                               const float* topk_w, int t_cap, const int32_t* t_live_dev,
                               int topk, int hidden, uint16_t* out, hipStream_t stream) {
  if (t_cap == 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(t_cap) * ((hidden + kCols - 1) / kCols);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, y, row_cap,
                     pair_to_row, topk_w, t_cap, t_live_dev, topk, hidden, out);
  return hipGetLastError();
}

}  // namespace moe
