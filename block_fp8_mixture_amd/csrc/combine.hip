// Top-k weighted unpermute/sum back to token order, BF16 out.
//
// TensorRT-LLM PR #21250 (rounding-fix commit): the routing weights scale the
// BF16 expert outputs in fp32 inside the top-k sum, not the FC2 accumulators.
// Terms are added in ascending k; dropped pairs (row -1) contribute nothing.
//
// One block per token; each lane owns 8 consecutive columns (16-byte loads of
// every routed row, one 16-byte store), so a row is read with fully
// coalesced 4 KiB-per-wave accesses.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxTopk = 64;

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint16_t* __restrict__ y, int row_cap, const int32_t* __restrict__ pair_to_row,
    const float* __restrict__ topk_w, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int hidden, uint16_t* __restrict__ out) {
  __shared__ int s_row[kMaxTopk];
  __shared__ float s_w[kMaxTopk];
  const int t = blockIdx.x;
  if (t >= clamp_live(t_live_dev, t_cap)) return;
  if (threadIdx.x < topk) {
    const int r = pair_to_row[static_cast<int64_t>(t) * topk + threadIdx.x];
    const bool ok = static_cast<unsigned>(r) < static_cast<unsigned>(row_cap);
    s_row[threadIdx.x] = ok ? r : -1;
    s_w[threadIdx.x] = topk_w[static_cast<int64_t>(t) * topk + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < hidden; c += kThreads * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int k = 0; k < topk; ++k) {
      const int r = s_row[k];
      if (r < 0) continue;
      const float wk = s_w[k];
      const uint4 raw = *reinterpret_cast<const uint4*>(y + static_cast<int64_t>(r) * hidden + c);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wk, bf16_to_f32(w4[i] & 0xFFFFu), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wk, bf16_to_f32(w4[i] >> 16), acc[2 * i + 1]);
      }
    }
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
    o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
    o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
    o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(t) * hidden + c) = o;
  }
}

}  // namespace

hipError_t launch_topk_combine(const uint16_t* y, int row_cap, const int32_t* pair_to_row,
                               const float* topk_w, int t_cap, const int32_t* t_live_dev,
                               int topk, int hidden, uint16_t* out, hipStream_t stream) {
  if (t_cap == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(t_cap), dim3(kThreads), 0, stream, y, row_cap,
                     pair_to_row, topk_w, t_cap, t_live_dev, topk, hidden, out);
  return hipGetLastError();
}

}  // namespace moe
