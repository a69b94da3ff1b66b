// 1x128 FP8 E4M3 quantization kernels: activations (per token) and the fused
// SiLU(gate) * up quantization of the FC2 input (per live aligned row).
//
// Rule (vLLM PR #65794, Details): scale = max(amax / 448, 1 / (448 * 512)),
// codes = E4M3(x / scale); power-of-two scales round up (vLLM PR #59128,
// Purpose: plain and power-of-two-rounded fp32 scales, packed UE8M0).
//
// Activations: 16 lanes own one 128-element group, 8 consecutive elements
// each (one 16-byte BF16 load); the group amax is a 4-step xor-shuffle
// reduction inside the 16 lanes. SiLU * up: one wave per group, 2 elements
// per lane. The scale leaves from the group's first lane.
#include "device_common.h"
#include "kernels.h"
#include "quant_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / 16;

template <int FMT>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(
    const uint16_t* __restrict__ x, int t_cap, const int32_t* __restrict__ t_live_dev,
    int hidden, uint8_t* __restrict__ xq, void* __restrict__ xs) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4);
  act_quant_group<FMT>(x, t_cap, t_live_dev, hidden, xq, xs, gid, threadIdx.x & 15);
}


// One wave per 128-column group (2 elements per lane): at decode sizes only a
// few dozen groups are live, so spreading each over a whole wave keeps the
// serial fp64 SiLU work per lane short. Waves walk the (row, group) space with
// a grid stride. The expert endpoints are staged in LDS once per block, so
// finding the expert of a row (to skip padding) is a search in LDS, not a
// chain of dependent global loads.
template <int FMT, int ACT>
__global__ __launch_bounds__(kThreads) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ gate_up, int inter, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int num_experts, int row_cap, float clamp_limit,
    uint8_t* __restrict__ hq, void* __restrict__ hs) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_cnt[kMaxExperts];
  constexpr int kWavesPerBlock = kThreads / 64;
  const int groups = inter / kGroup;
  const int lane = threadIdx.x & 63;
  const int64_t n_groups = static_cast<int64_t>(row_cap) * groups;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  int64_t gid = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  // The first group's inputs are loaded before the endpoints arrive (any row
  // below row_cap is inside gate_up).
  uint32_t graw = 0, uraw = 0;
  if (gid < n_groups) {
    const int64_t src = (gid / groups) * (2 * inter) + (gid % groups) * kGroup + lane * 2;
    graw = *reinterpret_cast<const uint32_t*>(gate_up + src);
    uraw = *reinterpret_cast<const uint32_t*>(gate_up + src + inter);
  }
  for (int e = threadIdx.x; e <= num_experts; e += kThreads) {
    s_off[e] = offsets[e];
    if (e < num_experts) s_cnt[e] = counts[e];
  }
  __syncthreads();
  const int total_rows = min(s_off[num_experts], row_cap);
  const double lim = clamp_limit;
  for (bool first = true; gid < static_cast<int64_t>(total_rows) * groups; gid += stride, first = false) {
    const int r = static_cast<int>(gid / groups);
    const int g = static_cast<int>(gid % groups);
    const int e = expert_of_row(s_off, num_experts, r);
    if (r < s_off[e] || r - s_off[e] >= s_cnt[e]) continue;  // pad row: untouched
    const int64_t src = static_cast<int64_t>(r) * (2 * inter) + g * kGroup + lane * 2;
    if (!first) {
      graw = *reinterpret_cast<const uint32_t*>(gate_up + src);
      uraw = *reinterpret_cast<const uint32_t*>(gate_up + src + inter);
    }
    const float y0 = swiglu<ACT>(bf16_to_f32(graw & 0xFFFFu), bf16_to_f32(uraw & 0xFFFFu), lim);
    const float y1 = swiglu<ACT>(bf16_to_f32(graw >> 16), bf16_to_f32(uraw >> 16), lim);
    const float amax = group_max<64>(fmaxf(fabsf(y0), fabsf(y1)));
    const float sc = group_scale(amax, FMT);
    const float inv = 1.0f / sc;  // IEEE division, once per group
    const uint32_t codes = cvt_pk_e4m3(scale_div(y0, sc, inv, FMT), scale_div(y1, sc, inv, FMT));
    *reinterpret_cast<uint16_t*>(hq + static_cast<int64_t>(r) * inter + g * kGroup + lane * 2) =
        static_cast<uint16_t>(codes);
    if (lane == 0) store_scale(hs, FMT, static_cast<int64_t>(g) * row_cap + r, sc);
  }
}

template <int FMT>
hipError_t act_quant_fmt(const uint16_t* x, int t_cap, const int32_t* t_live_dev, int hidden,
                         uint8_t* xq, void* xs, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(t_cap) * (hidden / kGroup);
  const int blocks = static_cast<int>((groups + kGroupsPerBlock - 1) / kGroupsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(act_quant_kernel<FMT>, dim3(blocks), dim3(kThreads), 0, stream, x, t_cap,
                     t_live_dev, hidden, xq, xs);
  return hipGetLastError();
}

template <int FMT, int ACT>
hipError_t smq_launch(const uint16_t* gate_up, int inter, const int32_t* counts,
                      const int32_t* offsets, int num_experts, int row_cap, float clamp_limit,
                      uint8_t* hq, void* hs, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(row_cap) * (inter / kGroup);
  const int64_t need = (groups + kThreads / 64 - 1) / (kThreads / 64);
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  const int blocks = static_cast<int>(need < cap ? need : cap);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((silu_mul_quant_kernel<FMT, ACT>), dim3(blocks), dim3(kThreads), 0, stream,
                     gate_up, inter, counts, offsets, num_experts, row_cap, clamp_limit, hq, hs);
  return hipGetLastError();
}

template <int FMT>
hipError_t smq_fmt(const uint16_t* gate_up, int inter, const int32_t* counts,
                   const int32_t* offsets, int num_experts, int row_cap, int act,
                   float clamp_limit, uint8_t* hq, void* hs, hipStream_t stream) {
  switch (act) {
    case kSwiglu:
      return smq_launch<FMT, kSwiglu>(gate_up, inter, counts, offsets, num_experts, row_cap,
                                      clamp_limit, hq, hs, stream);
    case kSwigluClamp:
      return smq_launch<FMT, kSwigluClamp>(gate_up, inter, counts, offsets, num_experts,
                                           row_cap, clamp_limit, hq, hs, stream);
    default:
      return smq_launch<FMT, kSwigluClampAfterSilu>(gate_up, inter, counts, offsets,
                                                    num_experts, row_cap, clamp_limit, hq, hs,
                                                    stream);
  }
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int t_cap, const int32_t* t_live_dev, int hidden,
                            int fmt, uint8_t* xq, void* xs, hipStream_t stream) {
  switch (fmt) {
    case kFp32: return act_quant_fmt<kFp32>(x, t_cap, t_live_dev, hidden, xq, xs, stream);
    case kFp32Pow2: return act_quant_fmt<kFp32Pow2>(x, t_cap, t_live_dev, hidden, xq, xs, stream);
    default: return act_quant_fmt<kUe8m0>(x, t_cap, t_live_dev, hidden, xq, xs, stream);
  }
}

hipError_t launch_silu_mul_quant(const uint16_t* gate_up, int inter, const int32_t* counts,
                                 const int32_t* offsets, int num_experts, int row_cap, int act,
                                 float clamp_limit, int fmt, uint8_t* hq, void* hs,
                                 hipStream_t stream) {
  switch (fmt) {
    case kFp32:
      return smq_fmt<kFp32>(gate_up, inter, counts, offsets, num_experts, row_cap, act,
                            clamp_limit, hq, hs, stream);
    case kFp32Pow2:
      return smq_fmt<kFp32Pow2>(gate_up, inter, counts, offsets, num_experts, row_cap, act,
                                clamp_limit, hq, hs, stream);
    default:
      return smq_fmt<kUe8m0>(gate_up, inter, counts, offsets, num_experts, row_cap, act,
                             clamp_limit, hq, hs, stream);
  }
}

}  // namespace moe
