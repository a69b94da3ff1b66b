// 1x128 FP8 E4M3 quantization kernels: activations (per token) and the fused
// SiLU(gate) * up quantization of the FC2 input (per live aligned row).
//
// Rule (vLLM PR #65794, Details): scale = max(amax / 448, 1 / (448 * 512)),
// codes = E4M3(x / scale); power-of-two scales round up (vLLM PR #59128,
// Purpose: plain and power-of-two-rounded fp32 scales, packed UE8M0).
//
// 16 lanes own one 128-element group, 8 consecutive elements each (one
// 16-byte BF16 load per operand); the group amax is a DPP reduction inside
// the 16 lanes, and the scale leaves from the group's first lane. The same
// layout serves the activations (per token) and SiLU * up (per live row).
#include <type_traits>

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
    int hidden, uint8_t* __restrict__ xq, void* __restrict__ xs, int rnd) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4);
  act_quant_group<FMT>(x, t_cap, t_live_dev, hidden, xq, xs, gid, threadIdx.x & 15, rnd);
}


// 16 lanes per 128-column group, 8 consecutive columns each: one 16-byte
// load of gate and one of up per lane, 8 independent SiLU evaluations, and
// the group amax by DPP moves inside the 16 lanes. Threads walk the (row,
// group) space with a grid stride, two groups per step whose four loads are
// issued before either is used; the expert of a row (to skip padding) is
// found by a search over endpoints staged in LDS once per block, while the
// loads are in flight. A block with at least kSmqLutGroups groups to do
// first fills the SiLU table of BF16 gates in LDS and takes SiLU from it
// (swiglu_lut, bit-identical to swiglu); smaller launches evaluate the fp64
// SiLU per element.
constexpr int kSmqThreads = 512;
constexpr int kSmqGroupsPerBlock = kSmqThreads / 16;
constexpr int kSmqLutGroups = 128;  // 16384 elements per block: four times the table's entries

template <int FMT, int ACT>
__global__ __launch_bounds__(kSmqThreads) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ gate_up, int inter, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int num_experts, int row_cap, float clamp_limit,
    uint8_t* __restrict__ hq, void* __restrict__ hs, int rnd, int seg_cap) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ double s_lut[kSiluLutSize];
  const int groups = inter / kGroup;
  const int l16 = threadIdx.x & 15;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kSmqGroupsPerBlock;
  for (int e = threadIdx.x; e <= num_experts; e += kSmqThreads) {
    s_off[e] = seg_cap > 0 ? e * seg_cap : offsets[e];  // the batched layout's fixed segments
    if (e < num_experts) s_cnt[e] = counts[e];
  }
  __syncthreads();
  const int64_t n = static_cast<int64_t>(min(s_off[num_experts], row_cap)) * groups;
  const double lim = clamp_limit;
  auto run = [&](auto use_lut) {
    for (int64_t gid = static_cast<int64_t>(blockIdx.x) * kSmqGroupsPerBlock + (threadIdx.x >> 4);
         gid < n; gid += 2 * stride) {
      int64_t rows[2];
      int gs[2];
      uint4 gr[2], ur[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int64_t q = gid + k * stride < n ? gid + k * stride : gid;  // in-range stand-in
        rows[k] = static_cast<uint32_t>(q) / static_cast<uint32_t>(groups);  // q < 2^31 (host check)
        gs[k] = static_cast<int>(static_cast<uint32_t>(q) - static_cast<uint32_t>(rows[k]) * groups);
        const int64_t src = rows[k] * (2 * inter) + gs[k] * kGroup + l16 * 8;
        gr[k] = *reinterpret_cast<const uint4*>(gate_up + src);
        ur[k] = *reinterpret_cast<const uint4*>(gate_up + src + inter);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = static_cast<int>(rows[k]);
        const int e = expert_of_row(s_off, num_experts, r);
        // Whole 16-lane groups agree on this test, so the DPP moves below
        // always see a fully active row of lanes.
        if (gid + k * stride >= n || r < s_off[e] || r - s_off[e] >= s_cnt[e]) continue;  // pad row
        const Vals8 g8 = unpack_bf16x8(gr[k]), u8 = unpack_bf16x8(ur[k]);
        Vals8 y;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if constexpr (decltype(use_lut)::value)
            y.v[i] = swiglu_lut<ACT>(g8.v[i], u8.v[i], lim, s_lut);
          else
            y.v[i] = swiglu<ACT>(g8.v[i], u8.v[i], lim);
        }
        if (rnd == kReciprocal) {  // the SwiGLU output rounded to BF16 first
#pragma unroll
          for (int i = 0; i < 8; ++i) y.v[i] = round_bf16(y.v[i]);
        }
        float sc;
        const uint2 codes = quantize8<FMT>(y, &sc, rnd);
        *reinterpret_cast<uint2*>(hq + static_cast<int64_t>(r) * inter + gs[k] * kGroup + l16 * 8) = codes;
        if (l16 == 0) store_scale(hs, FMT, static_cast<int64_t>(gs[k]) * row_cap + r, sc);
      }
    }
  };
  if (n >= static_cast<int64_t>(kSmqLutGroups) * gridDim.x) {  // uniform
    fill_silu_lut(s_lut, threadIdx.x, kSmqThreads);
    __syncthreads();
    run(std::true_type{});
  } else {
    run(std::false_type{});
  }
}

template <int FMT>
hipError_t act_quant_fmt(const uint16_t* x, int t_cap, const int32_t* t_live_dev, int hidden,
                         uint8_t* xq, void* xs, int rnd, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(t_cap) * (hidden / kGroup);
  const int blocks = static_cast<int>((groups + kGroupsPerBlock - 1) / kGroupsPerBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(act_quant_kernel<FMT>, dim3(blocks), dim3(kThreads), 0, stream, x, t_cap,
                     t_live_dev, hidden, xq, xs, rnd);
  return hipGetLastError();
}

template <int FMT, int ACT>
hipError_t smq_launch(const uint16_t* gate_up, int inter, const int32_t* counts,
                      const int32_t* offsets, int num_experts, int row_cap, float clamp_limit,
                      uint8_t* hq, void* hs, int rnd, int seg_cap, hipStream_t stream) {
  const int64_t groups = static_cast<int64_t>(row_cap) * (inter / kGroup);
  if (groups > INT32_MAX) return hipErrorInvalidValue;  // the kernel divides 32-bit group indices
  const int64_t need = (groups + 2 * kSmqGroupsPerBlock - 1) / (2 * kSmqGroupsPerBlock);
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 2;
  const int blocks = static_cast<int>(need < cap ? need : cap);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((silu_mul_quant_kernel<FMT, ACT>), dim3(blocks), dim3(kSmqThreads), 0, stream,
                     gate_up, inter, counts, offsets, num_experts, row_cap, clamp_limit, hq, hs, rnd,
                     seg_cap);
  return hipGetLastError();
}

template <int FMT>
hipError_t smq_fmt(const uint16_t* gate_up, int inter, const int32_t* counts,
                   const int32_t* offsets, int num_experts, int row_cap, int act,
                   float clamp_limit, uint8_t* hq, void* hs, int rnd, int seg_cap,
                   hipStream_t stream) {
  switch (act) {
    case kSwiglu:
      return smq_launch<FMT, kSwiglu>(gate_up, inter, counts, offsets, num_experts, row_cap,
                                      clamp_limit, hq, hs, rnd, seg_cap, stream);
    case kSwigluClamp:
      return smq_launch<FMT, kSwigluClamp>(gate_up, inter, counts, offsets, num_experts,
                                           row_cap, clamp_limit, hq, hs, rnd, seg_cap, stream);
    default:
      return smq_launch<FMT, kSwigluClampAfterSilu>(gate_up, inter, counts, offsets,
                                                    num_experts, row_cap, clamp_limit, hq, hs,
                                                    rnd, seg_cap, stream);
  }
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* x, int t_cap, const int32_t* t_live_dev, int hidden,
                            int fmt, int rounding, uint8_t* xq, void* xs, hipStream_t stream) {
  switch (fmt) {
    case kFp32: return act_quant_fmt<kFp32>(x, t_cap, t_live_dev, hidden, xq, xs, rounding, stream);
    case kFp32Pow2:
      return act_quant_fmt<kFp32Pow2>(x, t_cap, t_live_dev, hidden, xq, xs, rounding, stream);
    default: return act_quant_fmt<kUe8m0>(x, t_cap, t_live_dev, hidden, xq, xs, rounding, stream);
  }
}

hipError_t launch_silu_mul_quant(const uint16_t* gate_up, int inter, const int32_t* counts,
                                 const int32_t* offsets, int num_experts, int row_cap, int act,
                                 float clamp_limit, int fmt, int rounding, uint8_t* hq, void* hs,
                                 int seg_cap, hipStream_t stream) {
  const int rnd = rounding;
  switch (fmt) {
    case kFp32:
      return smq_fmt<kFp32>(gate_up, inter, counts, offsets, num_experts, row_cap, act,
                            clamp_limit, hq, hs, rnd, seg_cap, stream);
    case kFp32Pow2:
      return smq_fmt<kFp32Pow2>(gate_up, inter, counts, offsets, num_experts, row_cap, act,
                                clamp_limit, hq, hs, rnd, seg_cap, stream);
    default:
      return smq_fmt<kUe8m0>(gate_up, inter, counts, offsets, num_experts, row_cap, act,
                             clamp_limit, hq, hs, rnd, seg_cap, stream);
  }
}

}  // namespace moe
