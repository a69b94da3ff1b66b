// 1x128 FP8 E4M3 quantization kernels: activations (per token) and the fused
// SiLU(gate) * up quantization of the FC2 input (per live aligned row).
//
// Rule (vLLM PR #65794, Details): scale = max(amax / 448, 1 / (448 * 512)),
// codes = E4M3(x / scale); power-of-two scales round up (vLLM PR #59128,
// Purpose: plain and power-of-two-rounded fp32 scales, packed UE8M0).
//
// Layout: 16 lanes own one 128-element group, 8 consecutive elements each
// (one 16-byte BF16 load), so a 256-thread block quantizes 16 groups; the
// group amax is a 4-step xor-shuffle reduction inside the 16 lanes. Codes
// leave as one 8-byte store per lane, the scale from the group's first lane.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / 16;

struct Vals8 {
  float v[8];
};

__device__ __forceinline__ Vals8 unpack_bf16x8(uint4 raw) {
  Vals8 r;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    r.v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  return r;
}

// Quantizes the 8 values this lane holds against the group's scale; returns
// the 8 codes packed little-endian and writes the stored scale when asked.
template <int FMT>
__device__ __forceinline__ uint2 quantize8(const Vals8& x, float* scale_out) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x.v[i]));
  amax = group_max<16>(amax);
  const float s = group_scale(amax, FMT);
  const float inv = FMT == kFp32 ? 0.0f : 1.0f / s;  // exact for powers of two
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = scale_div(x.v[i], s, inv, FMT);
  uint2 out;
  out.x = cvt_pk_e4m3(q[0], q[1]) | (cvt_pk_e4m3(q[2], q[3]) << 16);
  out.y = cvt_pk_e4m3(q[4], q[5]) | (cvt_pk_e4m3(q[6], q[7]) << 16);
  *scale_out = s;
  return out;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(
    const uint16_t* __restrict__ x, int t_cap, const int32_t* __restrict__ t_live_dev,
    int hidden, uint8_t* __restrict__ xq, void* __restrict__ xs) {
  const int groups = hidden / kGroup;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4);
  const int l16 = threadIdx.x & 15;
  if (gid >= static_cast<int64_t>(t_cap) * groups) return;  // whole 16-lane groups exit
  const int t = static_cast<int>(gid / groups);
  const int g = static_cast<int>(gid % groups);
  const int64_t base = static_cast<int64_t>(t) * hidden + g * kGroup + l16 * 8;
  // The row is inside x whether or not the token is live, so its load is
  // issued together with the live-count load instead of after it.
  const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
  if (t >= clamp_live(t_live_dev, t_cap)) return;
  const Vals8 v = unpack_bf16x8(raw);
  float s;
  const uint2 codes = quantize8<FMT>(v, &s);
  *reinterpret_cast<uint2*>(xq + base) = codes;
  if (l16 == 0) store_scale(xs, FMT, static_cast<int64_t>(g) * t_cap + t, s);
}

enum Act : int { kSwiglu = 0, kSwigluClamp = 1, kSwigluClampAfterSilu = 2 };

// SiLU(g) * u in double, rounded once to float (vLLM PR #65794, Details: no
// intermediate BF16 rounding). Clamp variants as TensorRT-LLM PR #21250's
// test coverage names them, with limit L: clamp gate above and up to [-L, L]
// before SiLU, or clamp SiLU's output above and up to [-L, L].
template <int ACT>
__device__ __forceinline__ float swiglu(float gf, float uf, double lim) {
  double g = gf, u = uf;
  if (ACT == kSwigluClamp) {
    g = fmin(g, lim);
    u = fmin(fmax(u, -lim), lim);
  }
  double s = g / (1.0 + exp(-g));
  if (ACT == kSwigluClampAfterSilu) {
    s = fmin(s, lim);
    u = fmin(fmax(u, -lim), lim);
  }
  return static_cast<float>(s * u);
}

// Blocks walk the (row, group) space with a grid stride. The expert
// endpoints are staged in LDS once per block, so finding the expert of a row
// (to skip padding) is a search in LDS, not a chain of dependent global
// loads.
template <int FMT, int ACT>
__global__ __launch_bounds__(kThreads) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ gate_up, int inter, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int num_experts, int row_cap, float clamp_limit,
    uint8_t* __restrict__ hq, void* __restrict__ hs) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_cnt[kMaxExperts];
  const int groups = inter / kGroup;
  const int l16 = threadIdx.x & 15;
  const int64_t n_groups = static_cast<int64_t>(row_cap) * groups;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kGroupsPerBlock;
  int64_t gid = static_cast<int64_t>(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4);
  // First item's rows are loaded before the endpoints arrive (any row below
  // row_cap is inside gate_up).
  uint4 graw = {0, 0, 0, 0}, uraw = {0, 0, 0, 0};
  if (gid < n_groups) {
    const int64_t src = (gid / groups) * (2 * inter) + (gid % groups) * kGroup + l16 * 8;
    graw = *reinterpret_cast<const uint4*>(gate_up + src);
    uraw = *reinterpret_cast<const uint4*>(gate_up + src + inter);
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
    const int64_t src = static_cast<int64_t>(r) * (2 * inter) + g * kGroup + l16 * 8;
    if (!first) {
      graw = *reinterpret_cast<const uint4*>(gate_up + src);
      uraw = *reinterpret_cast<const uint4*>(gate_up + src + inter);
    }
    const Vals8 gv = unpack_bf16x8(graw);
    const Vals8 uv = unpack_bf16x8(uraw);
    Vals8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y.v[i] = swiglu<ACT>(gv.v[i], uv.v[i], lim);
    float s;
    const uint2 codes = quantize8<FMT>(y, &s);
    *reinterpret_cast<uint2*>(hq + static_cast<int64_t>(r) * inter + g * kGroup + l16 * 8) = codes;
    if (l16 == 0) store_scale(hs, FMT, static_cast<int64_t>(g) * row_cap + r, s);
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
  const int64_t need = (groups + kGroupsPerBlock - 1) / kGroupsPerBlock;
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
