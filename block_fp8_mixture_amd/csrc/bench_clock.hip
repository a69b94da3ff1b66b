// Device-clock marks for benchmarking (not part of the layer's C ABI; built
// into a separate library that only the benchmark loads).
//
// A mark is a one-thread kernel that takes the next slot from a device
// counter and stores the GPU's constant-rate wall clock there. Captured at
// both ends of a HIP graph, two marks bracket the graph's kernels on the GPU
// timeline, so their difference is the kernel span of one replay without the
// host-side graph launch latency that events around the replay include. The
// opening mark reads the clock as late as it can (after taking its slot), the
// closing mark as early as it can (before), so the span holds as little of
// the marks' own time as possible.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void mark_kernel(uint64_t* slots, uint32_t* counter, uint32_t cap, int closing) {
  const uint64_t t0 = closing ? wall_clock64() : 0;
  const uint32_t i = atomicAdd(counter, 1u);
  if (i < cap) slots[i] = closing ? t0 : wall_clock64();
}

}  // namespace

// Stores the wall clock into slots[(*counter)++] (skipped once the counter
// reaches cap) on `stream`: read after taking the slot, or before it when
// `closing` (the mark after the measured work). Returns 0, or 1 if the launch
// failed.
extern "C" int moe_bench_mark(uint64_t* slots, uint32_t* counter, uint32_t cap, int closing,
                              void* stream) {
  hipLaunchKernelGGL(mark_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), slots,
                     counter, cap, closing);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Ticks per second of the wall clock the marks read, or 0 on error.
extern "C" int64_t moe_bench_clock_hz(void) {
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, 0) != hipSuccess) return 0;
  return static_cast<int64_t>(khz) * 1000;
}

// Attainable peaks of this GPU, measured (the layer is compared with them
// beside the spec-sheet peaks).

namespace {

typedef int v8i_b __attribute__((ext_vector_type(8)));
typedef float v16f_b __attribute__((ext_vector_type(16)));

// Streaming read: every thread reads 16-byte chunks at a grid stride, eight in
// flight, and folds them into one word per thread (stored, so nothing is
// dead). Reads `n16` chunks of src.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
  }
  for (; i < n16; i += stride) acc ^= src[i].x;
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// FP8 matrix cores alone: each wave issues v_mfma_f32_32x32x64_f8f6f4 on four
// independent accumulators from register operands, `iters` times each.
__global__ __launch_bounds__(512, 1) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v8i_b a, b;
  for (int j = 0; j < 8; ++j) {  // E4M3 codes 0x28..0x37 (0.25 .. 0.9), varied per lane
    a[j] = static_cast<int>(0x28282828u + static_cast<uint32_t>((lane + j) & 15) * 0x01010101u);
    b[j] = static_cast<int>(0x28282828u + static_cast<uint32_t>((3 * lane + j) & 15) * 0x01010101u);
  }
  v16f_b c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Streaming read of `bytes` (a multiple of 16) from src on `stream`, with
// `blocks` workgroups of 256 threads; sink holds blocks * 256 words. Returns
// 0, or 1 if the launch failed.
extern "C" int moe_bench_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                                     void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// `blocks` workgroups of 8 waves, each wave 4 * iters FP8 MFMAs of
// 32 x 32 x 64 (131072 FLOPs each); sink holds blocks * 512 floats.
extern "C" int moe_bench_mfma_loop(int iters, float* sink, int blocks, void* stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream),
                     iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
