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
