// Routing alignment: a stable counting sort of (token, k) pairs by expert.
//
// vLLM PR #59128 (Purpose): a shared permutation helper produces the expert
// endpoints that both grouped GEMMs and the activation quantization consume.
// TensorRT-LLM PR #21250 (sequence diagram; review on expert parallelism):
// alignment yields padded expert blocks and sorted token ids, and ids outside
// the local expert range are dropped.
//
// One launch, no scratch memory. Block b owns pairs [b*kChunk, (b+1)*kChunk).
// Every block counts all live pairs per expert in LDS (so every block knows
// the endpoints) and, separately, the pairs before its chunk (so it knows
// where its chunk starts inside each segment). Inside the chunk, pairs are
// ranked stably: a wave groups its lanes by expert with ballots, and waves
// are ordered by an exclusive sum over per-wave counts.
#include "device_common.h"
#include "kernels.h"
#include "quant_device.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 4096;

// The work of align block `block` (all kThreads threads of a block call it).
__device__ __forceinline__ void align_block(
    int block, const int32_t* __restrict__ ids, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int num_experts, int align_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_pair,
    int32_t* __restrict__ pair_to_row) {
  __shared__ int s_total[kMaxExperts];
  __shared__ int s_before[kMaxExperts];
  __shared__ int s_run[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ uint16_t s_wave[kWaves][kMaxExperts];
  __shared__ int s_wsum[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = num_experts;
  // The first id this thread counts is loaded together with the live count
  // (ids holds t_cap * topk entries, so the load is in bounds either way).
  const int e_first = tid < static_cast<int64_t>(t_cap) * topk ? ids[tid] : -1;
  const int n_pairs = clamp_live(t_live_dev, t_cap) * topk;
  const int c0 = block * kChunk;
  if (block > 0 && c0 >= n_pairs) return;

  for (int e = tid; e < E; e += kThreads) {
    s_total[e] = 0;
    s_before[e] = 0;
    s_run[e] = 0;
  }
  for (int i = tid; i < kWaves * E; i += kThreads) s_wave[i / E][i % E] = 0;
  __syncthreads();

  // Phase 1: per-expert counts of all live pairs and of pairs before the chunk.
  for (int p = tid; p < n_pairs; p += kThreads) {
    const int e = p == tid ? e_first : ids[p];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
      atomicAdd(&s_total[e], 1);
      if (p < c0) atomicAdd(&s_before[e], 1);
    }
  }
  __syncthreads();

  // Phase 2: endpoints = exclusive prefix sum of counts rounded up to align_rows.
  // Thread t owns experts [t*per, t*per + per).
  {
    const int per = (E + kThreads - 1) / kThreads;
    const int b = tid * per;
    int local = 0;
    for (int e = b; e < b + per && e < E; ++e)
      local += (s_total[e] + align_rows - 1) / align_rows * align_rows;
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    // Earlier waves' totals: independent LDS reads (no dependent chain).
    int run = incl - local;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) run += w < wave ? s_wsum[w] : 0;
    for (int e = b; e < b + per && e < E; ++e) {
      s_off[e] = run;
      run += (s_total[e] + align_rows - 1) / align_rows * align_rows;
    }
    if (b < E && b + per >= E) s_off[E] = run;
    __syncthreads();
  }

  if (block == 0) {
    for (int e = tid; e < E; e += kThreads) {
      counts[e] = s_total[e];
      offsets[e] = s_off[e];
      for (int r = s_off[e] + s_total[e]; r < s_off[e + 1]; ++r) row_to_pair[r] = -1;
    }
    if (tid == 0) offsets[E] = s_off[E];
  }

  // Phase 3: stable ranks inside the chunk, one round of kThreads pairs at a time.
  const int c1 = min(c0 + kChunk, n_pairs);
  for (int base = c0; base < c1; base += kThreads) {
    const int p = base + tid;
    const bool in_range = p < c1;
    const int e = in_range ? (p == tid ? e_first : ids[p]) : -1;
    const bool ok = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(E);
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int rank = 0;
    uint64_t active = __ballot(ok);
    while (active) {
      // The leader is uniform, so its expert is read with v_readlane (a
      // scalar move), not a cross-lane LDS permute.
      const int leader = __ffsll(static_cast<unsigned long long>(active)) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);
      const uint64_t same = __ballot(ok && e == le);
      if (ok && e == le) rank = __popcll(same & below);
      if (lane == leader) s_wave[wave][le] = static_cast<uint16_t>(__popcll(same));
      active &= ~same;
    }
    __syncthreads();
    if (ok) {
      int prior = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) prior += w < wave ? s_wave[w][e] : 0;
      const int row = s_off[e] + s_before[e] + s_run[e] + prior + rank;
      row_to_pair[row] = p;
      pair_to_row[p] = row;
    } else if (in_range) {
      pair_to_row[p] = -1;
    }
    __syncthreads();
    if (base + kThreads >= c1) break;  // last round: the running counts are not needed again
    for (int x = tid; x < E; x += kThreads) {
      int s = 0;
      for (int w = 0; w < kWaves; ++w) {
        s += s_wave[w][x];
        s_wave[w][x] = 0;
      }
      s_run[x] += s;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int num_experts, int align_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_pair,
    int32_t* __restrict__ pair_to_row) {
  align_block(blockIdx.x, ids, t_cap, t_live_dev, topk, num_experts, align_rows, counts, offsets,
              row_to_pair, pair_to_row);
}

// Routing alignment and the activation quantization in one launch, for the
// whole-layer entry point: the two do not depend on each other, so running
// them as one grid removes a launch and overlaps their memory latencies.
// Blocks [0, n_align) align; the rest quantize kThreads / 16 groups each.
template <int FMT>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const int32_t* __restrict__ ids, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int num_experts, int align_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_pair,
    int32_t* __restrict__ pair_to_row, int n_align, const uint16_t* __restrict__ x, int hidden,
    uint8_t* __restrict__ xq, void* __restrict__ xs) {
  if (static_cast<int>(blockIdx.x) < n_align) {
    align_block(blockIdx.x, ids, t_cap, t_live_dev, topk, num_experts, align_rows, counts,
                offsets, row_to_pair, pair_to_row);
    return;
  }
  const int64_t gid = static_cast<int64_t>(blockIdx.x - n_align) * (kThreads / 16) + (threadIdx.x >> 4);
  act_quant_group<FMT>(x, t_cap, t_live_dev, hidden, xq, xs, gid, threadIdx.x & 15);
}

int align_blocks(int t_cap, int topk) {
  const int64_t pairs = static_cast<int64_t>(t_cap) * topk;
  return static_cast<int>(pairs > 0 ? (pairs + kChunk - 1) / kChunk : 1);
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                        int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                        int32_t* row_to_pair, int32_t* pair_to_row, hipStream_t stream) {
  const int blocks = align_blocks(t_cap, topk);
  hipLaunchKernelGGL(align_kernel, dim3(blocks), dim3(kThreads), 0, stream, ids, t_cap,
                     t_live_dev, topk, num_experts, align_rows, counts, offsets, row_to_pair,
                     pair_to_row);
  return hipGetLastError();
}

hipError_t launch_prep(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                       int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                       int32_t* row_to_pair, int32_t* pair_to_row, const uint16_t* x, int hidden,
                       int fmt, uint8_t* xq, void* xs, hipStream_t stream) {
  const int n_align = align_blocks(t_cap, topk);
  const int64_t groups = static_cast<int64_t>(t_cap) * (hidden / kGroup);
  const int64_t n_quant = (groups + kThreads / 16 - 1) / (kThreads / 16);
  if (n_align + n_quant > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(n_align + n_quant));
  if (fmt == kFp32)
    hipLaunchKernelGGL(prep_kernel<kFp32>, grid, dim3(kThreads), 0, stream, ids, t_cap, t_live_dev,
                       topk, num_experts, align_rows, counts, offsets, row_to_pair, pair_to_row,
                       n_align, x, hidden, xq, xs);
  else if (fmt == kFp32Pow2)
    hipLaunchKernelGGL(prep_kernel<kFp32Pow2>, grid, dim3(kThreads), 0, stream, ids, t_cap,
                       t_live_dev, topk, num_experts, align_rows, counts, offsets, row_to_pair,
                       pair_to_row, n_align, x, hidden, xq, xs);
  else
    hipLaunchKernelGGL(prep_kernel<kUe8m0>, grid, dim3(kThreads), 0, stream, ids, t_cap,
                       t_live_dev, topk, num_experts, align_rows, counts, offsets, row_to_pair,
                       pair_to_row, n_align, x, hidden, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
