// Routing alignment: a stable counting sort of (token, k) pairs by expert.
//
// vLLM PR #59128 (Purpose): a shared permutation helper produces the expert
// endpoints that both grouped GEMMs and the activation quantization consume.
// TensorRT-LLM PR #21250 (sequence diagram; review on expert parallelism):
// alignment yields padded expert blocks and sorted token ids, and ids outside
// the local expert range are dropped.
//
// Expert parallelism (TensorRT-LLM PR #21250, review comment: drop pairs of
// other ranks' experts): ids are read as local ids id - expert_start, and
// those outside [0, E) are dropped. The batched masked-M layout (vLLM PR
// #65794, Details, batched experts; batch_cap > 0): expert e owns the fixed
// rows [e*cap, (e+1)*cap), counts become masked_m = min(count, cap), pairs
// ranked at or past the capacity are dropped (and counted), and rows past
// masked_m are left untouched.
//
// One launch, no scratch memory. Block b owns pairs [b*kChunk, (b+1)*kChunk).
// Every block counts all live pairs per expert in LDS (so every block knows
// the endpoints) and, separately, the pairs before its chunk (so it knows
// where its chunk starts inside each segment). Inside the chunk (one pair
// per thread), pairs are ranked stably: each wave finds, per expert, the set
// of its lanes holding it (a 64-bit lane mask in LDS built by one atomic OR
// per lane when there are at most 256 experts, else a ballot loop over the
// wave's distinct experts), and waves are ordered by an exclusive sum over
// per-wave counts.
#include "device_common.h"
#include "kernels.h"
#include "quant_device.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = kThreads;  // pairs ranked by a block: one per thread
constexpr int kMaskExperts = 256;  // experts ranked by lane masks (32 KB of masks)
constexpr int kBatch = 8;  // ids in flight per thread in the counting pass

// The work of align block `block` (all kThreads threads of a block call it).
__device__ __forceinline__ void align_block(
    int block, const int32_t* __restrict__ ids, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int num_experts, int align_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_pair,
    int32_t* __restrict__ pair_to_row, int expert_start, int batch_cap,
    int32_t* __restrict__ overflow) {
  // Per expert: live pairs (low word) and live pairs before the chunk (high).
  __shared__ unsigned long long s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  // Per-wave ranking state, 32 KB: with at most kMaskExperts experts, bit l
  // of mask [wave][e] is set when lane l holds expert e; otherwise 16-bit
  // counts [wave][e] of the ballot loop.
  __shared__ __attribute__((aligned(16))) unsigned long long s_rank[kWaves * kMaxExperts / 4];
  __shared__ int s_wsum[kWaves];
  __shared__ int16_t s_chunk[kChunk];  // ids of this block's chunk (-1: dropped)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = num_experts;
  const int64_t cap_pairs = static_cast<int64_t>(t_cap) * topk;
  // kBatch ids per thread are loaded together, so their latencies overlap;
  // the first batch is in flight together with the live count (ids holds
  // t_cap * topk entries, so the loads are in bounds either way).
  int ev[kBatch];
  auto load_batch = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = p0 + i * kThreads + tid;
      ev[i] = p < cap_pairs ? ids[p] - expert_start : -1;
    }
  };
  load_batch(0);
  const int n_pairs = clamp_live(t_live_dev, t_cap) * topk;
  const int c0 = block * kChunk;
  if (block > 0 && c0 >= n_pairs) return;

  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
  for (int i = tid; i < kWaves * kMaxExperts / 8; i += kThreads)
    reinterpret_cast<uint4*>(s_rank)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  // Phase 1: per-expert counts of all live pairs and of pairs before the
  // chunk (one 64-bit LDS add per pair); the chunk's own ids are kept in LDS
  // for phase 3.
  for (int p0 = 0; p0 < n_pairs; p0 += kBatch * kThreads) {
    if (p0 > 0) load_batch(p0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = p0 + i * kThreads + tid;
      const int e = ev[i];
      const bool ok = p < n_pairs && static_cast<unsigned>(e) < static_cast<unsigned>(E);
      if (ok) atomicAdd(&s_cnt[e], p < c0 ? 0x100000001ull : 1ull);
      if (p >= c0 && p < c0 + kChunk && p < n_pairs) s_chunk[p - c0] = static_cast<int16_t>(ok ? e : -1);
    }
  }
  __syncthreads();
  auto total = [&](int e) { return static_cast<int>(static_cast<uint32_t>(s_cnt[e])); };

  // Phase 2: endpoints = exclusive prefix sum of counts rounded up to
  // align_rows (thread t owns experts [t*per, t*per + per)), or the fixed
  // segments e*cap of the batched layout.
  if (batch_cap > 0) {
    for (int e = tid; e <= E; e += kThreads) s_off[e] = e * batch_cap;
    __syncthreads();
  } else {
    const int per = (E + kThreads - 1) / kThreads;
    const int b = tid * per;
    int local = 0;
    for (int e = b; e < b + per && e < E; ++e)
      local += (total(e) + align_rows - 1) / align_rows * align_rows;
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
      run += (total(e) + align_rows - 1) / align_rows * align_rows;
    }
    if (b < E && b + per >= E) s_off[E] = run;
    __syncthreads();
  }

  if (block == 0) {
    if (batch_cap > 0) {
      int over = 0;
      for (int e = tid; e < E; e += kThreads) {
        counts[e] = min(total(e), batch_cap);
        if (offsets) offsets[e] = s_off[e];  // implicit in the batched layout: optional
        over += max(total(e) - batch_cap, 0);
      }
      if (overflow) {
        if (tid == 0) s_wsum[0] = 0;
        __syncthreads();
        if (over) atomicAdd(&s_wsum[0], over);
        __syncthreads();
        if (tid == 0) *overflow = s_wsum[0];
      }
    } else {
      for (int e = tid; e < E; e += kThreads) {
        counts[e] = total(e);
        offsets[e] = s_off[e];
        for (int r = s_off[e] + total(e); r < s_off[e + 1]; ++r) row_to_pair[r] = -1;
      }
    }
    if (tid == 0 && offsets) offsets[E] = s_off[E];
  }

  // Phase 3: stable ranks inside the chunk (kChunk == kThreads: one pair per
  // thread). The row of pair p is its segment's start + the pairs of its
  // expert before the chunk + those in earlier waves + those in earlier
  // lanes of its own wave.
  const int p = c0 + tid;
  const bool in_range = p < min(c0 + kChunk, n_pairs);
  const int e = in_range ? s_chunk[tid] : -1;
  const bool ok = e >= 0;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int rank = 0, prior = 0;
  if (E <= kMaskExperts) {  // uniform
    unsigned long long* mask = s_rank;  // [kWaves][kMaskExperts]
    if (ok) atomicOr(&mask[wave * kMaskExperts + e], 1ull << lane);
    // The LDS runs a wave's instructions in order, so the read sees the
    // bits of every lane of this wave.
    if (ok)
      rank = __popcll(__hip_atomic_load(&mask[wave * kMaskExperts + e], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP) & below);
    __syncthreads();
    if (ok) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) prior += w < wave ? __popcll(mask[w * kMaskExperts + e]) : 0;
    }
  } else {
    uint16_t* cnt = reinterpret_cast<uint16_t*>(s_rank);  // [kWaves][kMaxExperts]
    uint64_t active = __ballot(ok);
    while (active) {
      // The leader is uniform, so its expert is read with v_readlane (a
      // scalar move), not a cross-lane LDS permute.
      const int leader = __ffsll(static_cast<unsigned long long>(active)) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);
      const uint64_t same = __ballot(ok && e == le);
      if (ok && e == le) rank = __popcll(same & below);
      if (lane == leader) cnt[wave * kMaxExperts + le] = static_cast<uint16_t>(__popcll(same));
      active &= ~same;
    }
    __syncthreads();
    if (ok) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) prior += w < wave ? cnt[w * kMaxExperts + e] : 0;
    }
  }
  const int within = ok ? static_cast<int>(s_cnt[e] >> 32) + prior + rank : 0;
  if (ok && (batch_cap == 0 || within < batch_cap)) {
    const int row = s_off[e] + within;
    row_to_pair[row] = p;
    pair_to_row[p] = row;
  } else if (in_range) {
    pair_to_row[p] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int t_cap, const int32_t* __restrict__ t_live_dev,
    int topk, int num_experts, int align_rows, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_pair,
    int32_t* __restrict__ pair_to_row, int expert_start, int batch_cap,
    int32_t* __restrict__ overflow) {
  align_block(blockIdx.x, ids, t_cap, t_live_dev, topk, num_experts, align_rows, counts, offsets,
              row_to_pair, pair_to_row, expert_start, batch_cap, overflow);
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
    uint8_t* __restrict__ xq, void* __restrict__ xs, int rnd, AlignMode mode) {
  if (static_cast<int>(blockIdx.x) < n_align) {
    align_block(blockIdx.x, ids, t_cap, t_live_dev, topk, num_experts, align_rows, counts,
                offsets, row_to_pair, pair_to_row, mode.expert_start, mode.batch_cap,
                mode.overflow);
    return;
  }
  const int64_t gid = static_cast<int64_t>(blockIdx.x - n_align) * (kThreads / 16) + (threadIdx.x >> 4);
  act_quant_group<FMT>(x, t_cap, t_live_dev, hidden, xq, xs, gid, threadIdx.x & 15, rnd);
}

int align_blocks(int t_cap, int topk) {
  const int64_t pairs = static_cast<int64_t>(t_cap) * topk;
  return static_cast<int>(pairs > 0 ? (pairs + kChunk - 1) / kChunk : 1);
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                        int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                        int32_t* row_to_pair, int32_t* pair_to_row, AlignMode mode,
                        hipStream_t stream) {
  const int blocks = align_blocks(t_cap, topk);
  hipLaunchKernelGGL(align_kernel, dim3(blocks), dim3(kThreads), 0, stream, ids, t_cap,
                     t_live_dev, topk, num_experts, align_rows, counts, offsets, row_to_pair,
                     pair_to_row, mode.expert_start, mode.batch_cap, mode.overflow);
  return hipGetLastError();
}

hipError_t launch_prep(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                       int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                       int32_t* row_to_pair, int32_t* pair_to_row, const uint16_t* x, int hidden,
                       int fmt, int rounding, uint8_t* xq, void* xs, AlignMode mode,
                       hipStream_t stream) {
  const int n_align = align_blocks(t_cap, topk);
  const int64_t groups = static_cast<int64_t>(t_cap) * (hidden / kGroup);
  const int64_t n_quant = (groups + kThreads / 16 - 1) / (kThreads / 16);
  if (n_align + n_quant > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(n_align + n_quant));
  if (fmt == kFp32)
    hipLaunchKernelGGL(prep_kernel<kFp32>, grid, dim3(kThreads), 0, stream, ids, t_cap, t_live_dev,
                       topk, num_experts, align_rows, counts, offsets, row_to_pair, pair_to_row,
                       n_align, x, hidden, xq, xs, rounding, mode);
  else if (fmt == kFp32Pow2)
    hipLaunchKernelGGL(prep_kernel<kFp32Pow2>, grid, dim3(kThreads), 0, stream, ids, t_cap,
                       t_live_dev, topk, num_experts, align_rows, counts, offsets, row_to_pair,
                       pair_to_row, n_align, x, hidden, xq, xs, rounding, mode);
  else
    hipLaunchKernelGGL(prep_kernel<kUe8m0>, grid, dim3(kThreads), 0, stream, ids, t_cap,
                       t_live_dev, topk, num_experts, align_rows, counts, offsets, row_to_pair,
                       pair_to_row, n_align, x, hidden, xq, xs, rounding, mode);
  return hipGetLastError();
}

}  // namespace moe
