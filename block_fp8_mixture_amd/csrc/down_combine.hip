// FC2 and the top-k combine of a decode-sized layer in one launch.
//
// TensorRT-LLM PR #21250 (description; rounding-fix commit): at decode sizes
// the FC2 GEMM streams the weights of the few live experts, and the top-k sum
// scales the BF16 expert outputs by the routing weights in fp32. vLLM PR
// #65794 (Details): the FC2 input is SiLU(gate) * up quantized per 1x128
// group with the activation rule.
//
// A workgroup (8 waves, one per CU) owns 16 output columns -- 16 weight rows
// of every live expert -- so the whole top-k sum of those columns is formed in
// its LDS, with no further launch and no synchronisation between workgroups.
// Its prologue compacts the live experts from the endpoints; the FC2 input
// rows (fp32, written by the gated FC1) are then quantized, streamed against
// and combined as fc2_decode.h describes. Workgroup 0 also stores the FC2
// input codes and scales to the workspace, bit-identical to
// moe_silu_mul_quant.
#include "device_common.h"
#include "fc2_decode.h"
#include "gemm_device.h"
#include "kernels.h"

namespace moe {
namespace {

template <int FMT>
__global__ __launch_bounds__(kDecThreads, 1) void down_combine_kernel(DownCombineArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kDecWaves * kDecDepth * kDecStage];
  __shared__ __attribute__((aligned(16))) uint8_t s_tok[kDcTokBytes];  // codes, row stride I + 16
  __shared__ float s_sa[kDcMaxScales];   // token scale of (compact row, K block)
  __shared__ __attribute__((aligned(16))) float s_slot[kDcMaxPairs * 16];  // pair q's 16 columns
  __shared__ int s_e[kDcMaxPairs];       // list entry -> expert
  __shared__ int s_cnt[kDcMaxPairs];     //   its live rows
  __shared__ int s_c0[kDcMaxPairs];      //   its first compact row
  __shared__ int s_r0[kDcMaxPairs];      //   its first source row
  __shared__ int s_row[kDcMaxPairs];     // compact row -> source row
  __shared__ int s_pair[kDcMaxPairs];    //   its pair
  __shared__ int s_p2r[kDcMaxPairs];     // pair -> row
  __shared__ float s_tw[kDcMaxPairs];    // pair -> routing weight
  __shared__ int s_wn[kDecWaves], s_wr[kDecWaves];
  __shared__ int s_nlist, s_nrows;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = p.num_experts, N = p.hidden, I = p.inter, KB = I / kGroup, TK = p.topk;
  const int TS = I + 16;              // token row stride in LDS (odd multiple of 16 bytes)
  const int PQ = p.t_cap * TK;        // pairs of capacity (<= kDcMaxPairs)
  const int n_cb = N / 16;
  const int G = gridDim.x;
  // Table limits (all met by consistent metadata of a problem the host admitted).
  const int list_cap = min(kDcMaxPairs, kDcMaxScales / KB);
  const int row_cap_lds = min(list_cap, kDcTokBytes / TS);

  // ---- 1. live experts, in expert order (two 512-expert chunks)
  int cnt_c[2] = {0, 0}, row0_c[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c == 1 && E <= kDecThreads) break;  // uniform
    const int e = tid + c * kDecThreads;
    const int ec = e < E ? e : E - 1;
    row0_c[c] = p.offsets[ec];
    cnt_c[c] = e < E ? segment_rows(row0_c[c], p.offsets[ec + 1], p.counts[ec], p.row_cap) : 0;
  }
  if (tid < PQ) {
    s_p2r[tid] = p.pair_to_row[tid];
    s_tw[tid] = p.topk_w[tid];
  }
  // Through the scalar cache: a vector load still in flight here would be
  // waited for (vmcnt) in the middle of the prologue's prefetch.
  const int t_live = p.t_live_dev ? min(max(scalar_load(p.t_live_dev), 0), p.t_cap) : p.t_cap;
  if (tid == 0) {
    s_nlist = 0;
    s_nrows = 0;
  }
  for (int x = tid; x < PQ * 16; x += kDecThreads) s_slot[x] = 0.0f;  // ordered by the barriers below
  int run_n = 0, run_r = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c == 1 && E <= kDecThreads) break;  // uniform
    const int cnt = cnt_c[c];
    const bool flag = cnt > 0;
    const uint64_t mask = __ballot(flag);
    const int pos = __popcll(mask & ((uint64_t(1) << lane) - 1));
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) {
      s_wn[wave] = __popcll(mask);
      s_wr[wave] = incl;
    }
    __syncthreads();
    int bn = run_n, br = run_r;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      bn += w < wave ? s_wn[w] : 0;
      br += w < wave ? s_wr[w] : 0;
    }
    const int i = bn + pos, c0 = br + incl - cnt;
    if (flag && i < list_cap && c0 + cnt <= row_cap_lds) {  // the valid entries form a prefix
      s_e[i] = tid + c * kDecThreads;
      s_cnt[i] = cnt;
      s_c0[i] = c0;
      s_r0[i] = row0_c[c];
      atomicMax(&s_nlist, i + 1);
      atomicMax(&s_nrows, c0 + cnt);
    }
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      run_n += s_wn[w];
      run_r += s_wr[w];
    }
    __syncthreads();
  }
  // Nothing is in flight yet; an explicit wait here also tells the compiler
  // that the endpoint loads are done on every path, so it does not wait for
  // them (and with them for the stream) when it reuses their registers.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  DecodeTables t;
  t.e = s_e;
  t.cnt = s_cnt;
  t.c0 = s_c0;
  t.r0 = s_r0;
  t.row = s_row;
  t.pair = s_pair;
  t.p2r = s_p2r;
  t.tw = s_tw;
  t.n_list = __builtin_amdgcn_readfirstlane(s_nlist);
  t.n_rows = __builtin_amdgcn_readfirstlane(s_nrows);
  t.n_pairs = PQ;

  Fc2Stream<false> st;
  st.init(p.w, p.w_scales, t, s_ring + wave * (kDecDepth * kDecStage), N, I, wave, lane);
  int cb = blockIdx.x;  // < n_cb: the grid has at most n_cb workgroups
  st.start(cb * 16, 0, kDecPreStages);
  // The rows' pairs come with them (row_to_pair), filling s_row / s_pair.
  fc2_quant_rows<FMT, false>(t, wave, lane, p.act, I, s_tok, s_sa, blockIdx.x == 0, p.hq, p.hs,
                             p.row_cap, p.row_to_pair, s_row, s_pair, p.rounding);
  st.start(cb * 16, kDecPreStages, kDecDepth - 1);
  for (; cb < n_cb; cb += G) {
    const int n0 = cb * 16;
    if (cb != static_cast<int>(blockIdx.x)) {
      for (int x = tid; x < PQ * 16; x += kDecThreads) s_slot[x] = 0.0f;
      lds_barrier();  // zeroed slots visible
      st.start(n0, 0, kDecDepth - 1);
    }
    fc2_stream_block<kDecDepth>(st, n0, t, s_tok, s_sa, s_slot, lane);
    lds_barrier();  // every slot of this column block written
    fc2_combine(t, s_slot, t_live, TK, p.row_cap, N, n0, p.out, p.y, tid);
    lds_barrier();  // slots free for the next column block
  }
}

}  // namespace

hipError_t launch_down_combine(const DownCombineArgs& a, hipStream_t stream) {
  if (a.t_cap == 0) return hipSuccess;
  if (!down_combine_fits(a.t_cap, a.topk, a.inter) || a.hidden % 16 != 0 ||
      a.num_experts > kMaxExperts || a.num_experts < 1)
    return hipErrorInvalidValue;
  const int n_cb = a.hidden / 16;
  const int cus = device_cu_count();
  const int grid = n_cb < cus ? n_cb : cus;
  if (a.fmt == kFp32)
    hipLaunchKernelGGL(down_combine_kernel<kFp32>, dim3(grid), dim3(kDecThreads), 0, stream, a);
  else if (a.fmt == kFp32Pow2)
    hipLaunchKernelGGL(down_combine_kernel<kFp32Pow2>, dim3(grid), dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(down_combine_kernel<kUe8m0>, dim3(grid), dim3(kDecThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
