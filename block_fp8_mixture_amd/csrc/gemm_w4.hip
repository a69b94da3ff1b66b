// Grouped GEMM with FP8 E4M3 activations and MXFP4 weights.
//
// vLLM PR #59128 (description) names FP4 weights, whose GEMM consumes the
// same prefix-sum expert endpoints as the FP8 one; the pages give no format,
// and it is read as OCP MXFP4: E2M1 codes, two per byte (the even K element
// in the low nibble), one E8M0 scale per 32 consecutive weights along K.
// Activations keep the layer's 1x128 groups with fp32, power-of-two or
// UE8M0 scales (vLLM PR #65794, Details).
//
// gfx950's scaled MFMA takes the weight scales in hardware:
// v_mfma_scale_f32_32x32x64_f8f6f4 with an E2M1 A operand (the weights) and
// an E4M3 B operand (the tokens). Its operand layout, measured on the chip:
//  - E2M1 A: lane l holds weight row l % 32 and the 32 consecutive K values
//    [32 h, 32 h + 32) of the instruction's 64, h = l / 32, low nibble first
//    (16 bytes: the first 4 dwords of the operand);
//  - the scale operand of lane l (byte 0) scales row l % 32 over those same
//    32 K values, the same block the lane's own codes cover;
//  - E4M3 B: lane l holds token l % 32 and, in bytes 0..15, K values
//    [16 h, 16 h + 16), in bytes 16..31 K values [32 + 16 h, 48 + 16 h) (the
//    same scale blocks as A: bytes 0..15 of both halves belong to block 0);
//  - the result is the usual 32x32 layout: lane l holds token l % 32 and
//    weight rows 8 (v / 4) + 4 h + v % 4 of its 16 values v.
// Each 128-wide K step (one activation group) runs two instructions chained
// from zero, then the step's activation scale multiplies the partial sum
// into the accumulator (16 FMAs per lane): the oracle's order, one
// activation block at a time.
//
// Work: a wave task is (expert, 32 token rows, 32 weight rows, 1/S of K).
// A 4-wave workgroup runs 4/S tasks at once; the S waves of a task add their
// partial sums in LDS in wave order, so the result does not depend on which
// finishes first. S (1, 2 or 4) is picked on the device so that the tasks
// fill the grid's waves. Tasks run expert by expert, token tile by token
// tile, and the weight tiles fastest, so neighbouring tasks share their
// token rows in L2. Weights and tokens go straight from global memory into
// the MFMA registers, two K steps ahead.
#include "device_common.h"
#include "gemm_device.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kW4Threads = 256;
constexpr int kW4Waves = kW4Threads / 64;
constexpr int kW4Tile = 32;  // token rows and weight rows of a wave task

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int w4_seg_start(const W4Args& p, int e) {
  return p.seg_cap > 0 ? e * p.seg_cap : p.offsets[e];
}
__device__ __forceinline__ int w4_rows(const W4Args& p, int e) {
  const int s0 = w4_seg_start(p, e);
  const int s1 = p.seg_cap > 0 ? s0 + p.seg_cap : p.offsets[e + 1];
  return segment_rows(s0, s1, p.counts[e], p.row_cap);
}

// The loads of one K step of a wave task, in MFMA operand order.
struct W4Step {
  uint4 w[2];   // E2M1 codes of the two instructions
  uint4 t[4];   // E4M3 token codes: instruction 0 bytes 0..15, 16..31, instruction 1 ...
  uint32_t ws;  // the row's four E8M0 bytes of the step
  float sa;     // the token's activation scale of the step
};

template <bool UE8M0, bool GATHER>
__global__ __launch_bounds__(kW4Threads, 2) void gemm_w4_kernel(W4Args p) {
  __shared__ int s_pref[kMaxExperts + 1];  // exclusive prefix of 32-row token tiles over experts
  __shared__ int s_wsum[kW4Waves];
  __shared__ __attribute__((aligned(16))) float s_red[kW4Waves][64 * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int E = p.num_experts;

  // ---- token tiles per expert and their prefix (every workgroup, in LDS)
  constexpr int kPer = (kMaxExperts + kW4Threads - 1) / kW4Threads;
  int tiles[kPer], run = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    tiles[i] = e < E ? (w4_rows(p, e) + kW4Tile - 1) / kW4Tile : 0;
    run += tiles[i];
  }
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = incl - run;
  for (int w = 0; w < wave; ++w) base += s_wsum[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    if (e < E) s_pref[e] = base;
    base += tiles[i];
  }
  if (tid == kW4Threads - 1) s_pref[E] = base;
  __syncthreads();

  const int N = p.n, K = p.k, KB = K / kGroup;
  const int nt = N / kW4Tile;
  const int T0 = s_pref[E] * nt;  // (token tile, weight tile) tasks
  if (T0 == 0) return;
  int lgS = 0;
  const int target = static_cast<int>(gridDim.x) * kW4Waves;
  while (lgS < 2 && (T0 << (lgS + 1)) <= target && (KB & ((2 << lgS) - 1)) == 0) ++lgS;
  const int S = 1 << lgS;
  const int per_wg = kW4Waves >> lgS;  // tasks of a workgroup unit
  const int n_units = (T0 + per_wg - 1) / per_wg;
  const int ks = wave & (S - 1);
  const int kbs = KB >> lgS;  // K steps of a share
  const v16f zero = {};

  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int t = unit * per_wg + (wave >> lgS);
    const bool live = t < T0;
    v16f acc = zero;
    int e = 0, rows_here = 0, row0 = 0, n0 = 0;
    if (live) {
      const int tm_all = t / nt;
      n0 = (t - tm_all * nt) * kW4Tile;
      int lo = 0, hi = E - 1;  // the expert whose token tiles hold tm_all
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] <= tm_all) lo = mid; else hi = mid - 1;
      }
      e = lo;
      const int mt = tm_all - s_pref[e];
      rows_here = min(kW4Tile, w4_rows(p, e) - mt * kW4Tile);
      row0 = w4_seg_start(p, e) + mt * kW4Tile;

      // This lane's weight row and token row (a dead token row reads a live
      // one's codes; its results are never stored).
      const int64_t wrow = static_cast<int64_t>(e) * N + n0 + (lane & 31);
      const uint8_t* wp = p.w + wrow * (K / 2) + 16 * h;
      const uint8_t* sp = p.w_scales + wrow * (K / kMxBlock);
      const int j = lane & 31;
      int src = -1;
      if (j < rows_here) {
        const int r = row0 + j;
        src = GATHER ? p.a_row_map[r] / p.a_row_div : r;
        if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) src = -1;
      }
      const int src_ld = src < 0 ? 0 : src;
      const uint8_t* tp = p.a + static_cast<int64_t>(src_ld) * K + 16 * h;

      auto load = [&](int kb, W4Step& s) {
        s.w[0] = *reinterpret_cast<const uint4*>(wp + kb * 64);
        s.w[1] = *reinterpret_cast<const uint4*>(wp + kb * 64 + 32);
        s.ws = *reinterpret_cast<const uint32_t*>(sp + kb * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) s.t[q] = *reinterpret_cast<const uint4*>(tp + kb * kGroup + 32 * q);
        const int64_t si = static_cast<int64_t>(kb) * p.a_rows + src_ld;
        if constexpr (UE8M0)
          s.sa = __uint_as_float(static_cast<uint32_t>(static_cast<const uint8_t*>(p.a_scales)[si]) << 23);
        else
          s.sa = static_cast<const float*>(p.a_scales)[si];
      };
      auto compute = [&](const W4Step& s) {
        v16f part = zero;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const v8i wa = {static_cast<int>(s.w[kk].x), static_cast<int>(s.w[kk].y),
                          static_cast<int>(s.w[kk].z), static_cast<int>(s.w[kk].w), 0, 0, 0, 0};
          const uint4 b0 = s.t[2 * kk], b1 = s.t[2 * kk + 1];
          const v8i tb = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                          static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                          static_cast<int>(b1.z), static_cast<int>(b1.w)};
          const int sc = static_cast<int>((s.ws >> (8 * (2 * kk + h))) & 0xFFu);
          part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, tb, part, 4, 0, 0, sc, 0, 127);
        }
        const float sa = src < 0 ? 0.0f : s.sa;
        acc += part * sa;
      };

      // Two K steps in flight ahead of the one computed.
      const int kb0 = ks * kbs, kb1 = kb0 + kbs;
      W4Step s0, s1, s2;
      load(kb0, s0);
      if (kb0 + 1 < kb1) load(kb0 + 1, s1);
      int kb = kb0;
      for (; kb + 2 < kb1; kb += 3) {
        load(kb + 2, s2);
        compute(s0);
        if (kb + 3 < kb1) load(kb + 3, s0);
        compute(s1);
        if (kb + 4 < kb1) load(kb + 4, s1);
        compute(s2);
      }
      if (kb < kb1) compute(s0);
      if (kb + 1 < kb1) compute(s1);
    }
    if (S > 1) {
      // K-split partials: each wave's 16 values per lane to LDS, the task's
      // first share adds the S of them in wave order.
      float* mine = s_red[wave] + lane * 16;
#pragma unroll
      for (int v = 0; v < 16; v += 4) *reinterpret_cast<float4*>(mine + v) = make_float4(acc[v], acc[v + 1], acc[v + 2], acc[v + 3]);
      __syncthreads();
      if (ks == 0) {
        acc = zero;
        for (int w = wave; w < wave + S; ++w) {
          const float* src = s_red[w] + lane * 16;
#pragma unroll
          for (int v = 0; v < 16; v += 4) {
            const float4 x = *reinterpret_cast<const float4*>(src + v);
            acc[v] += x.x;
            acc[v + 1] += x.y;
            acc[v + 2] += x.z;
            acc[v + 3] += x.w;
          }
        }
      }
      __syncthreads();  // the slots are free for the next unit
    }
    if (live && ks == 0 && (lane & 31) < rows_here) {
      uint16_t* crow = p.c + static_cast<int64_t>(row0 + (lane & 31)) * N + n0 + 4 * h;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f v = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        *reinterpret_cast<uint2*>(crow + 8 * g) = pack_bf16x4(v);
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm_w4(const W4Args& g, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(4 * device_cu_count()));
  const bool u = g.fmt == kUe8m0, m = g.a_row_map != nullptr;
  if (u && m) hipLaunchKernelGGL((gemm_w4_kernel<true, true>), grid, dim3(kW4Threads), 0, stream, g);
  else if (u) hipLaunchKernelGGL((gemm_w4_kernel<true, false>), grid, dim3(kW4Threads), 0, stream, g);
  else if (m) hipLaunchKernelGGL((gemm_w4_kernel<false, true>), grid, dim3(kW4Threads), 0, stream, g);
  else hipLaunchKernelGGL((gemm_w4_kernel<false, false>), grid, dim3(kW4Threads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moe
