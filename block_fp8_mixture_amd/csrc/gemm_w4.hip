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
// Two kernels split the experts by their live rows, as the FP8 GEMM does:
//  - gemm_w4_kernel (experts with at most kW4SmallMax rows, or every expert
//    when the launch's bound says none is larger): a wave task is (expert,
//    32 token rows, 32 weight rows, 1/S of K). A 4-wave workgroup runs 4/S
//    tasks at once; the S waves of a task add their partial sums in LDS in
//    wave order, so the result does not depend on which finishes first. S
//    (1, 2 or 4) is picked on the device so that the tasks fill the grid's
//    waves. Weights and tokens go straight from global memory into the MFMA
//    registers, two K steps ahead.
//  - larger experts, when the launch's bound on 256 x 256 tiles fills the
//    CUs twice: the FP8 GEMM's ping-pong kernel with E2M1 weight slabs
//    (launch_tiled_w4 in gemm.hip);
//  - gemm_w4_tiled_kernel (larger experts otherwise): a workgroup tile is 64
//    token rows x 128 weight rows; the tile's token rows pass through LDS by
//    direct-to-LDS loads (double buffered, one K step ahead, 128-byte rows
//    XOR-swizzled by row pair so the fragment reads are conflict-free) and
//    each wave streams its 32 weight rows from global memory one K step
//    ahead, for the 2 token sub-tiles (4 sub-tiles held twice the registers
//    the accumulators and operands fit in).
// Tasks run expert by expert, token tile by token tile, and the weight tiles
// fastest, so neighbouring tasks share their token rows in L2.
#include "device_common.h"
#include "gemm_device.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kW4Threads = 256;
constexpr int kW4Waves = kW4Threads / 64;
constexpr int kW4Tile = 32;       // token rows and weight rows of a wave task
constexpr int kW4TiledM = 64;     // token rows of a tiled workgroup
constexpr int kW4Subs = kW4TiledM / 32;  // its 32-row token sub-tiles
constexpr int kW4TiledN = 128;    // weight rows of a tiled workgroup (32 per wave)
constexpr int kW4SmallMax = 64;   // experts with more live rows go to the tiled kernel

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

// Exclusive prefix over the experts of units(rows) for the experts `want`
// keeps (0 for the others), into s_pref[0..E]; all threads call it.
template <typename Want, typename Units>
__device__ void w4_prefix(const W4Args& p, Want want, Units units, int* s_pref, int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.num_experts;
  constexpr int kPer = (kMaxExperts + kW4Threads - 1) / kW4Threads;
  int tiles[kPer], run = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid * kPer + i;
    const int rows = e < E ? w4_rows(p, e) : 0;
    tiles[i] = want(rows) ? units(rows) : 0;
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
}

// The expert whose units hold unit u (s_pref ascending, s_pref[0] = 0).
__device__ __forceinline__ int w4_expert_of(const int* s_pref, int E, int u) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pref[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct W4Any {
  __device__ bool operator()(int rows) const { return rows > 0; }
};
struct W4SmallRows {
  __device__ bool operator()(int rows) const { return rows > 0 && rows <= kW4SmallMax; }
};
struct W4LargeRows {
  __device__ bool operator()(int rows) const { return rows > kW4SmallMax; }
};
template <int M>
struct W4TilesOf {
  __device__ int operator()(int rows) const { return (rows + M - 1) / M; }
};

template <bool UE8M0, bool GATHER, bool SMALL_ONLY>
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
  if constexpr (SMALL_ONLY)
    w4_prefix(p, W4SmallRows(), W4TilesOf<kW4Tile>(), s_pref, s_wsum);
  else
    w4_prefix(p, W4Any(), W4TilesOf<kW4Tile>(), s_pref, s_wsum);

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
      e = w4_expert_of(s_pref, E, tm_all);
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


// The loads of one K step of a tiled wave: its weight rows' codes and scale
// bytes, and the activation scale of its token in each sub-tile.
constexpr int kW4StepLoads = 3 + kW4Subs;  // vector loads of load_w: 2 code, 1 scale, 1 per sub
struct W4TStep {
  uint4 w[2];
  uint32_t ws;
  float sa[kW4Subs];
};

template <bool UE8M0, bool GATHER>
__global__ __launch_bounds__(kW4Threads, 2) void gemm_w4_tiled_kernel(W4Args p) {
  __shared__ int s_pref[kMaxExperts + 1];  // exclusive prefix of the token tiles over experts
  __shared__ int s_wsum[kW4Waves];
  __shared__ int s_src[kW4TiledM];         // A row of each token row of the tile (-1: none)
  __shared__ __attribute__((aligned(1024))) uint8_t s_tok[2][kW4TiledM * kGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int E = p.num_experts;
  w4_prefix(p, W4LargeRows(), W4TilesOf<kW4TiledM>(), s_pref, s_wsum);

  const int N = p.n, K = p.k, KB = K / kGroup;
  const int ntn = N / kW4TiledN;
  const int total = s_pref[E] * ntn;
  const v16f zero = {};

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int tm_all = tile / ntn;
    const int n0 = (tile - tm_all * ntn) * kW4TiledN;
    const int e = w4_expert_of(s_pref, E, tm_all);
    const int mt = tm_all - s_pref[e];
    const int rows_here = min(kW4TiledM, w4_rows(p, e) - mt * kW4TiledM);
    const int row0 = w4_seg_start(p, e) + mt * kW4TiledM;

    __syncthreads();  // the previous tile is done with s_src and s_tok
    if (tid < kW4TiledM) {
      int src = -1;
      if (tid < rows_here) {
        const int r = row0 + tid;
        src = GATHER ? p.a_row_map[r] / p.a_row_div : r;
        if (static_cast<unsigned>(src) >= static_cast<unsigned>(p.a_rows)) src = -1;
      }
      s_src[tid] = src;
    }
    __syncthreads();

    // Token staging by direct-to-LDS loads: instruction q of wave w fills the
    // 1 KB at slot (4 q + w) * 64 of a stage (16-byte slots), so lane l lands
    // in row 32 q + 8 w + l / 8, slot l % 8, and fetches the chunk that the
    // row-pair swizzle keeps there. Rows without a source load row 0 of A
    // (never stored).
    const uint8_t* tsrc[kW4Subs];
#pragma unroll
    for (int q = 0; q < kW4Subs; ++q) {
      const int row = 32 * q + 8 * wave + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      const int src = s_src[row];
      tsrc[q] = p.a + static_cast<int64_t>(src < 0 ? 0 : src) * K + chunk * 16;
    }
    auto load_tok = [&](int kb, int buf) {
#pragma unroll
      for (int q = 0; q < kW4Subs; ++q)
        __builtin_amdgcn_global_load_lds(tsrc[q] + kb * kGroup,
                                         (lds_void*)(s_tok[buf] + (4 * q + wave) * 1024), 16, 0, 0);
    };

    // This wave's weight rows and its tokens' scales.
    const int64_t wrow = static_cast<int64_t>(e) * N + n0 + 32 * wave + (lane & 31);
    const uint8_t* wp = p.w + wrow * (K / 2) + 16 * h;
    const uint8_t* sp = p.w_scales + wrow * (K / kMxBlock);
    int tsrc_lane[kW4Subs];
#pragma unroll
    for (int sub = 0; sub < kW4Subs; ++sub) tsrc_lane[sub] = s_src[32 * sub + (lane & 31)];
    auto load_w = [&](int kb, W4TStep& st) {
      st.w[0] = *reinterpret_cast<const uint4*>(wp + kb * 64);
      st.w[1] = *reinterpret_cast<const uint4*>(wp + kb * 64 + 32);
      st.ws = *reinterpret_cast<const uint32_t*>(sp + kb * 4);
#pragma unroll
      for (int sub = 0; sub < kW4Subs; ++sub) {
        const int src = tsrc_lane[sub] < 0 ? 0 : tsrc_lane[sub];
        const int64_t si = static_cast<int64_t>(kb) * p.a_rows + src;
        if constexpr (UE8M0)
          st.sa[sub] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint8_t*>(p.a_scales)[si]) << 23);
        else
          st.sa[sub] = static_cast<const float*>(p.a_scales)[si];
        if (tsrc_lane[sub] < 0) st.sa[sub] = 0.0f;
      }
    };
    v16f acc[kW4Subs];
#pragma unroll
    for (int sub = 0; sub < kW4Subs; ++sub) acc[sub] = zero;
    auto compute = [&](int kb, const W4TStep& st) {
      const uint8_t* buf = s_tok[kb & 1];
#pragma unroll
      for (int sub = 0; sub < kW4Subs; ++sub) {
        const int row = 32 * sub + (lane & 31);
        v16f part = zero;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint4 b0 = *reinterpret_cast<const uint4*>(buf + swz128(row, 4 * kk + h));
          const uint4 b1 = *reinterpret_cast<const uint4*>(buf + swz128(row, 4 * kk + 2 + h));
          const v8i wa = {static_cast<int>(st.w[kk].x), static_cast<int>(st.w[kk].y),
                          static_cast<int>(st.w[kk].z), static_cast<int>(st.w[kk].w), 0, 0, 0, 0};
          const v8i tb = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                          static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                          static_cast<int>(b1.z), static_cast<int>(b1.w)};
          const int sc = static_cast<int>((st.ws >> (8 * (2 * kk + h))) & 0xFFu);
          part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, tb, part, 4, 0, 0, sc, 0, 127);
        }
        acc[sub] += part * st.sa[sub];
        // One sub-tile's fragments at a time: reads of the next are not
        // hoisted above this one's MFMAs (that would hold 32 fragments).
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // One K step: the next step's tokens (direct to the other LDS buffer,
    // free since the last barrier) and weights (to registers), this step's
    // MFMAs, then a wait for this wave's token loads (the weight and scale
    // loads issued after them, kW4StepLoads, may stay in flight) and a barrier.
    auto step = [&](int kb, const W4TStep& cur, W4TStep& nxt) {
      const bool more = kb + 1 < KB;
      if (more) load_tok(kb + 1, (kb + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      if (more) load_w(kb + 1, nxt);
      compute(kb, cur);
      if (more)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4StepLoads));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);  // no scheduling across steps (registers)
    };

    W4TStep s0, s1;
    load_tok(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_w(0, s0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kW4StepLoads));
    lds_barrier();
    int kb = 0;
    for (; kb + 1 < KB; kb += 2) {
      step(kb, s0, s1);
      step(kb + 1, s1, s0);
    }
    if (kb < KB) step(kb, s0, s1);

#pragma unroll
    for (int sub = 0; sub < kW4Subs; ++sub) {
      const int j = 32 * sub + (lane & 31);
      if (j < rows_here) {
        uint16_t* crow = p.c + static_cast<int64_t>(row0 + j) * N + n0 + 32 * wave + 4 * h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v4f v = {acc[sub][4 * g], acc[sub][4 * g + 1], acc[sub][4 * g + 2], acc[sub][4 * g + 3]};
          *reinterpret_cast<uint2*>(crow + 8 * g) = pack_bf16x4(v);
        }
      }
    }
  }
}

}  // namespace

template <bool U, bool M>
static hipError_t launch_w4(const W4Args& g, bool large, hipStream_t stream) {
  const int cus = device_cu_count();
  if (!large) {  // every expert to the wave-task kernel
    hipLaunchKernelGGL((gemm_w4_kernel<U, M, false>), dim3(4 * cus), dim3(kW4Threads), 0, stream, g);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_w4_kernel<U, M, true>), dim3(4 * cus), dim3(kW4Threads), 0, stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The larger experts: the FP8 kernel's 256 x 256 ping-pong tiles with E2M1
  // weight slabs when there are enough tiles to fill the CUs, else 64 x 128
  // tiles here. Both take the experts of more than kW4SmallMax rows.
  static_assert(kW4SmallMax == kStreamMaxRows, "the two large-expert kernels split experts alike");
  GemmArgs t{};
  t.a = g.a;
  t.a_scales = g.a_scales;
  t.fmt = g.fmt;
  t.a_rows = g.a_rows;
  t.a_row_map = g.a_row_map;
  t.a_row_div = g.a_row_div;
  t.w = g.w;
  t.w_scales = nullptr;
  t.w_mx = g.w_scales;
  t.counts = g.counts;
  t.offsets = g.offsets;
  t.num_experts = g.num_experts;
  t.row_cap = g.row_cap;
  t.max_rows_per_expert = g.max_rows_per_expert;
  t.max_live_experts = g.num_experts;
  t.n = g.n;
  t.k = g.k;
  t.c = g.c;
  t.tiles_visited = nullptr;
  t.seg_cap = g.seg_cap;
  if (launch_tiled_w4(t, stream, &e)) return e;
  hipLaunchKernelGGL((gemm_w4_tiled_kernel<U, M>), dim3(2 * cus), dim3(kW4Threads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_w4(const W4Args& g, hipStream_t stream) {
  // The tiled kernel only when some expert can hold more than kW4SmallMax rows.
  const bool large = g.max_rows_per_expert > kW4SmallMax;
  const bool u = g.fmt == kUe8m0, m = g.a_row_map != nullptr;
  if (u && m) return launch_w4<true, true>(g, large, stream);
  if (u) return launch_w4<true, false>(g, large, stream);
  if (m) return launch_w4<false, true>(g, large, stream);
  return launch_w4<false, false>(g, large, stream);
}

}  // namespace moe
