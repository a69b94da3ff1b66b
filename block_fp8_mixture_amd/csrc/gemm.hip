// Grouped FP8 x FP8 GEMM with 128x128 weight block scales and 1x128
// activation scales, over the live rows of each expert segment only.
//
// vLLM PR #59128 (Purpose; SM90 on H200): both grouped GEMMs read the
// prefix-sum expert endpoints and skip unused whole tiles; padding inside a
// partially filled tile is still computed (masked here). TensorRT-LLM PR
// #21250 (description): FP8 x FP8 GEMMs with 128x128 weight scales whose
// grid covers only the expert blocks the batch can occupy; at decode sizes
// most experts are empty and the GEMM must stream weights at bandwidth.
//
// Both kernels compute C^T tiles (weights are the MFMA "A" operand, tokens
// "B"), which makes the weight block scale uniform over a wave and the
// activation scale a single value per lane.
//
// Work is found on the device: every workgroup compacts the experts it owns
// (by row count) from expert_counts into LDS, then walks its share of the
// resulting item list, so padded capacity and empty experts cost nothing.
//
//  * gemm_stream_kernel -- experts with 1..64 rows, on
//    v_mfma_f32_16x16x128_f8f6f4 (one MFMA = one 128-wide scale block; 16x16
//    result with token = lane % 16, weight row = 4 * (lane / 16) + v). An item
//    is (expert, 16*WN weight rows); the 4 waves split it as WN row blocks x
//    KSPLIT K ranges and walk the expert's 16-row token tiles. Each K block
//    is one MFMA into a zeroed temporary and four FMAs acc += t * (sa * sw);
//    K-split partial sums are added in a fixed order through LDS. This is the
//    weight-streaming (HBM-bound) path.
//  * gemm_tiled_kernel -- experts with more rows: persistent, XCD-grouped
//    256 x 256 tiles (256 x 128 or 256 x 64 when wide tiles would leave CUs
//    idle, picked on the device) on v_mfma_f32_32x32x64_f8f6f4, operands
//    staged through a 4-deep LDS ring of 64-byte K stages by direct-to-LDS
//    loads, scales applied by rescaling the accumulator once per 128-wide
//    block. The 256-wide kernel runs a ping-pong schedule (the two waves of a
//    SIMD alternate MFMA and load phases) and also serves MXFP4 weights
//    (launch_tiled_w4: E2M1 weight slabs, the E8M0 scales applied by the
//    scaled MFMA). Between tiles, the next tile's coordinates, row-map
//    entries and weight scales load during the output staging, and its
//    first stages go out during the output stores. Details at the kernel.
#include <type_traits>

#include "device_common.h"
#include "gemm_device.h"
#include "kernels.h"
#include "quant_device.h"

namespace moe {
namespace {

constexpr int kThreads = 256;


// Segment of expert e: from the endpoints, or the batched layout's fixed
// rows [e*seg_cap, (e+1)*seg_cap).
__device__ __forceinline__ int seg_start(const GemmArgs& p, int e) {
  return p.seg_cap > 0 ? e * p.seg_cap : p.offsets[e];
}
__device__ __forceinline__ int seg_end(const GemmArgs& p, int e) {
  return p.seg_cap > 0 ? (e + 1) * p.seg_cap : p.offsets[e + 1];
}

__device__ __forceinline__ int expert_rows(const GemmArgs& p, int e) {
  return segment_rows(seg_start(p, e), seg_end(p, e), p.counts[e], p.row_cap);
}

// A row feeding output row r, or -1 when the map points outside A. GATHER
// is whether a row map is given (the kernels are specialised on it).
template <bool GATHER>
__device__ __forceinline__ int a_source_row(const GemmArgs& p, int r) {
  const int ar = GATHER ? p.a_row_map[r] / p.a_row_div : r;
  return static_cast<unsigned>(ar) < static_cast<unsigned>(p.a_rows) ? ar : -1;
}

// Ordered compaction of the experts whose row count satisfies `want`, into
// s_list[0..n). s_pref[i] gets the exclusive prefix sum of units(count) over
// the listed experts and s_pref[n] the total; when s_cnt / s_row0 are given
// they get each listed expert's live rows and first row (s_cnt == s_list
// packs the expert id into bits 0..15 and the rows above them, for counts
// below 2^15). Returns n. All threads call it.
template <int NT, typename Want, typename Units>
__device__ int build_expert_list(const GemmArgs& p, Want want, Units units, int* s_list,
                                 int* s_pref, int* s_tmp, int* s_cnt = nullptr,
                                 int* s_row0 = nullptr) {
  const int num_experts = p.num_experts;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kW = NT / 64;
  constexpr int kC = (kMaxExperts + NT - 1) / NT;
  // All metadata loads are issued before the first wait (unconditionally,
  // at a clamped index, so no branch separates them).
  int cnts[kC], row0s[kC];
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int e = c * NT + tid < num_experts ? c * NT + tid : num_experts - 1;
    row0s[c] = seg_start(p, e);
    cnts[c] = seg_end(p, e);
    cnts[c] = segment_rows(row0s[c], cnts[c], p.counts[e], p.row_cap);
    if (c * NT + tid >= num_experts) cnts[c] = 0;
  }
  int run_n = 0, run_u = 0;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int base = c * NT;
    if (base >= num_experts) break;
    const int e = base + tid;
    const int cnt = cnts[c];
    const bool flag = e < num_experts && want(cnt);
    const int u = flag ? units(cnt) : 0;
    const uint64_t mask = __ballot(flag);
    const int pos = __popcll(mask & ((uint64_t(1) << lane) - 1));
    int incl = u;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) {
      s_tmp[wave] = __popcll(mask);
      s_tmp[kW + wave] = incl;
    }
    __syncthreads();
    int bn = run_n, bu = run_u;
    for (int w = 0; w < wave; ++w) {
      bn += s_tmp[w];
      bu += s_tmp[kW + w];
    }
    if (flag) {
      if (s_cnt != s_list) s_list[bn + pos] = e;
      s_pref[bn + pos] = bu + incl - u;
      if (s_cnt == s_list) {  // packed: expert id in bits 0..15, count above
        s_list[bn + pos] = e | (cnt << 16);
        s_row0[bn + pos] = row0s[c];
      } else if (s_cnt) {
        s_cnt[bn + pos] = cnt;
        s_row0[bn + pos] = row0s[c];
      }
    }
    for (int w = 0; w < kW; ++w) {
      run_n += s_tmp[w];
      run_u += s_tmp[kW + w];
    }
    __syncthreads();
  }
  if (tid == 0) s_pref[run_n] = run_u;
  __syncthreads();
  return run_n;
}

struct WantSmall {
  __device__ bool operator()(int c) const { return c > 0 && c <= kStreamMaxRows; }
};
struct WantLarge {
  __device__ bool operator()(int c) const { return c > kStreamMaxRows; }
};
struct NoUnits {
  __device__ int operator()(int) const { return 0; }
};
struct TiledUnits {
  __device__ int operator()(int c) const { return (c + kTiledTileM - 1) / kTiledTileM; }
};

// ---------------------------------------------------------------- streaming

struct TokenTiles {
  __device__ int operator()(int c) const { return (c + kStreamTileM - 1) / kStreamTileM; }
};

// Task t of the ordered list of a kernel whose tasks are (expert, block of
// weight rows, 16-row token tile): expert L.list[i], weight block rb, token
// rows [16 mt, 16 mt + 16) of the expert's segment. Decoded from LDS only,
// so finding a task never waits on global memory.
struct StreamTask {
  int e, rb, mt, cnt, row0;
};

struct StreamLists {
  const int* list;  // expert id | live rows << 16
  const int* pref;
  const int* row0;
  int n;
};

// t is uniform over the wave; readfirstlane tells the compiler so, which
// keeps the task bookkeeping in scalar registers and branches. The entry is
// found by the whole wave at once: the prefixes are strictly increasing
// from pref[0] = 0, so the last entry with pref <= key is the number of
// entries i >= 1 with pref[i] <= key -- one LDS read per lane and a ballot
// per 64 entries, instead of a chain of dependent reads.
__device__ __forceinline__ StreamTask stream_task(const StreamLists& L, int n_rb, int t) {
  const int key = t / n_rb;
  const int lane = threadIdx.x & 63;
  int lo = 0;
  for (int base = 1; base < L.n; base += 64) {
    const int i = base + lane;
    const uint64_t le = __ballot(i < L.n && L.pref[i] <= key);
    lo += __popcll(le);
    if (~le != 0) break;  // an entry past the key (or the list's end) in this round
  }
  lo = __builtin_amdgcn_readfirstlane(lo);
  StreamTask r;
  const int packed = __builtin_amdgcn_readfirstlane(L.list[lo]);
  r.e = packed & 0xFFFF;
  r.cnt = packed >> 16;
  const int p0 = __builtin_amdgcn_readfirstlane(L.pref[lo]);
  const int n_mt = __builtin_amdgcn_readfirstlane(L.pref[lo + 1]) - p0;
  const int local = t - p0 * n_rb;
  r.rb = local / n_mt;
  r.mt = local % n_mt;
  r.row0 = __builtin_amdgcn_readfirstlane(L.row0[lo]);
  return r;
}


// The LDS reads of one streaming stage: weight and token fragments (two
// 16-byte halves each, 1 KB apart) and the two scales. Written as assembly
// with its own lgkmcnt wait, so the compiler neither sees LDS reads that
// might alias the direct-to-LDS loads in flight into other stages (it would
// make them wait for every vector-memory operation) nor can use a result
// early. Outputs are early-clobber: none may share a register with an
// address that a later read of the block still needs.
__device__ __forceinline__ void read_stage(uint32_t w0_addr, uint32_t w1_addr, uint32_t a0_addr,
                                           uint32_t a1_addr, uint32_t sa_addr, uint32_t sw_addr,
                                           uint4& w0, uint4& w1, uint4& a0, uint4& a1,
                                           uint32_t& sa, uint32_t& sw) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b32 %4, %10\n\t"
      "ds_read_b32 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w0), "=&v"(w1), "=&v"(a0), "=&v"(a1), "=&v"(sa), "=&v"(sw)
      : "v"(w0_addr), "v"(w1_addr), "v"(a0_addr), "v"(a1_addr), "v"(sa_addr), "v"(sw_addr));
}


// Two ways to cut the work into tasks, chosen per launch on the device:
//  A: (expert, 64 weight rows, 16-token tile); the 4 waves own 16 weight rows
//     each; a stage is one 128-wide K block (64 rows x 128 B of weights).
//  B, when there are fewer A tasks than about 3/4 of the workgroups (few live
//     experts): (expert, 16 weight rows, 16-token tile); a stage is 4
//     consecutive K blocks, one per wave, and the waves' partial sums are
//     added in LDS in wave order at the end of the task. Four times as many
//     tasks, so few live experts still keep every CU streaming.
constexpr int kSRowsA = 64;  // weight rows of an A task
constexpr int kSRowsB = 16;  // weight rows of a B task
// A stage: [W: wave w's rows 16w..16w+15, 128 B each, swz128] 8 KB,
//          [tokens: 16 rows x 128 B, swz128] 2 KB,
//          [token scales: 64 x 4 B, lane l -> token l % 16] [weight scale].
// B stage: [W of K block w: 16 rows x 128 B, swz128] 4 x 2 KB,
//          [tokens of K block w: 16 rows x 128 B, swz128] 4 x 2 KB,
//          [token scales: lane l -> K block l / 16, token l % 16]
//          [weight scales: lane l -> K block l % 4].
constexpr int kOffTokA = kSRowsA * kGroup;
constexpr int kOffSclA = kOffTokA + kStreamTileM * kGroup;
constexpr int kSStageA = kOffSclA + 512;  // 10752
constexpr int kOffTokB = 4 * 2048;
constexpr int kOffSclB = 8 * 2048;
constexpr int kSStageB = kOffSclB + 512;  // 16896
constexpr int kSDA = 6;                   // stages in an A ring
constexpr int kSDB = 4;                   // stages in a B ring
constexpr int kSLoadsA = 3;               // loads per wave and stage
constexpr int kSLoadsB = 5;
constexpr int kSRing = kSDA * kSStageA > kSDB * kSStageB ? kSDA * kSStageA : kSDB * kSStageB;
constexpr int kSGroupsPerCu = 2;          // streaming workgroups per CU

// One wave's fp32 partial (16 B per lane) to LDS, and the in-order sum of the
// 4 waves' partials (1 KB apart), as assembly for the same reason as
// read_stage.
__device__ __forceinline__ void lds_store_v4f(uint32_t addr, v4f v) {
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ v4f lds_sum4_v4f(uint32_t addr) {
  v4f a, b, c, d;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(addr));
  return ((a + b) + c) + d;
}

// Decode-sized experts (1..64 rows): weight streaming, bound by HBM.
//
// Tasks are ordered expert-major, then weight block, then token tile, and
// consecutive tasks go to workgroups on the same XCD, so the token tiles of
// one weight block (at most 4) share its reads in L2. The stages of a
// workgroup's tasks form one stream, staged through a ring of LDS buffers by
// direct-to-LDS loads issued (ring - 1) stages ahead, so loads stay in
// flight across task boundaries. Each load moves whole 128-byte lines (8 rows
// x 128 bytes): the number of lines a CU can have in flight, not bytes, is
// what bounds its share of HBM bandwidth. Every wave issues the same number
// of loads per stage, so one vmcnt immediate fits all waves.
//
// Per K block: one v_mfma_f32_16x16x128_f8f6f4 into a zeroed temporary
// (result: token = lane % 16, weight row = 4 * (lane / 16) + v), then
// acc += t * (sa * sw) with four FMAs. Lanes whose token is past the expert's
// rows load stand-in data from valid addresses and are never stored.
//
// GATED (FC1 of a decode layer, weight rows = [gate; up]): each 16-row block
// holds gate columns j..j+7 in its rows 0..7 and the up columns j..j+7 in
// rows 8..15, so after the last K block a lane of the lower half holds
// gate values whose up partners sit 32 lanes higher; one cross-lane swap
// brings them together and the activation is applied to the BF16-rounded
// pair (the values C holds), written in fp32 for the FC2 prologue.
template <bool UE8M0, bool GATHER, bool GATED>
__global__ __launch_bounds__(kThreads, kSGroupsPerCu) void gemm_stream_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kSRing];
  __shared__ int s_list[kMaxExperts];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_tmp[2 * kThreads / 64];
  __shared__ int s_row0[kMaxExperts];

  const int n_list = build_expert_list<kThreads>(p, WantSmall(), TokenTiles(), s_list, s_pref,
                                                 s_tmp, s_list, s_row0);
  const StreamLists L{s_list, s_pref, s_row0, __builtin_amdgcn_readfirstlane(n_list)};
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = p.n, K = p.k, KB = K / kGroup;
  const int I = N / 2;  // GATED: gate rows [0, I), up rows [I, N)
  const int tiles = __builtin_amdgcn_readfirstlane(s_pref[L.n]);
  const int G = gridDim.x;
  // The stage loop is compiled once per task shape (mode), so neither
  // carries the other's instructions.
  auto run = [&](auto mode_tag) {
    constexpr bool modeB = decltype(mode_tag)::value;
    constexpr int rows_t = modeB ? kSRowsB : kSRowsA;  // weight rows per task
    const int n_rb = N / rows_t;
    const int n_tasks = tiles * n_rb;
    const int per_task = modeB ? (KB + 3) / 4 : KB;  // stages per task
    constexpr int SS = modeB ? kSStageB : kSStageA;
    constexpr int D = modeB ? kSDB : kSDA;
    const int vid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    if (vid >= n_tasks) return;  // uniform over the workgroup; no barrier has been passed yet
    const int total = ((n_tasks - vid + G - 1) / G) * per_task;  // stages this workgroup streams
    const int tok = lane & 15;
    const int grow = lane >> 3;

    // ---- issue side. Loads move whole 128-byte lines: lane l covers row
    // 8 h + l / 8 of a 16-row slab (h = 0, 1) and 16-byte chunk
    // (l % 8) ^ ((row >> 1) & 7), which lands in LDS slot l % 8 (swz128).
    int i_task = vid, i_st = 0;
    const uint8_t* i_w0 = nullptr;  // this lane's weight bytes at K block 0, slab rows 0..7
    const uint8_t* i_w1 = nullptr;  //   slab rows 8..15
    const uint8_t* i_t0 = nullptr;  // token bytes: A, the wave's token half; B, tokens 0..7
    const uint8_t* i_t1 = nullptr;  // B: tokens 8..15
    const uint8_t* i_s = nullptr;   // scale loads (A: waves 2, 3; B: all waves, fifth load)
    int64_t i_sstep = 0;            // their bytes per K block
    auto chunk_of = [&](int row) { return ((lane & 7) ^ ((row >> 1) & 7)) << 4; };
    auto start_task = [&](int t) {
      const StreamTask k = stream_task(L, n_rb, t);
      // A: the wave's 16 of the task's 64 rows. B: the task's 16 rows.
      // GATED: 8 gate rows from jg and the 8 up rows of the same columns.
      const int r0 = k.rb * rows_t + (modeB ? 0 : wave * 16);
      const int jg = k.rb * (rows_t / 2) + (modeB ? 0 : wave * 8);
      const int rlo = GATED ? jg : r0, rhi = GATED ? I + jg : r0 + 8;
      const uint8_t* we = p.w + static_cast<int64_t>(k.e) * N * K;
      i_w0 = we + (rlo + grow) * static_cast<int64_t>(K) + chunk_of(grow);
      i_w1 = we + (rhi + grow) * static_cast<int64_t>(K) + chunk_of(grow + 8);
      const float* ws_e = p.w_scales + static_cast<int64_t>(k.e) * (N / kGroup) * KB;
      // Weight scale rows of the lower and upper 8 rows (one block unless GATED).
      const uint8_t* wsp = reinterpret_cast<const uint8_t*>(ws_e + (rlo / kGroup) * KB);
      const uint8_t* wsp_hi = reinterpret_cast<const uint8_t*>(ws_e + (rhi / kGroup) * KB);
      // Tokens whose rows this lane loads (ta, tb) and whose scale it loads
      // (tok). Row-map entries come via the scalar cache, each index kept
      // inside the expert's segment.
      const int first = k.mt * kStreamTileM;
      const int last = k.row0 + k.cnt - 1;
      const int ta = modeB ? grow : wave * 8 + grow;
      const int tb = grow + 8;
      int ra = k.row0 + first + ta, rb = k.row0 + first + tb, rs = k.row0 + first + tok;
      if constexpr (GATHER) {
        int ma = 0, mb = 0, ms = 0;
#pragma unroll
        for (int i = 0; i < kStreamTileM; ++i) {
          const int r = k.row0 + first + i < last ? k.row0 + first + i : last;
          const int v = scalar_load(p.a_row_map + r);
          ma = ta == i ? v : ma;
          mb = tb == i ? v : mb;
          ms = tok == i ? v : ms;
        }
        ra = ma / p.a_row_div;
        rb = mb / p.a_row_div;
        rs = ms / p.a_row_div;
      }
      auto valid = [&](int tk, int ar) {
        return first + tk < k.cnt && static_cast<unsigned>(ar) < static_cast<unsigned>(p.a_rows);
      };
      // Stand-ins for idle lanes: the lane's own weight bytes, or the weight
      // scales (valid addresses for every K block).
      i_t0 = valid(ta, ra) ? p.a + static_cast<int64_t>(ra) * K + chunk_of(ta) : i_w0;
      i_t1 = valid(tb, rb) ? p.a + static_cast<int64_t>(rb) * K + chunk_of(tb) : i_w1;
      const bool loads_sa = modeB ? wave == 0 : wave == 2;
      if (loads_sa && valid(tok, rs)) {
        i_s = static_cast<const uint8_t*>(p.a_scales) + static_cast<int64_t>(rs) * (UE8M0 ? 1 : 4);
        i_sstep = static_cast<int64_t>(p.a_rows) * (UE8M0 ? 1 : 4);
      } else {
        // Weight scales. GATED: lanes whose copy serves the upper 8 rows (A:
        // lanes 32..63; B: lanes with bit 2 set) load the up rows' scale.
        const bool hi = GATED && (modeB ? ((lane >> 2) & 1) != 0 : lane >= 32);
        i_s = hi ? wsp_hi : wsp;
        i_sstep = 4;
      }
    };
    auto issue = [&](uint8_t* st) {
      if constexpr (!modeB) {
        const int kb = i_st;
        __builtin_amdgcn_global_load_lds(i_w0 + kb * kGroup, (lds_void*)(st + wave * 2048), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(i_w1 + kb * kGroup, (lds_void*)(st + wave * 2048 + 1024), 16, 0, 0);
        if (wave < 2)
          __builtin_amdgcn_global_load_lds(i_t0 + kb * kGroup, (lds_void*)(st + kOffTokA + wave * 1024), 16, 0, 0);
        else if (wave == 2 && UE8M0)
          __builtin_amdgcn_global_load_lds(i_s + kb * i_sstep, (lds_void*)(st + kOffSclA), 1, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(i_s + kb * i_sstep, (lds_void*)(st + kOffSclA + (wave - 2) * 256), 4, 0, 0);
      } else {
        const int kb = min(4 * i_st + wave, KB - 1);  // past the end: clamped, never used
        __builtin_amdgcn_global_load_lds(i_w0 + kb * kGroup, (lds_void*)(st + wave * 2048), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(i_w1 + kb * kGroup, (lds_void*)(st + wave * 2048 + 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(i_t0 + kb * kGroup, (lds_void*)(st + kOffTokB + wave * 2048), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(i_t1 + kb * kGroup, (lds_void*)(st + kOffTokB + wave * 2048 + 1024), 16, 0, 0);
        // Wave 0: token scales of the stage's 4 K blocks (lane l, block l / 16).
        // Waves 1..3: the weight scales (lane l, block l % 4; waves 2 and 3
        // store the same values as wave 1).
        const int kbs = min(4 * i_st + (wave == 0 ? lane >> 4 : lane & 3), KB - 1);
        if (wave == 0 && UE8M0)
          __builtin_amdgcn_global_load_lds(i_s + kbs * i_sstep, (lds_void*)(st + kOffSclB), 1, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(i_s + kbs * i_sstep, (lds_void*)(st + kOffSclB + (wave == 0 ? 0 : 256)), 4, 0, 0);
      }
      if (++i_st == per_task) {
        i_st = 0;
        i_task += G;
        if (i_task < n_tasks) start_task(i_task);
      }
    };

    // ---- compute side
    int c_task = vid, c_st = 0;
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const uint8_t* st) {
      const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(st));
      const int c0 = 2 * (lane >> 4);  // fragment chunks c0, c0 + 1 of row tok
      if (c_st == 0) acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      const bool active = !modeB || 4 * c_st + wave < KB;  // B: this wave's K block exists
      if (active) {
        union {
          uint4 u[2];
          v8i v;
        } wf, af;
        uint32_t sraw, swraw;
        const uint32_t wr = base + wave * 2048;
        const uint32_t tr = modeB ? base + kOffTokB + wave * 2048 : base + kOffTokA;
        const uint32_t sa = modeB ? base + kOffSclB + (wave * 16 + tok) * 4 : base + kOffSclA + tok * 4;
        // Result rows 8..15 (lanes 32..63) take the upper rows' weight scale.
        const int hi = GATED ? lane >> 5 : 0;
        const uint32_t sw = modeB ? base + kOffSclB + 256 + (wave + 4 * hi) * 4
                                  : base + kOffSclA + 256 + hi * 128;
        read_stage(wr + swz128(tok, c0), wr + swz128(tok, c0 + 1), tr + swz128(tok, c0),
                   tr + swz128(tok, c0 + 1), sa, sw, wf.u[0], wf.u[1], af.u[0], af.u[1], sraw, swraw);
        const float fa = UE8M0 ? __uint_as_float(sraw << 23) : __uint_as_float(sraw);
        acc = fma4(mfma_fp8(wf.v, af.v), fa * __uint_as_float(swraw), acc);
      }
      if (++c_st < per_task) return;
      const StreamTask k = stream_task(L, n_rb, c_task);
      const int j = k.mt * kStreamTileM + tok;
      uint16_t* crow = p.c + static_cast<int64_t>(k.row0 + j) * N + k.rb * rows_t + 4 * (lane >> 4);
      const bool count_tile = threadIdx.x == 0 && p.tiles_visited && (k.rb * rows_t) % kColTile == 0;
      // GATED epilogue of one 16-row block with first gate column jg.
      auto gated_store = [&](v4f v, int jg) {
        const uint2 packed = pack_bf16x4(v);
        const int col = (lane < 32 ? jg : I + jg) + 4 * ((lane >> 4) & 1);
        const int64_t row = k.row0 + j;
        uint2 other;
        other.x = __shfl_xor(packed.x, 32, 64);
        other.y = __shfl_xor(packed.y, 32, 64);
        if (j >= k.cnt) return;
        *reinterpret_cast<uint2*>(p.c + row * N + col) = packed;
        if (lane >= 32) return;
        const double lim = p.act_limit;
        float4 a;
        a.x = swiglu_any(p.act, bf16_to_f32(packed.x & 0xFFFFu), bf16_to_f32(other.x & 0xFFFFu), lim, p.rounding);
        a.y = swiglu_any(p.act, bf16_to_f32(packed.x >> 16), bf16_to_f32(other.x >> 16), lim, p.rounding);
        a.z = swiglu_any(p.act, bf16_to_f32(packed.y & 0xFFFFu), bf16_to_f32(other.y & 0xFFFFu), lim, p.rounding);
        a.w = swiglu_any(p.act, bf16_to_f32(packed.y >> 16), bf16_to_f32(other.y >> 16), lim, p.rounding);
        *reinterpret_cast<float4*>(p.act_out + row * I + col) = a;
      };
      if constexpr (!modeB) {
        if constexpr (GATED)
          gated_store(acc, k.rb * (kSRowsA / 2) + wave * 8);
        else if (j < k.cnt)
          *reinterpret_cast<uint2*>(crow + wave * 16) = pack_bf16x4(acc);
      } else {
        // Every wave is done reading this stage once all pass the barrier; its
        // first 4 KB then hold the 4 partials, summed by wave 0 in wave order.
        // (The buffer is refilled only after the next stage's barrier.)
        lds_barrier();
        lds_store_v4f(base + wave * 1024 + lane * 16, acc);
        lds_barrier();
        if (wave == 0) {
          const v4f sum = lds_sum4_v4f(base + lane * 16);
          if constexpr (GATED)
            gated_store(sum, k.rb * (kSRowsB / 2));
          else if (j < k.cnt)
            *reinterpret_cast<uint2*>(crow) = pack_bf16x4(sum);
        }
      }
      if (count_tile) atomicAdd(p.tiles_visited, 1);
      c_st = 0;
      c_task += G;
    };

    start_task(i_task);
    for (int d = 0; d < D - 1; ++d)
      if (d < total) issue(s_ring + d * SS);
    // Stage s: wait for this wave's loads of stage s (in the steady state
    // stages s+1 .. s+D-2 are still in flight, near the end fewer, and then
    // everything is waited for), barrier so every wave's part is visible and
    // stage s-1 is free, issue stage s+D-1 into it, compute s.
    int slot = 0;  // s % D
    for (int s = 0; s < total; ++s) {
      if (s + D - 2 >= total)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((modeB ? kSLoadsB : kSLoadsA) * (D - 2)));
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      const int prev = slot == 0 ? D - 1 : slot - 1;
      if (s + D - 1 < total) issue(s_ring + prev * SS);
      compute(s_ring + slot * SS);
      slot = slot == D - 1 ? 0 : slot + 1;
    }
  };
  if (4 * tiles * (N / kSRowsA) < 3 * G)
    run(std::true_type{});
  else
    run(std::false_type{});
}

hipError_t launch_stream(const GemmArgs& g, hipStream_t stream) {
  const int grid = device_cu_count() * kSGroupsPerCu;
  const bool u = g.fmt == kUe8m0, m = g.a_row_map != nullptr;
  if (g.act_out) {
    if (!m) return hipErrorInvalidValue;
    if (u) hipLaunchKernelGGL((gemm_stream_kernel<true, true, true>), dim3(grid), dim3(kThreads), 0, stream, g);
    else hipLaunchKernelGGL((gemm_stream_kernel<false, true, true>), dim3(grid), dim3(kThreads), 0, stream, g);
  }
  else if (u && m) hipLaunchKernelGGL((gemm_stream_kernel<true, true, false>), dim3(grid), dim3(kThreads), 0, stream, g);
  else if (u) hipLaunchKernelGGL((gemm_stream_kernel<true, false, false>), dim3(grid), dim3(kThreads), 0, stream, g);
  else if (m) hipLaunchKernelGGL((gemm_stream_kernel<false, true, false>), dim3(grid), dim3(kThreads), 0, stream, g);
  else hipLaunchKernelGGL((gemm_stream_kernel<false, false, false>), dim3(grid), dim3(kThreads), 0, stream, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tiled

constexpr int TM = kTiledTileM;   // token rows per tile (256)
constexpr int TN = 256;           // weight rows per tile (the narrow variant: 64)
constexpr int SK = 64;            // K bytes per pipeline stage (half a scale block)
constexpr int kTiledThreads = 512;
constexpr int kStageA = TM * SK;              // token part of a stage (16 KB)
constexpr int kStageBytes = (TM + TN) * SK;   // 32 KB
constexpr int kMaxKBlocks = 256;              // K <= 32768 on this path
// Scales below this are treated as this value inside the accumulator's
// normalizer: a block whose scale is zero then adds 2^-64 times its raw dot
// products (about 1e-20 of any real block's contribution) instead of making
// the ratios overflow.
constexpr float kScaleFloor = 5.42101086e-20f;  // 2^-64

typedef float v16f __attribute__((ext_vector_type(16)));

// Byte offset of 16-byte chunk c (0..3) of row `row` in a [rows][64 B] LDS
// slab. gfx950's LDS has 64 four-byte banks, so rows r, r+4, r+8, r+12 start
// on the same bank; XOR-ing the chunk with (row >> 2) & 3 gives the 16 lanes
// one ds_read_b128 cycle serves (16 consecutive rows, same chunk) 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int c) { return row * SK + ((c ^ ((row >> 2) & 3)) << 4); }

union Frag {
  uint4 u[2];
  v8i v;
};


// Tile `local` of an expert with mt row tiles: weight column tile local / mt,
// row tile local % mt. Consecutive tiles go to one XCD, so a round of its
// workgroups covers a few column tiles x all row tiles of an expert, and each
// weight slab is read by workgroups that share its XCD's L2 at about the
// same time. (Grouping 4, 8 or 16 column tiles x all row tiles measured
// 0.2-5% slower at 4096 tokens.)
__device__ __forceinline__ void tile_coords(int local, int mt, int* m, int* n) {
  *n = local / mt;
  *m = local - *n * mt;
}

// A tile of the large-expert GEMM: its expert's weights, first output row,
// live rows and first weight row, and the per-lane offsets of its operand
// loads. The kernel prepares the next tile's while one finishes, and the
// next tile's first stages go out during the output stores. (Namespace
// scope: as local classes of the kernel template, hipcc's host pass emits
// no launch stubs for the kernel.)
struct TiledTile {
  const uint8_t* wb;
  int e, row0, rows_here, n0, sa_row;
  uint32_t aoff[2], woff[2];
};
// A tile before its row-map entries have arrived: raw[0..1] are the map
// entries (or output rows) of the lane's two staged rows, raw[2] its
// token's.
struct TiledTileFetch {
  int e, row0, rows_here, n0;
  int raw[3];
};

// Large-expert GEMM. A workgroup computes a 256 token x TNT weight tile
// (TNT = 256, or 128 or 64 -- picked on the device, see PICK -- when wide
// tiles would leave CUs idle) with 8 waves as 4 (tokens) x 2 (weights);
// wave (wm, wn) owns tokens
// [64 wm, 64 wm + 64) x weights [TNT/2 wn, TNT/2 (wn + 1)), as 2 x TNT/64
// tiles of v_mfma_f32_32x32x64_f8f6f4 (weights are the MFMA "A" operand,
// tokens "B"; lane l holds token l % 32 and 16 weight rows, so the token
// scale is one value per lane and the weight block scale one value per
// wave). The narrower variants keep the stage layout: W slab rows past TNT
// are neither loaded nor read.
//
// K is walked in 64-byte stages: both operand slabs of a stage (256 x 64 B
// each, 32 KB) are staged in LDS by direct-to-LDS loads through a ring of 4
// stages issued 3 stages ahead; a 128-wide scale block is two stages.
//
// Scales: the accumulator is kept in units of the current block's scale
// s = sa[token] * sw. At the first stage of each block it is multiplied by
// s_prev / s (the token part comes precomputed from LDS, the weight part is
// one value per wave), then the MFMAs add the block's raw FP8 dot products
// into it; the epilogue multiplies by the last s. One VALU multiply per
// element and block, no temporaries, no wait on an MFMA result. Power-of-two
// ratios are exact.
//
// Output (SOUT): the 256-wide kernel stages the BF16 tile in LDS and stores
// whole 16-byte row chunks; the narrow kernels store each lane's 8-byte
// pieces straight from the accumulators.
//
// W4: MXFP4 weights (E2M1 codes two per byte, one E8M0 byte per 32 along K;
// p.w_mx holds the bytes, [E, N, K/32]), 256-wide tiles only. A stage's
// weight slab is then 256 rows x 32 bytes (one load per wave; 16-byte
// chunks XOR-swizzled by bit 3 of the row, which keeps the fragment reads
// conflict-free), and at each block start waves 4..7 load the tile rows' 4
// scale bytes of the block in place of the sink load. The MFMA is the scaled
// one with the E2M1 weights as operand A (a lane holds K values [32 h, 32 h +
// 32) of its row, h = lane / 32, and that MX block's byte as its scale) and
// the tokens as operand B (16-byte chunks h and 2 + h of the stage's 64, the
// order the matrix core pairs with E2M1, as measured); the accumulator's
// normalizer is the token scale alone. With UE8M0 token scales the token's
// byte is B's scale operand and the accumulator is never rescaled: every
// factor is a power of two, so the result is bit-identical to rescaling.
template <bool UE8M0, bool GATHER, int TNT, bool PICK, bool SOUT, bool W4 = false>
__global__ __launch_bounds__(kTiledThreads, 1) void gemm_tiled_kernel(GemmArgs p) {
  static_assert(TNT == 256 || TNT == 128 || TNT == 64, "tile widths");
  static_assert(!PICK || TNT != 256, "the pick is between 64 and 128");
  static_assert(!W4 || (TNT == 256 && !PICK), "MXFP4 weights: the 256-wide kernel");
  constexpr int WN = TNT / 2;   // weight rows of a wave
  constexpr int WT = WN / 32;   // its 32-row MFMA tiles
  constexpr int LPS = W4 ? 3 : TNT == 256 ? 4 : 3;  // direct-to-LDS loads per wave and stage
  // MXFP4 weights with UE8M0 token scales: both scales are powers of two and
  // the scaled MFMA applies both (the token's byte as B's scale), so the
  // accumulator holds the result itself and is never rescaled.
  constexpr bool kHwScales = W4 && UE8M0;
  // Four stages and two token-scale buffers, all distinct objects, so the
  // compiler can tell that a read never aliases a direct-to-LDS load in
  // flight and does not wait for the prefetch.
  __shared__ __attribute__((aligned(1024))) uint8_t s_st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_st1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_st2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_st3[kStageBytes];
  __shared__ uint32_t s_sr0[TM];  // raw token scales of even / odd scale blocks
  __shared__ uint32_t s_sr1[TM];  // (UE8M0 bytes arrive zero-extended)
  __shared__ uint32_t s_srx[TM];  // sink of waves 4..7's copy of the scale loads
  __shared__ uint32_t s_wsc[W4 ? 2 * TM : 1];  // W4: rows' scale bytes of even / odd blocks
  __shared__ __attribute__((aligned(16))) float s_rt[2][TM];  // token scale ratio of a block
  __shared__ float s_sl[TM];                                  // token scale of the last block
  __shared__ float s_wsf[2 * kMaxKBlocks];  // weight block scales of the tile, [block][K block] with row stride KB
  __shared__ int s_list[kMaxExperts];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_cnt[kMaxExperts];   // listed expert -> its live rows
  __shared__ int s_row0[kMaxExperts];  //   and its first row
  __shared__ int s_tmp[2 * kTiledThreads / 64];

  const int n_list = build_expert_list<kTiledThreads>(p, WantLarge(), TiledUnits(), s_list,
                                                      s_pref, s_tmp, s_cnt, s_row0);
  if constexpr (PICK) {
    // The 64- and 128-wide kernels are launched together on the same grid;
    // both find the same row tiles and agree on which one runs: the fewer
    // rounds of tiles over the grid times the relative time of one tile
    // (measured at K = 6144: 64 -> 20, 128 -> 23; a tile streams 256 token
    // rows and TNT weight rows per stage). The other exits here.
    const int rows = s_pref[n_list], G = gridDim.x;
    auto cost = [&](int w, int c) { return (rows * (p.n / w) + G - 1) / G * c; };
    if ((cost(64, 20) < cost(128, 23)) != (TNT == 64)) return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Waves are spread over the 4 SIMDs round-robin; pairing (wm, wn) as
  // below puts the two waves of a 64-token slice on different SIMDs, so a
  // tail tile of up to 128 rows still keeps all four SIMDs busy.
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int N = p.n, K = p.k, KB = K / kGroup, NS = K / SK;
  const int nt = (N + TNT - 1) / TNT;
  const int total = s_pref[n_list] * nt;
  const int G = gridDim.x;
  // Persistent grid: consecutive tiles go to one XCD (workgroups are
  // dispatched round-robin over the 8 XCDs).
  const int vid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const int tok = tid & (TM - 1);

  auto tile_fetch = [&](int tile) {
    TiledTileFetch f;
    const int tm_all = tile / nt;
    int lo = 0, hi = n_list - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= tm_all) lo = mid; else hi = mid - 1;
    }
    f.e = __builtin_amdgcn_readfirstlane(s_list[lo]);
    const int mt_e = s_pref[lo + 1] - s_pref[lo];
    int mt, ntile;
    tile_coords(tile - s_pref[lo] * nt, mt_e, &mt, &ntile);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[lo]);
    f.rows_here = min(TM, cnt - mt * TM);
    f.row0 = __builtin_amdgcn_readfirstlane(s_row0[lo]) + mt * TM;
    f.n0 = ntile * TNT;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int row = i < 2 ? wave * 32 + 16 * i + (lane >> 2) : tok;
      f.raw[i] = !GATHER ? f.row0 + row : row < f.rows_here ? p.a_row_map[f.row0 + row] : 0;
    }
    return f;
  };
  // Stage loads: wave w stages rows [32 w, 32 w + 32) of both slabs as 2
  // instructions of 16 rows each (128 weight rows: rows [16 w, 16 w + 16)
  // as one instruction; 64: rows [8 w, 8 w + 8) as one instruction of 32
  // lanes); lane l lands in slot
  // l & 3 of row 32 w + 16 i + (l >> 2) and fetches the chunk swz() keeps
  // there.
  auto tile_finish = [&](const TiledTileFetch& f) {
    TiledTile t;
    t.e = f.e;
    t.row0 = f.row0;
    t.rows_here = f.rows_here;
    t.n0 = f.n0;
    t.wb = p.w + static_cast<int64_t>(f.e) * N * (W4 ? K / 2 : K);
    // A row feeding output row row0 + row, or -1 (as a_source_row)
    auto source = [&](int row, int raw) {
      if (row >= f.rows_here) return -1;
      const int ar = GATHER ? raw / p.a_row_div : raw;
      return static_cast<unsigned>(ar) < static_cast<unsigned>(p.a_rows) ? ar : -1;
    };
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wave * 32 + 16 * i + (lane >> 2);
      const int chunk = ((lane & 3) ^ ((row >> 2) & 3)) << 4;
      const int ar = source(row, f.raw[i]);
      t.aoff[i] = static_cast<uint32_t>(ar < 0 ? 0 : ar) * K + chunk;
      const int wrow = TNT == 256 ? row : TNT == 128 ? wave * 16 + (lane >> 2) : wave * 8 + (lane >> 2) % 8;
      const int wchunk = TNT == 256 ? chunk : ((lane & 3) ^ ((wrow >> 2) & 3)) << 4;
      const int wr = f.n0 + wrow < N ? f.n0 + wrow : f.n0;
      t.woff[i] = static_cast<uint32_t>(wr) * K + wchunk;
    }
    if constexpr (W4) {
      // wave w: weight rows [32 w, 32 w + 32), two lanes per 32-byte row
      const int wrow = wave * 32 + (lane >> 1);
      const int wchunk = ((lane & 1) ^ ((wrow >> 3) & 1)) << 4;
      const int wr = f.n0 + wrow < N ? f.n0 + wrow : f.n0;
      t.woff[0] = static_cast<uint32_t>(wr) * (K / 2) + wchunk;
    }
    t.sa_row = source(tok, f.raw[2]);
    return t;
  };
  // The weight block scales of a tile's two 128-row blocks into s_wsf
  // (direct-to-LDS, one value per thread: 2 KB <= 512). A block past the
  // last weight row repeats the last block; no working wave reads it, since
  // N is a multiple of 128.
  auto ws_load = [&](const TiledTileFetch& f) {
    const int i = tid < 2 * KB ? tid : 0;
    const int kb = i % KB;
    const int nb = min(f.n0 / kGroup + i / KB, N / kGroup - 1);
    __builtin_amdgcn_global_load_lds(p.w_scales + (static_cast<int64_t>(f.e) * (N / kGroup) + nb) * KB + kb,
                                     (lds_void*)(s_wsf + wave * 64), 4, 0, 0);
  };
  auto issue_t = [&](const TiledTile& t, int j, uint8_t* stage) {  // operand slabs of stage j
    const int s = j < NS ? j : NS - 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(p.a + (t.aoff[i] + s * SK), (lds_void*)(stage + (wave * 32 + 16 * i) * SK), 16, 0, 0);
    if constexpr (W4) {
      __builtin_amdgcn_global_load_lds(t.wb + (t.woff[0] + s * (SK / 2)), (lds_void*)(stage + kStageA + wave * 32 * (SK / 2)), 16, 0, 0);
    } else if constexpr (TNT == 256) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(t.wb + (t.woff[i] + s * SK), (lds_void*)(stage + kStageA + (wave * 32 + 16 * i) * SK), 16, 0, 0);
    } else if constexpr (TNT == 128) {
      __builtin_amdgcn_global_load_lds(t.wb + (t.woff[0] + s * SK), (lds_void*)(stage + kStageA + wave * 16 * SK), 16, 0, 0);
    } else if (lane < 32) {
      __builtin_amdgcn_global_load_lds(t.wb + (t.woff[0] + s * SK), (lds_void*)(stage + kStageA + wave * 8 * SK), 16, 0, 0);
    }
  };
  // Token scales of block kb. Waves 0..3 load them into `buf`; waves
  // 4..7 load the same values into a sink so that every wave has the same
  // number of loads in flight and one vmcnt immediate fits all of them.
  // W4: waves 4..7 load the scale bytes of the tile's 256 weight rows
  // instead (4 bytes per row and block) into s_wsc, by block parity.
  auto issue_s_t = [&](const TiledTile& t, int kb, uint32_t* buf) {
    const int kbc = kb < KB ? kb : KB - 1;
    if constexpr (W4) {
      if (wave >= TM / 64) {
        const int row = t.n0 + (wave & 3) * 64 + lane;
        const int64_t widx = (static_cast<int64_t>(t.e) * N + (row < N ? row : t.n0)) * (K / kMxBlock) + kbc * 4;
        __builtin_amdgcn_global_load_lds(p.w_mx + widx, (lds_void*)(s_wsc + (kb & 1) * TM + (wave & 3) * 64), 4, 0, 0);
        return;
      }
    }
    uint32_t* dst = (wave < TM / 64 ? buf : s_srx) + (wave & 3) * 64;
    const int64_t idx = static_cast<int64_t>(kbc) * p.a_rows + (t.sa_row < 0 ? 0 : t.sa_row);
    if constexpr (UE8M0)
      __builtin_amdgcn_global_load_lds(static_cast<const uint8_t*>(p.a_scales) + idx, (lds_void*)dst, 1, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(static_cast<const uint32_t*>(p.a_scales) + idx, (lds_void*)dst, 4, 0, 0);
  };
  // A tile's prologue: stages 0..2 and the token scales of blocks 0 and 1;
  // each stage issues [A x2][W x2] then, when it starts a block, [S]. The
  // order is pinned so the vmcnt waits can count. prologue_part(t, b) is
  // what goes after stage buffer b is free.
  auto prologue_part = [&](const TiledTile& t, int b) {
    issue_t(t, b, b == 0 ? s_st0 : b == 1 ? s_st1 : s_st2);
    __builtin_amdgcn_sched_barrier(0);
    if (b == 0) issue_s_t(t, 0, s_sr0);
    if (b == 2) issue_s_t(t, 1, s_sr1);
    __builtin_amdgcn_sched_barrier(0);
  };

  TiledTile cur{};
  if (vid < total) {
    const TiledTileFetch f = tile_fetch(vid);
    if constexpr (!W4) ws_load(f);
    cur = tile_finish(f);
    prologue_part(cur, 0);
    prologue_part(cur, 1);
    prologue_part(cur, 2);
  }

  for (int tile = vid; tile < total; tile += G) {
    const int row0 = cur.row0, rows_here = cur.rows_here, n0 = cur.n0, sa_row = cur.sa_row;
    const bool wave_on = wm * 64 < rows_here && n0 + wn * WN < N;
    auto issue = [&](int j, uint8_t* stage) { issue_t(cur, j, stage); };
    auto issue_s = [&](int kb, uint32_t* buf) { issue_s_t(cur, kb, buf); };
    auto decode_sa = [&](uint32_t raw) -> float {
      const float v = sa_row < 0 ? 1.0f : __uint_as_float(UE8M0 ? raw << 23 : raw);
      return v > kScaleFloor ? v : kScaleFloor;
    };

    v16f acc[WT][2];  // [weight tile][token tile]
#pragma unroll
    for (int i = 0; i < WT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
    float tok_prev = 1.0f;  // this thread's token scale of the previous block
    float sw_norm = 1.0f;   // weight part of the accumulator's normalizer

    // The prologue's loads went out before the loop (first tile) or during
    // the previous tile's output stores; the barrier keeps this tile's
    // writes of s_rt and s_sl behind the previous tile's last reads.
    lds_barrier();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS + 1));  // stage 0 and block 0's scales landed
    if (tid < TM) {
      tok_prev = decode_sa(s_sr0[tok]);
      s_rt[0][(tok & 31) * 8 + (tok >> 5)] = 1.0f;
      if (KB == 1) s_sl[(tok & 31) * 8 + (tok >> 5)] = tok_prev;
    }

    // Stage j. Entry: stage j is visible to all waves (barrier of stage j-1
    // or the prologue's); stages j+1 and j+2 may be in flight. Each stage
    // issues [A x2][W x2, or x1 for the narrow tile] (LPS loads) for stage
    // j+3, then [S] if stage j+3 starts a block. Stage j+1 (and, when it
    // starts a block, its scales) has landed once only stage j+2's loads
    // remain: LPS when j+1 starts a block, else LPS plus the scales issued
    // after stage j+2. If stage j+1 starts block kb,
    // its token ratios are published; then the barrier, the loads, and the 8
    // MFMAs of stage j.
    auto stage = [&](int j, const uint8_t* cur, uint8_t* fill, const uint32_t* sr_next,
                     float* rt_next, const float* rt_cur, uint32_t* sr_fill, bool next_starts,
                     bool cur_starts, bool fill_starts) {
      if (next_starts)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS + 1));
      if (next_starts) {
        const int kb_next = (j + 1) >> 1;
        const float t = decode_sa(sr_next[tok]);
        const float r = tok_prev * __builtin_amdgcn_rcpf(t);
        if (tid < TM && kb_next < KB) {
          rt_next[(tok & 31) * 8 + (tok >> 5)] = r;
          if (kb_next == KB - 1) s_sl[(tok & 31) * 8 + (tok >> 5)] = t;
        }
        tok_prev = t;
      }
      lds_barrier();
      issue(j + 3, fill);
      __builtin_amdgcn_sched_barrier(0);
      if (fill_starts) issue_s((j + 3) >> 1, sr_fill);
      __builtin_amdgcn_sched_barrier(0);
      if (!wave_on || j >= NS) return;
      if (cur_starts) {
        const int kb = j >> 1;
        const float sw = fmaxf(s_wsf[((wn * WN) / kGroup) * KB + kb], kScaleFloor);
        const float q = sw_norm * __builtin_amdgcn_rcpf(sw);
        sw_norm = sw;
        const float2 r2 = *reinterpret_cast<const float2*>(rt_cur + (lane & 31) * 8 + wm * 2);
        const float ratio0 = r2.x * q, ratio1 = r2.y * q;
#pragma unroll
        for (int wt = 0; wt < WT; ++wt) {
          acc[wt][0] = acc[wt][0] * ratio0;
          acc[wt][1] = acc[wt][1] * ratio1;
        }
      }
      const uint8_t* sA = cur;
      const uint8_t* sW = cur + kStageA;
      const int c0 = 2 * (lane >> 5);
      Frag af[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int r = wm * 64 + tt * 32 + (lane & 31);
        af[tt].u[0] = *reinterpret_cast<const uint4*>(sA + swz(r, c0));
        af[tt].u[1] = *reinterpret_cast<const uint4*>(sA + swz(r, c0 + 1));
      }
#pragma unroll
      for (int wt = 0; wt < WT; ++wt) {
        const int r = wn * WN + wt * 32 + (lane & 31);
        Frag wf;
        wf.u[0] = *reinterpret_cast<const uint4*>(sW + swz(r, c0));
        wf.u[1] = *reinterpret_cast<const uint4*>(sW + swz(r, c0 + 1));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          acc[wt][tt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf.v, af[tt].v, acc[wt][tt],
                                                                         0, 0, 0, 0, 0, 0);
      }
    };

    lds_barrier();
    // Four stages per iteration (unconditional: past the end a stage only
    // loads clamped, unused data and skips its compute, so every path issues
    // the same vector-memory sequence). Stage j uses buffer j % 4; block
    // kb's token scales use buffer kb % 2.
    if constexpr (TNT == 256) {
      // Ping-pong. The two waves that share a SIMD (w and w + 4) take turns:
      // while one issues the MFMAs of its stage (raised issue priority), the
      // other reads its next stage's fragments from LDS and issues the
      // direct-to-LDS loads, so the matrix core is not left idle while a wave
      // waits on LDS or on the address unit. Every phase ends at a workgroup
      // barrier; group 1 (waves 4..7) runs one phase behind group 0, which
      // costs each group one extra barrier (before the loop for group 1,
      // after it for group 0).
      //
      // L(j): stage j's fragments into registers; at a block start the
      // block's scale ratios; the loads of stage j+3 (+ its token scales when
      // it starts a block); then this wave's loads of stage j+1 (and the
      // scales issued with it) have landed once 9 loads remain (stages j+2
      // and j+3, one of which starts a block); at j odd, group 0 publishes
      // the token ratios of block (j+1)/2.
      // M(j): the 8 MFMAs of stage j, at a block start each accumulator
      // rescaled just before its MFMA (16 multiplies between MFMAs).
      //
      // Buffers: stage j's slot j % 4 is refilled with stage j+4 by L(j+1);
      // its last reader, group 1's L(j), ended one phase earlier. Block kb's
      // ratios (slot kb % 2) are written in L(2kb-1) by group 0 and read in
      // L(2kb) by both groups; the next writer of the slot is L(2kb+3).
      const bool grp1 = wave >= 4;
      Frag af[2], wf[W4 ? 1 : WT];
      uint4 wf4[W4 ? WT : 1];           // W4: a lane's 32 E2M1 codes of each weight tile
      uint32_t wsc[W4 ? WT : 1] = {};   // W4: its row's 4 scale bytes of the current block
      uint32_t scb[W4 ? WT : 1] = {};   // W4: the stage's scale byte (low byte) per weight tile
      float ratio0 = 1.0f, ratio1 = 1.0f;
      uint32_t tsb0 = 127, tsb1 = 127;  // kHwScales: the lane's two tokens' E8M0 bytes of the block
      auto lphase = [&](int j, const uint8_t* cur, uint8_t* fill, const float* rt_cur,
                        uint32_t* sr_fill, const uint32_t* sr_next, float* rt_next, auto even_t) {
        constexpr bool even = decltype(even_t)::value;
        if (W4 && wave_on && j < NS) {
          const int h = lane >> 5;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int r = wm * 64 + tt * 32 + (lane & 31);
            af[tt].u[0] = *reinterpret_cast<const uint4*>(cur + swz(r, h));
            af[tt].u[1] = *reinterpret_cast<const uint4*>(cur + swz(r, 2 + h));
          }
#pragma unroll
          for (int wt = 0; wt < (W4 ? WT : 1); ++wt) {
            const int r = wn * WN + wt * 32 + (lane & 31);
            wf4[wt] = *reinterpret_cast<const uint4*>(cur + kStageA + r * (SK / 2) + ((h ^ ((r >> 3) & 1)) << 4));
          }
          if constexpr (even) {
            const int kb = j >> 1;
#pragma unroll
            for (int wt = 0; wt < (W4 ? WT : 1); ++wt)
              wsc[wt] = s_wsc[W4 ? (kb & 1) * TM + wn * WN + wt * 32 + (lane & 31) : 0];
            if constexpr (kHwScales) {
              // the block's raw token bytes (its buffer is refilled one phase later)
              tsb0 = sr_next[wm * 64 + (lane & 31)];
              tsb1 = sr_next[wm * 64 + 32 + (lane & 31)];
            } else {
              const float2 r2 = *reinterpret_cast<const float2*>(rt_cur + (lane & 31) * 8 + wm * 2);
              ratio0 = r2.x;
              ratio1 = r2.y;
            }
          }
          // MX blocks 2 (j & 1) + h of the 128-wide block: this stage's half of it
#pragma unroll
          for (int wt = 0; wt < (W4 ? WT : 1); ++wt) scb[wt] = wsc[wt] >> (8 * (2 * (j & 1) + h));
        } else if (!W4 && wave_on && j < NS) {
          const int c0 = 2 * (lane >> 5);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int r = wm * 64 + tt * 32 + (lane & 31);
            af[tt].u[0] = *reinterpret_cast<const uint4*>(cur + swz(r, c0));
            af[tt].u[1] = *reinterpret_cast<const uint4*>(cur + swz(r, c0 + 1));
          }
#pragma unroll
          for (int wt = 0; wt < (W4 ? 1 : WT); ++wt) {
            const int r = wn * WN + wt * 32 + (lane & 31);
            wf[wt].u[0] = *reinterpret_cast<const uint4*>(cur + kStageA + swz(r, c0));
            wf[wt].u[1] = *reinterpret_cast<const uint4*>(cur + kStageA + swz(r, c0 + 1));
          }
          if constexpr (even) {
            const int kb = j >> 1;
            const float sw = fmaxf(s_wsf[((wn * WN) / kGroup) * KB + kb], kScaleFloor);
            const float q = sw_norm * __builtin_amdgcn_rcpf(sw);
            sw_norm = sw;
            const float2 r2 = *reinterpret_cast<const float2*>(rt_cur + (lane & 31) * 8 + wm * 2);
            ratio0 = r2.x * q;
            ratio1 = r2.y * q;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(j + 3, fill);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!even) issue_s((j + 3) >> 1, sr_fill);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPS + 1));
        if constexpr (!even) {
          if (!grp1) {
            const int kb_next = (j + 1) >> 1;
            const float t = decode_sa(sr_next[tok]);
            const float r = tok_prev * __builtin_amdgcn_rcpf(t);
            if (kb_next < KB) {
              rt_next[(tok & 31) * 8 + (tok >> 5)] = r;
              if (kb_next == KB - 1) s_sl[(tok & 31) * 8 + (tok >> 5)] = t;
            }
            tok_prev = t;
          }
        }
      };
      auto mphase = [&](int j, auto even_t) {
        constexpr bool even = decltype(even_t)::value;
        if (!wave_on || j >= NS) return;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int wt = 0; wt < WT; ++wt)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            if constexpr (even && !kHwScales) acc[wt][tt] = acc[wt][tt] * (tt == 0 ? ratio0 : ratio1);
            if constexpr (W4) {
              const uint4 w = wf4[wt];
              const v8i wa = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                              static_cast<int>(w.w), 0, 0, 0, 0};
              const int tsb = kHwScales ? static_cast<int>(tt == 0 ? tsb0 : tsb1) : 127;
              acc[wt][tt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, af[tt].v, acc[wt][tt], 4, 0, 0,
                                                                             static_cast<int>(scb[wt]), 0, tsb);
            } else {
              acc[wt][tt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[wt].v, af[tt].v, acc[wt][tt],
                                                                             0, 0, 0, 0, 0, 0);
            }
          }
        if constexpr (even && !kHwScales) {
#pragma unroll
          for (int i = 0; i < 2 * WT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // VALU: one accumulator's rescale
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // its MFMA
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      };
      const std::true_type ev;
      const std::false_type od;
      if (grp1) lds_barrier();
      for (int j = 0; j < NS; j += 4) {
        lphase(j, s_st0, s_st3, s_rt[0], s_sr1, s_sr0, s_rt[0], ev);
        lds_barrier();
        mphase(j, ev);
        lds_barrier();
        lphase(j + 1, s_st1, s_st0, s_rt[0], s_sr0, s_sr1, s_rt[1], od);
        lds_barrier();
        mphase(j + 1, od);
        lds_barrier();
        lphase(j + 2, s_st2, s_st1, s_rt[1], s_sr0, s_sr1, s_rt[1], ev);
        lds_barrier();
        mphase(j + 2, ev);
        lds_barrier();
        lphase(j + 3, s_st3, s_st2, s_rt[1], s_sr1, s_sr0, s_rt[0], od);
        lds_barrier();
        mphase(j + 3, od);
        lds_barrier();
      }
      if (!grp1) lds_barrier();
    } else {
    for (int j = 0; j < NS; j += 4) {
      stage(j, s_st0, s_st3, s_sr0, s_rt[0], s_rt[0], s_sr1, false, true, false);
      stage(j + 1, s_st1, s_st0, s_sr1, s_rt[1], s_rt[0], s_sr0, true, false, true);
      stage(j + 2, s_st2, s_st1, s_sr1, s_rt[1], s_rt[1], s_sr0, false, true, false);
      stage(j + 3, s_st3, s_st2, s_sr0, s_rt[0], s_rt[1], s_sr1, true, false, true);
    }
    }
    __builtin_amdgcn_s_waitcnt(0);  // trailing loads of this tile done before any stage is reused
    __syncthreads();

    // The next tile: its coordinates and row-map entries now (loads into
    // registers, in flight during the output staging); its weight scales
    // and prologue follow once the staging's LDS writes are done, the
    // prologue as the stage buffers free up. (A direct-to-LDS load in
    // flight would make the compiler wait for it before the staging writes,
    // whose buffer it cannot tell apart.)
    const bool has_next = tile + G < total;
    TiledTileFetch nf{};
    if (has_next) nf = tile_fetch(tile + G);
    TiledTile nxt = cur;

    if constexpr (!SOUT) {
      if (has_next) {
        if constexpr (!W4) ws_load(nf);
        nxt = tile_finish(nf);
        prologue_part(nxt, 0);
        prologue_part(nxt, 1);
        prologue_part(nxt, 2);
      }
      // Each lane stores its 4-column pieces straight from the accumulator.
      if (wave_on) {
        const float f = sw_norm;
        const float2 sl = *reinterpret_cast<const float2*>(s_sl + (lane & 31) * 8 + wm * 2);
        const float fs[2] = {kHwScales ? 1.0f : sl.x * f, kHwScales ? 1.0f : sl.y * f};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int j = wm * 64 + tt * 32 + (lane & 31);
          if (j < rows_here) {
            uint16_t* crow = p.c + static_cast<int64_t>(row0 + j) * N + n0 + wn * WN + 4 * (lane >> 5);
#pragma unroll
            for (int wt = 0; wt < WT; ++wt)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                v4f v = {acc[wt][tt][4 * g], acc[wt][tt][4 * g + 1], acc[wt][tt][4 * g + 2], acc[wt][tt][4 * g + 3]};
                *reinterpret_cast<uint2*>(crow + wt * 32 + g * 8) = pack_bf16x4(v * fs[tt]);
              }
          }
        }
      }
    } else {
      // Output tile through the free stage buffers: each wave writes its
      // scaled BF16 results there (row j in buffer j / kRowsPerBuf, 16-byte
      // chunk q of the row at slot q ^ (j % 4), so the 32 rows of one write
      // spread over 4 bank groups), then every wave stores whole 16-byte row
      // chunks, 8 lanes to a 128-byte line. A wider swizzle would spread the
      // writes further but needs a write address per chunk and lane, and
      // those registers cost the main loop more than the bank conflicts.
      constexpr int kRowBytes = TNT * 2;
      constexpr int kChunks = kRowBytes / 16;
      constexpr int kRowsPerBuf = kStageBytes / kRowBytes;
      auto out_row = [&](int j) -> uint8_t* {
        const int b = j / kRowsPerBuf;
        uint8_t* base = b == 0 ? s_st0 : b == 1 ? s_st1 : b == 2 ? s_st2 : s_st3;
        return base + (j % kRowsPerBuf) * kRowBytes;
      };
      if (wave_on) {
        const float f = sw_norm;
        const float2 sl = *reinterpret_cast<const float2*>(s_sl + (lane & 31) * 8 + wm * 2);
        const float fs[2] = {kHwScales ? 1.0f : sl.x * f, kHwScales ? 1.0f : sl.y * f};
        // j % 4 equals lane % 4; formed here behind an opaque move so the
        // compiler does not hoist the slot offsets out of the tile loop (they
        // would stay live across it).
        int sw = lane & 3;
        asm volatile("" : "+v"(sw));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int j = wm * 64 + tt * 32 + (lane & 31);
          uint8_t* row = out_row(j);
#pragma unroll
          for (int wt = 0; wt < WT; ++wt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              v4f v = {acc[wt][tt][4 * g], acc[wt][tt][4 * g + 1], acc[wt][tt][4 * g + 2], acc[wt][tt][4 * g + 3]};
              // chunk of these 8 columns: q % 4 == g, so q ^ sw keeps q's
              // upper bits (an immediate offset) and swizzles g
              const int q = (wn * WN + wt * 32 + g * 8) / 8;
              *reinterpret_cast<uint2*>(row + (((q & ~3) | (g ^ sw)) << 4) + 8 * (lane >> 5)) = pack_bf16x4(v * fs[tt]);
            }
        }
      }
      __syncthreads();
      // The next tile's row-map entries have landed (no store is in flight
      // yet, so this waits for nothing else).
      __builtin_amdgcn_s_waitcnt(0);
      if (has_next) {
        if constexpr (!W4) ws_load(nf);
        nxt = tile_finish(nf);
      }
      {
        // Pass it = b * kPasses + q stores rows it * RPI + tr; thread (tr, tq)
        // takes chunk tq. RPI is a multiple of 4, so the row's swizzle is
        // tr % 4 in every pass. Once every wave has read stage buffer b (rows
        // [b * kRowsPerBuf, (b + 1) * kRowsPerBuf)), the next tile's prologue
        // part for that buffer goes out; the stores in flight only lengthen
        // its first wait.
        constexpr int RPI = kTiledThreads / kChunks;
        constexpr int kPasses = kRowsPerBuf / RPI;  // passes per stage buffer
        static_assert(RPI % 4 == 0, "passes start at rows divisible by 4");
        static_assert(kPasses * RPI == kRowsPerBuf && TM == 4 * kRowsPerBuf, "whole passes over four buffers");
        const int tq = tid % kChunks, tr = tid / kChunks;
        int lb = tr * kRowBytes + ((tq ^ (tr & 3)) << 4);
        asm volatile("" : "+v"(lb));
        uint16_t* gc = p.c + static_cast<int64_t>(row0 + tr) * N + n0 + tq * 8;
        int step = RPI * N;  // opaque, so per-pass offsets are not hoisted
        asm volatile("" : "+s"(step));
        const bool col_ok = n0 + tq * 8 < N;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          uint4 v[kPasses];  // a buffer's passes read together, then stored
#pragma unroll
          for (int q = 0; q < kPasses; ++q)
            v[q] = *reinterpret_cast<const uint4*>(out_row((b * kPasses + q) * RPI) + lb);
#pragma unroll
          for (int q = 0; q < kPasses; ++q, gc += step) {
            const int j0 = (b * kPasses + q) * RPI;  // first row of the pass
            if (col_ok && j0 + tr < rows_here) *reinterpret_cast<uint4*>(gc) = v[q];
          }
          if (b < 3 && has_next) {
            lds_barrier();  // every wave's reads of buffer b have returned
            prologue_part(nxt, b);
          }
        }
      }
    }
    if (tid == 0 && p.tiles_visited)  // (row tile, 128-column tile) pairs, each counted once
      atomicAdd(p.tiles_visited, TNT >= kColTile ? min(TNT, N - n0) / kColTile : (n0 % kColTile == 0 ? 1 : 0));
    cur = nxt;
  }
}

}  // namespace

bool launch_tiled_w4(const GemmArgs& g, hipStream_t stream, hipError_t* err) {
  const int live_bound = g.max_live_experts < g.num_experts ? g.max_live_experts : g.num_experts;
  if (live_bound <= 0 || g.max_rows_per_expert <= kStreamMaxRows || !g.w_mx || g.k % kGroup != 0) return false;
  // The tile bound of launch_grouped_gemm; the 256-wide kernel only where it
  // keeps the CUs busy (the narrow cases stay with the MXFP4 kernels).
  const int64_t rows = g.row_cap;
  const int64_t large = rows / (kStreamMaxRows + 1) < live_bound ? rows / (kStreamMaxRows + 1) : live_bound;
  const int64_t row_tiles = (rows + TM - 1) / TM + large;
  const int64_t cap = device_cu_count();
  const int64_t tiles = row_tiles * ((g.n + TN - 1) / TN);
  if (tiles < 2 * cap) return false;
  const int grid = static_cast<int>(tiles < cap ? tiles : cap);
  const bool u = g.fmt == kUe8m0, m = g.a_row_map != nullptr;
  const dim3 gr(grid), bl(kTiledThreads);
  if (u && m) hipLaunchKernelGGL((gemm_tiled_kernel<true, true, TN, false, true, true>), gr, bl, 0, stream, g);
  else if (u) hipLaunchKernelGGL((gemm_tiled_kernel<true, false, TN, false, true, true>), gr, bl, 0, stream, g);
  else if (m) hipLaunchKernelGGL((gemm_tiled_kernel<false, true, TN, false, true, true>), gr, bl, 0, stream, g);
  else hipLaunchKernelGGL((gemm_tiled_kernel<false, false, TN, false, true, true>), gr, bl, 0, stream, g);
  *err = hipGetLastError();
  return true;
}

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t stream) {
  const int live_bound = g.max_live_experts < g.num_experts ? g.max_live_experts : g.num_experts;
  if (live_bound <= 0) return hipSuccess;
  if (g.act_out && (g.max_rows_per_expert > kStreamMaxRows || g.n % 64 != 0)) return hipErrorInvalidValue;
  hipError_t err = launch_stream(g, stream);
  if (err != hipSuccess) return err;
  if (g.max_rows_per_expert > kStreamMaxRows) {
    // Tiles of the large experts: at most ceil(rows / TM) + one partial row
    // tile per expert that can be large, times the column tiles.
    const int64_t rows = g.row_cap;
    const int64_t large = rows / (kStreamMaxRows + 1) < live_bound ? rows / (kStreamMaxRows + 1) : live_bound;
    const int64_t row_tiles = (rows + TM - 1) / TM + large;
    const int64_t cap = device_cu_count();
    // 256-wide weight tiles, or, when those would leave CUs idle (few large
    // experts on a narrow N, e.g. FC1 of a 256-intermediate layer), the 64-
    // and 128-wide kernels together, of which the one that suits the actual
    // row tiles runs (the pick needs the endpoints, which only the device
    // has). The grid covers the most tiles a launch could have, up to one
    // workgroup per CU.
    const bool narrow = row_tiles * ((g.n + TN - 1) / TN) < 2 * cap;
    const int64_t tiles = row_tiles * (narrow ? g.n / 64 : (g.n + TN - 1) / TN);
    const int grid = static_cast<int>(tiles < cap ? tiles : cap);
    if (grid > 0) {
      const bool u = g.fmt == kUe8m0, m = g.a_row_map != nullptr;
      const dim3 gr(grid), bl(kTiledThreads);
      auto launch = [&](auto tnt, auto pick, auto sout) {
        constexpr int W = decltype(tnt)::value;
        constexpr bool P = decltype(pick)::value, S = decltype(sout)::value;
        if (u && m) hipLaunchKernelGGL((gemm_tiled_kernel<true, true, W, P, S>), gr, bl, 0, stream, g);
        else if (u) hipLaunchKernelGGL((gemm_tiled_kernel<true, false, W, P, S>), gr, bl, 0, stream, g);
        else if (m) hipLaunchKernelGGL((gemm_tiled_kernel<false, true, W, P, S>), gr, bl, 0, stream, g);
        else hipLaunchKernelGGL((gemm_tiled_kernel<false, false, W, P, S>), gr, bl, 0, stream, g);
      };
      if (narrow) {
        launch(std::integral_constant<int, 64>{}, std::true_type{}, std::false_type{});
        if (hipGetLastError() == hipSuccess)
          launch(std::integral_constant<int, 128>{}, std::true_type{}, std::false_type{});
      } else {
        launch(std::integral_constant<int, TN>{}, std::false_type{}, std::true_type{});
      }
      err = hipGetLastError();
    }
  }
  return err;
}

}  // namespace moe
