// The decode-sized layer in one launch, and its FC1 half on its own.
//
// vLLM PR #59128 (Purpose) and TensorRT-LLM PR #21250 (sequence diagram):
// alignment yields per-expert contiguous rows and prefix-sum endpoints, and
// the FC1 grouped GEMM visits only the rows that exist. vLLM PR #65794
// (Details): activations are quantized per 1x128 group. TensorRT-LLM PR
// #21250 (For MoE owners; Performance): at decode sizes the fixed cost of
// each launch is a large part of the layer.
//
// With at most 64 routed pairs, every workgroup (8 waves, one per CU) derives
// the routing itself:
//  1. Prologue. The ids, the live count and all tokens' BF16 rows are loaded
//     together. Wave 0 finds the distinct experts of the live pairs with
//     ballots (stable ranks in pair order, as moe_align), orders them by
//     expert id and lays out their aligned rows. All tokens are quantized into
//     LDS with the 1x128 rule. Workgroup 0 also writes the alignment and the
//     quantized activations to the workspace, bit-identical to moe_align and
//     moe_act_quant.
//  2. Stream. A task is (live expert, 8 gate rows with the 8 up rows of the
//     same columns, 16-token tile) over the full K. Each wave streams its
//     tasks' 2 KB weight stages and their two weight block scales through a
//     private LDS ring by direct-to-LDS loads (whole 128-byte lines); a wave
//     only waits for its own loads, so the loop has no workgroup barrier.
//     With MXFP4 weights (one-launch layer, W4) a stage is the same 16 rows x
//     128 packed bytes, i.e. two K blocks, with the rows' E8M0 scale bytes
//     as its third load (fc2_decode.h).
//     Token fragments come from the resident LDS copy. The ring is 6 stages
//     deep, or 4 in the one-launch layer's variant for up to 60 KB of token
//     codes (the LDS the two stages free holds them).
//  3. Epilogue of a task. One cross-lane swap pairs gate and up values; C1
//     gets both BF16 halves, and act the fp32 SiLU(gate) * up of the
//     BF16-rounded pair (fp64 inside, rounded once).
// The one-launch layer (FUSED) goes on:
//  4. A barrier across the grid (every workgroup resident, one per CU): the
//     act rows, written through to memory, are complete once it opens.
//  5. FC2 and the top-k combine for the workgroup's 16 output columns, as
//     fc2_decode.h describes, in the same LDS (token codes -> FC2 input
//     codes, K-split partials -> pair slots, each wave's ring -> its FC2
//     stream). The first FC2 stages go out before the barrier.
#include <type_traits>

#include "device_common.h"
#include "fc2_decode.h"
#include "gemm_device.h"
#include "kernels.h"
#include "quant_device.h"

#include <atomic>

namespace moe {
namespace {

// The one-launch layer reuses each wave's ring for FC2, so both streams
// share the ring geometry of fc2_decode.h.
constexpr int kF1Threads = kDecThreads;
constexpr int kF1Waves = kDecWaves;
constexpr int kF1StageW = kDecStageW;        // 8 gate + 8 up rows x 128 bytes
constexpr int kF1Stage = kDecStage;          // + the two weight scales (64 x 4-byte slots)
constexpr int kF1Loads = kDecLoads;          // loads per wave and stage

// Grid barrier of the one-launch layer: per workgroup the epoch (launch
// count) it has reached, the epoch workgroup 0 has released (with
// kDlFailBit set when one of its waits gave up), and a sticky count of waits
// that gave up (a workgroup that was not resident).
__device__ unsigned g_dl_flag[kDlMaxGrid];
__device__ unsigned g_dl_release;
__device__ unsigned g_dl_timeouts;
constexpr unsigned kDlFailBit = 0x80000000u;
constexpr unsigned kDlEpochMask = ~kDlFailBit;

__device__ __forceinline__ unsigned flag_load(const unsigned* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(unsigned* a, unsigned v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// Waits until (*a & mask) == v; after `limit` polls (or at once when limit
// is negative) it gives up, counts itself and returns false.
__device__ __forceinline__ bool flag_wait(const unsigned* a, unsigned v, int limit, unsigned mask = ~0u) {
  if (limit < 0) {
    atomicAdd(&g_dl_timeouts, 1u);
    return false;
  }
  for (int it = 0; (flag_load(a) & mask) != v; ++it) {
    if (it == limit) {
      atomicAdd(&g_dl_timeouts, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return true;
}

// DEPTH: stages in a wave's ring, kDecDepth; or 4 in the wide variant of the
// one-launch layer, whose LDS then holds kF1TokBytesWide of token codes.
// W4: MXFP4 weights (one-launch layer only).
template <int FMT, bool FUSED, int DEPTH, bool W4>
__global__ __launch_bounds__(kF1Threads, 1) void fc1_decode_kernel(DecodeLayerArgs a) {
  constexpr bool kWide = DEPTH != kDecDepth;
  static_assert(!kWide || (DEPTH == 4 && FUSED), "the wide variant: one-launch layer, 4 stages");
  static_assert(!W4 || FUSED, "MXFP4 weights: one-launch layer only");
  constexpr int kTokBytes = kWide ? kF1TokBytesWide : kF1TokBytes;
  constexpr int kMaxScales = kWide ? kF1MaxScalesWide : kF1MaxScales;
  constexpr int kXLoads = kTokBytes / 8 / kF1Threads;  // 16-byte (8-value) activation loads per thread
  const DecodeFc1Args& p = a.f1;
  const DownCombineArgs& q = a.f2;
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kF1Waves * DEPTH * kF1Stage];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kTokBytes];  // codes, row stride H + 16
  __shared__ __attribute__((aligned(16))) float s_xs[kMaxScales];  // token scale of (token, K block) at t * KB + kb
  __shared__ int s_e[kDcMaxPairs];        // live entry (in expert order) -> expert
  __shared__ int s_cnt[kDcMaxPairs];      //   its live rows
  __shared__ int s_c0[kDcMaxPairs];       //   its first compact row
  __shared__ int s_row0[kDcMaxPairs];     //   its first aligned row
  __shared__ int s_tp[kDcMaxPairs + 1];   //   prefix of its 16-token tiles
  __shared__ int s_ctok[kDcMaxPairs];     // compact row -> token
  __shared__ int s_crow[kDcMaxPairs];     //   its aligned row
  __shared__ int s_cpair[kDcMaxPairs];    //   its pair
  __shared__ int s_prow[kDcMaxPairs];     // pair -> aligned row, or -1
  __shared__ int s_nlive, s_total;
  // K-split partial sums: [task parity][wave][lane] x 16 bytes, and per group
  // of waves the number of shares that have arrived (counts up for good).
  __shared__ __attribute__((aligned(16))) uint8_t s_part[2 * kF1Waves * 64 * 16];
  __shared__ int s_arrive[kF1Waves];
  __shared__ float s_tw[kDcMaxPairs];     // pair -> routing weight (one-launch layer)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int TK = p.topk, E = p.num_experts, H = p.hidden, I = p.inter, N = 2 * I;
  const int KB = H / kGroup, XS = H + 16, A = p.align_rows;
  const int PQ = p.t_cap * TK;  // <= kDcMaxPairs
  const int gpr = H / kGroup;   // activation groups per token

  // ---- 1. everything the prologue reads, issued together
  const int my_id = tid < PQ ? p.ids[tid] - p.expert_start : -1;  // local expert id
  const float my_tw = FUSED && tid < PQ ? q.topk_w[tid] : 0.0f;
  // This launch's epoch at the grid barrier.
  const unsigned epoch = FUSED ? flag_load(&g_dl_flag[blockIdx.x]) + 1u : 0u;
  const int t_live = p.t_live_dev ? min(max(scalar_load(p.t_live_dev), 0), p.t_cap) : p.t_cap;
  const int n_chunks = p.t_cap * H / 8;  // 16-byte chunks of x
  uint4 xr[kXLoads];
#pragma unroll
  for (int k = 0; k < kXLoads; ++k) {
    const int ci = min(tid + k * kF1Threads, n_chunks - 1);
    xr[k] = *reinterpret_cast<const uint4*>(p.x + static_cast<int64_t>(ci) * 8);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // ---- routing (wave 0; lane = pair). Expert ids are compared bit by bit,
  // most significant first, with one ballot per bit: every lane learns the
  // valid lanes with the same expert (eq) and with a smaller one (lt), so
  // ranks in pair order, counts, the entry index in expert order and the
  // compact offset are popcounts; the aligned-row and tile prefixes over the
  // entries are one wave scan.
  if (tid < kF1Waves) s_arrive[tid] = 0;
  if (FUSED && tid < PQ) s_tw[tid] = my_tw;
  if (wave == 0) {
    const int n_pairs = t_live * TK;
    const bool live = lane < n_pairs && lane < PQ;
    const bool ok = live && static_cast<unsigned>(my_id) < static_cast<unsigned>(E);
    const uint64_t below = (uint64_t(1) << lane) - 1;
    const uint64_t valid = __ballot(ok);
    const int nb = 32 - __builtin_clz(static_cast<unsigned>(max(E - 1, 1)));  // bits of an expert id
    uint64_t eq = valid, lt = 0;
    for (int b = nb - 1; b >= 0; --b) {
      const bool bit = (my_id >> b) & 1;
      const uint64_t m = __ballot(ok && bit);
      if (bit) {
        lt |= eq & ~m;
        eq &= m;
      } else {
        eq &= ~m;
      }
    }
    const int rank = __popcll(eq & below), cnt = __popcll(eq);
    const uint64_t leaders = __ballot(ok && rank == 0);
    const int n_live = __popcll(leaders);
    const int pos = __popcll(lt & leaders);  // entry of this lane's expert
    const int c0 = __popcll(lt);             // live pairs of smaller experts
    if (ok && rank == 0) {
      s_e[pos] = my_id;
      s_cnt[pos] = cnt;
      s_c0[pos] = c0;
      s_row0[pos] = (cnt + A - 1) / A * A;                          // prefixed below
      s_tp[pos] = (cnt + kStreamTileM - 1) / kStreamTileM;          // prefixed below
    }
    // Exclusive prefixes over the entries (lane = entry; one wave, so its LDS
    // accesses are ordered).
    const int vr = lane < n_live ? s_row0[lane] : 0;
    const int vt = lane < n_live ? s_tp[lane] : 0;
    int ir = vr, it = vt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int ur = __shfl_up(ir, d, 64), ut = __shfl_up(it, d, 64);
      if (lane >= d) {
        ir += ur;
        it += ut;
      }
    }
    if (lane < n_live) {
      s_row0[lane] = ir - vr;
      s_tp[lane] = it - vt;
    }
    if (lane == 63) {
      s_nlive = n_live;
      s_total = ir;
      s_tp[n_live] = it;
    }
    if (ok) {
      const int row = s_row0[pos] + rank;
      const int c = c0 + rank;
      s_ctok[c] = lane / TK;
      s_crow[c] = row;
      s_cpair[c] = lane;
      s_prow[lane] = row;
    } else if (live) {
      s_prow[lane] = -1;
    }
  }
  __syncthreads();
  const int n_live = __builtin_amdgcn_readfirstlane(s_nlive);
  const int total_rows = __builtin_amdgcn_readfirstlane(s_total);
  // Lane j's copies of entry j's tile prefix and expert (j <= n_live; the
  // prefix past the last entry is tp_end), so that decoding a task is one
  // ballot and a few lane reads instead of a search through LDS.
  const int tp_lane = s_tp[min(lane, n_live)];
  const int tp_end = __builtin_amdgcn_readfirstlane(s_tp[n_live]);
  const int e_lane = lane < n_live ? s_e[lane] : 0;
  // The first entry whose expert is >= e (n_live if none).
  auto entry_ge = [&](int e) {
    int lo = 0, hi = n_live;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_e[mid] < e) lo = mid + 1; else hi = mid;
    }
    return lo;
  };

  // ---- the alignment to the workspace (workgroup 0), as moe_align writes
  // it; nothing in this launch reads it, so it is written once workgroup 0
  // is off the critical path (after its FC1 stream, or after releasing the
  // grid barrier)
  auto write_alignment = [&]() {
    for (int e = tid; e <= E; e += kF1Threads) {
      const int i = entry_ge(e);
      if (e < E) p.counts[e] = i < n_live && s_e[i] == e ? s_cnt[i] : 0;
      p.offsets[e] = i < n_live ? s_row0[i] : total_rows;
    }
    for (int r = tid; r < total_rows; r += kF1Threads) {
      int lo = 0, hi = n_live - 1;  // the entry whose aligned rows hold r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_row0[mid] <= r) lo = mid; else hi = mid - 1;
      }
      const int j = r - s_row0[lo];
      p.row_to_pair[r] = j < s_cnt[lo] ? s_cpair[s_c0[lo] + j] : -1;
    }
    if (tid < min(t_live * TK, PQ)) p.pair_to_row[tid] = s_prow[tid];
  };

  // ---- per-wave task stream. A workgroup takes a contiguous block of the
  // tasks (neighbouring row blocks of an expert stay on one CU, which streams
  // faster than spreading them), the blocks split as evenly as the grid
  // allows. With few tasks (1 token: one per 16 weight rows of each live
  // expert) S waves of a workgroup share each task, each over its own 1/S of
  // K; S is the largest power of two up to 8 that still leaves at most one
  // task per group of S waves and divides the K blocks.
  const int n_rb = I / 8;  // 16-row blocks (8 gate + 8 up rows)
  const int KS = W4 ? KB / 2 : KB;  // weight stages per task (MXFP4: two K blocks each)
  const int n_tasks = s_tp[n_live] * n_rb;
  const int G1 = gridDim.x;
  // (blockIdx.x + 1) * n_tasks < 2^32: n_tasks <= 64 tiles x I / 8.
  const int t_lo = static_cast<int>(blockIdx.x * static_cast<uint32_t>(n_tasks) / static_cast<uint32_t>(G1));
  const int t_hi = static_cast<int>((blockIdx.x + 1) * static_cast<uint32_t>(n_tasks) / static_cast<uint32_t>(G1));
  const int wg_max = (n_tasks + G1 - 1) / G1;  // tasks of the fullest workgroup
  int lgS = 0;  // S = 2^lgS
  while (lgS < 3 && (wg_max << (lgS + 1)) <= kF1Waves && (KS & ((2 << lgS) - 1)) == 0) ++lgS;
  lgS = __builtin_amdgcn_readfirstlane(lgS);
  const int S = 1 << lgS;
  const int NG = kF1Waves >> lgS;  // groups of S waves in a workgroup
  const int gl = wave >> lgS;      // this wave's group
  const int kbs = KS >> lgS;       // weight stages of a share
  const int kb_lo = (wave & (S - 1)) * kbs, kb_hi = kb_lo + kbs;
  const int my_tasks = gl < t_hi - t_lo ? ((t_hi - t_lo - 1 - gl) >> (3 - lgS)) + 1 : 0;
  const int total = my_tasks * kbs;  // stages of this wave
  uint8_t* ring = s_ring + wave * (DEPTH * kF1Stage);
  const int grow = lane >> 3;
  const int chunk_lo = ((lane & 7) ^ ((grow >> 1) & 7)) << 4;        // slab row grow
  const int chunk_hi = ((lane & 7) ^ (((grow + 8) >> 1) & 7)) << 4;  // slab row grow + 8
  struct Task {
    int ent, rb, mt;
  };
  // Quotient of non-negative integers a < 2^24 and b > 0 with a / b < 2^16:
  // the float estimate is off by less than one.
  auto small_div = [](int a, int b) {
    int q = static_cast<int>(static_cast<float>(a) * __builtin_amdgcn_rcpf(static_cast<float>(b)));
    if (q * b > a) --q;
    if ((q + 1) * b <= a) ++q;
    return q;
  };
  auto decode_task = [&](int t) {
    const int key = small_div(t, n_rb);
    // Entries whose tile prefix is <= key: a prefix of the entries (the
    // prefixes do not decrease), entry 0's is 0.
    Task k;
    k.ent = static_cast<int>(__popcll(__ballot(lane < n_live && tp_lane <= key))) - 1;
    const int base = __builtin_amdgcn_readlane(tp_lane, k.ent);
    const int next = k.ent + 1 < 64 ? __builtin_amdgcn_readlane(tp_lane, (k.ent + 1) & 63) : tp_end;
    const int tiles = next - base;
    const int local = t - base * n_rb;
    k.rb = small_div(local, tiles);
    k.mt = local - k.rb * tiles;
    return k;
  };
  // Issue side: stage pointers of the current task. Stand-ins (valid
  // addresses) serve the stages past a wave's last one that the stream start
  // issues so that it always issues the same number of loads.
  int i_task = t_lo + gl, i_kb = kb_lo;
  const uint8_t* i_w0 = p.w + lane * 16;
  const uint8_t* i_w1 = p.w + lane * 16;
  const uint8_t* i_s = static_cast<const uint8_t*>(p.w_scales);
  auto i_set = [&]() {
    const Task k = decode_task(i_task);
    const int e = __builtin_amdgcn_readlane(e_lane, k.ent);
    const int jg = k.rb * 8;  // first gate column
    const int64_t rs = W4 ? H / 2 : H;  // bytes per weight row
    const uint8_t* we = p.w + static_cast<int64_t>(e) * N * rs;
    i_w0 = we + static_cast<int64_t>(jg + grow) * rs + chunk_lo;
    i_w1 = we + static_cast<int64_t>(I + jg + grow) * rs + chunk_hi;
    if constexpr (W4) {
      // Lane 2r + h (and 32 + 2r + h) loads scale bytes 4h..4h+3 of slab row
      // r: gate rows 0..7, up rows 8..15.
      const int r = (lane & 31) >> 1;
      const int wr = r < 8 ? jg + r : I + jg + r - 8;
      i_s = static_cast<const uint8_t*>(p.w_scales) + (static_cast<int64_t>(e) * N + wr) * (H / kMxBlock) + (lane & 1) * 4;
    } else {
      // Lane 1 loads the up rows' block scale, every other lane the gate rows'.
      const int sb = lane == 1 ? (I + jg) / kGroup : jg / kGroup;
      i_s = reinterpret_cast<const uint8_t*>(static_cast<const float*>(p.w_scales) +
                                             (static_cast<int64_t>(e) * (N / kGroup) + sb) * KB);
    }
  };
  auto issue_stage = [&](uint8_t* st) {
    __builtin_amdgcn_global_load_lds(i_w0 + i_kb * kGroup, (lds_void*)(st), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(i_w1 + i_kb * kGroup, (lds_void*)(st + 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(i_s + i_kb * (W4 ? 8 : 4), (lds_void*)(st + kF1StageW), 4, 0, 0);
  };
  auto advance = [&]() {
    if (++i_kb == kb_hi) {
      i_kb = kb_lo;
      i_task += NG;
      if (i_task < t_hi) i_set();
    }
  };
  if (total > 0) i_set();
  // Stream start: always DEPTH - 1 stages; past the wave's last stage the
  // stand-ins repeat it (or the initial addresses) and are never read.
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) {
    issue_stage(ring + d * kF1Stage);
    if (d + 1 < total) advance();
  }

  // ---- 2. all tokens' codes and scales into LDS (workgroup 0 also stores
  // them to the workspace); 16 lanes per group, as moe_act_quant
  const int l16 = tid & 15;
#pragma unroll
  for (int k = 0; k < kXLoads; ++k) {
    const int ci = tid + k * kF1Threads;
    if (ci >= n_chunks) break;  // whole 16-lane groups (512 is a multiple of 16)
    const int gid = ci >> 4;
    const int t = gid / gpr, g = gid % gpr;
    if (t >= t_live) continue;  // tokens past the live count: not written
    float sc;
    const uint2 codes = quantize8<FMT>(unpack_bf16x8(xr[k]), &sc, p.rounding);
    *reinterpret_cast<uint2*>(s_x + t * XS + g * kGroup + l16 * 8) = codes;
    if (l16 == 0) s_xs[t * KB + g] = sc;
    if (blockIdx.x == 0) {
      *reinterpret_cast<uint2*>(p.xq + static_cast<int64_t>(t) * H + g * kGroup + l16 * 8) = codes;
      if (l16 == 0) store_scale(p.xs, FMT, static_cast<int64_t>(g) * p.t_cap + t, sc);
    }
  }
  lds_barrier();  // tokens visible to every wave

  // ---- 3. stream: wait for stage s, refill the slot of stage s - 1, compute s
  const int tok = lane & 15;
  // fragment chunks c0f, c0f + 1 of a 128-byte K block (MXFP4: token chunks g, g + 4)
  const int c0f = W4 ? (lane >> 4) : 2 * (lane >> 4);
  const uint32_t x_base = lds_addr(s_x) + c0f * 16;
  const uint32_t xs_base = lds_addr(s_xs);
  int c_task = t_lo + gl, c_kb = kb_lo, slot = 0, c_iter = 0;
  Task ck{0, 0, 0};
  int c_rows = 0, c_crow0 = 0, c_t = 0;  // task's live rows in the tile, compact row base, lane's token
  auto c_set = [&]() {
    ck = decode_task(c_task);
    const int cnt = __builtin_amdgcn_readfirstlane(s_cnt[ck.ent]);
    c_rows = min(kStreamTileM, cnt - ck.mt * kStreamTileM);
    c_crow0 = __builtin_amdgcn_readfirstlane(s_c0[ck.ent]) + ck.mt * kStreamTileM;
    c_t = s_ctok[c_crow0 + min(tok, c_rows - 1)];
  };
  if (total > 0) c_set();
  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const double lim = p.act_limit;
  for (int s = 0; s < total; ++s) {
    // Stages issued after s: DEPTH - 2, or max(DEPTH - 2, total - 1) - s
    // near the end (the start always issues DEPTH - 1), as in
    // fc2_stream_block.
    if (s + DEPTH - 2 >= total)
      wait_stages<kF1Loads>(max(DEPTH - 2, total - 1) - s);
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kF1Loads * (DEPTH - 2)));
    const int prev = slot == 0 ? DEPTH - 1 : slot - 1;
    if (s + DEPTH - 1 < total) {
      issue_stage(ring + prev * kF1Stage);
      advance();
    }
    const uint32_t st = lds_addr(ring + slot * kF1Stage);
    if constexpr (W4) {
      // stage c_kb holds K blocks 2 c_kb and 2 c_kb + 1
      W4Frags f;
      lds_read_stage_w4(st + swz128(tok, c0f), st + swz128(tok, 4 + c0f), st + kF1StageW + 8 * tok + c0f,
                        x_base + c_t * XS + c_kb * 2 * kGroup, xs_base + (c_t * KB + 2 * c_kb) * 4, f);
      acc = w4_stage_step(f, acc);
    } else {
      union {
        uint4 u[2];
        v8i v;
      } wf, af;
      float sa, sw;
      const uint32_t ta = x_base + c_t * XS + c_kb * kGroup;
      lds_read_stage(st + swz128(tok, c0f), st + swz128(tok, c0f + 1), ta, ta + 16,
                    xs_base + (c_t * KB + c_kb) * 4, st + kF1StageW + ((lane >> 5) << 2), wf.u[0],
                    wf.u[1], af.u[0], af.u[1], sa, sw);
      acc = fma4(mfma_fp8(wf.v, af.v), sa * sw, acc);
    }
    if (++c_kb == kb_hi) {
      // This wave's share of the task is done. With S > 1 the partial goes to
      // LDS and the last share of the group to arrive adds the S partials in
      // wave order (a fixed order, whoever arrives last) and stores.
      bool store = true;
      if (S > 1) {
        const uint32_t part = lds_addr(s_part) + (((c_iter & 1) * kF1Waves) * 64 + lane) * 16;
        const uint32_t mine = part + wave * 1024;
        asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(mine), "v"(acc) : "memory");
        int old = 0;
        if (lane == 0) old = atomicAdd(&s_arrive[wave / S], 1);
        old = __builtin_amdgcn_readfirstlane(old);
        store = (old + 1) % S == 0;
        if (store) {
          const uint32_t first = part + (wave / S) * S * 1024;
          acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          for (int w = 0; w < S; ++w) {
            v4f v;
            asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(first + w * 1024) : "memory");
            acc += v;
          }
        }
      }
      // Task done. Lanes 0..31 hold gate columns jg + 4 (lane / 16) + v of
      // token tok, lanes 32..63 the up values of the same columns.
      const uint2 packed = pack_bf16x4(acc);
      uint2 other;
      other.x = __shfl_xor(packed.x, 32, 64);
      other.y = __shfl_xor(packed.y, 32, 64);
      if (store && tok < c_rows) {
        const int jg = ck.rb * 8;
        const int col = (lane < 32 ? jg : I + jg) + 4 * ((lane >> 4) & 1);
        const int64_t row = s_crow[c_crow0 + tok];
        *reinterpret_cast<uint2*>(p.c1 + row * N + col) = packed;
        if (lane < 32) {
          float4 av;
          av.x = swiglu_any(p.act, bf16_to_f32(packed.x & 0xFFFFu), bf16_to_f32(other.x & 0xFFFFu), lim, p.rounding);
          av.y = swiglu_any(p.act, bf16_to_f32(packed.x >> 16), bf16_to_f32(other.x >> 16), lim, p.rounding);
          av.z = swiglu_any(p.act, bf16_to_f32(packed.y & 0xFFFFu), bf16_to_f32(other.y & 0xFFFFu), lim, p.rounding);
          av.w = swiglu_any(p.act, bf16_to_f32(packed.y >> 16), bf16_to_f32(other.y >> 16), lim, p.rounding);
          if constexpr (FUSED)  // read by other workgroups after the grid barrier
            gstore_b128_wt(p.act_out + row * I + col, u32x4{__float_as_uint(av.x), __float_as_uint(av.y),
                                                            __float_as_uint(av.z), __float_as_uint(av.w)});
          else
            *reinterpret_cast<float4*>(p.act_out + row * I + col) = av;
        }
      }
      acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      c_kb = kb_lo;
      c_task += NG;
      ++c_iter;
      if (c_task < t_hi) c_set();
    }
    slot = slot == DEPTH - 1 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // stand-in stages of a wave with few stages
  if (!FUSED && blockIdx.x == 0) write_alignment();
  if constexpr (FUSED) {
    // ---- 4. FC2 and the top-k combine in the same launch (fc2_decode.h). A
    // workgroup owns 16 output columns of every live expert (column blocks
    // blockIdx.x + G j), as launch_down_combine; the list of live experts and
    // their rows is the routing above.
    const int G = gridDim.x;
    const int n_cb = H / 16;
    DecodeTables t;
    t.e = s_e;
    t.cnt = s_cnt;
    t.c0 = s_c0;
    t.r0 = s_row0;
    t.row = s_crow;
    t.pair = s_cpair;
    t.p2r = s_prow;
    t.tw = s_tw;
    t.n_list = n_live;
    t.n_rows = n_live > 0 ? __builtin_amdgcn_readfirstlane(s_c0[n_live - 1] + s_cnt[n_live - 1]) : 0;
    t.n_pairs = PQ;
    uint8_t* const s_tok = s_x;                             // FC2 input codes, row stride I + 16
    float* const s_sa = s_xs;                               // their scales
    float* const s_slot = reinterpret_cast<float*>(s_part);  // pair q's 16 columns
    Fc2Stream<W4> st;
    st.init(q.w, q.w_scales, t, ring, H, I, wave, lane);
    int cb = blockIdx.x;
    const bool has_cb = cb < n_cb;  // uniform
    // The first FC2 stages go out before the barrier: the ring of a wave is
    // free once its FC1 stream is done, and the weights do not depend on FC1.
    if (has_cb) st.start(cb * 16, 0, kDecPreStages);

    // ---- grid barrier. Every wave has waited for its act stores (write-
    // through) above; after the workgroup barrier thread 0 publishes the
    // workgroup's epoch, workgroup 0 waits for every workgroup's epoch and
    // releases the epoch. Waits are bounded: one that gives up is counted,
    // workgroup 0 then releases with the failure bit, and every workgroup
    // that gave up or saw that bit writes NaN to its output columns of the
    // live tokens instead of computing them (the act rows it would read may
    // be incomplete) and reports it in its status slot.
    __shared__ int s_failed;
    lds_barrier();
    if (tid == 0) {
      s_failed = 0;
      flag_store(&g_dl_flag[blockIdx.x], epoch);
    }
    lds_barrier();
    const int limit = a.spin_limit;
    if (blockIdx.x == 0) {
      bool ok = true;
      for (int j = tid; j < G; j += kF1Threads) ok &= flag_wait(&g_dl_flag[j], epoch, limit);
      if (!ok) s_failed = 1;
      lds_barrier();
      if (tid == 0) flag_store(&g_dl_release, s_failed ? (epoch | kDlFailBit) : epoch);
    } else if (tid == 0) {
      if (!flag_wait(&g_dl_release, epoch, limit, kDlEpochMask) || (flag_load(&g_dl_release) & kDlFailBit))
        s_failed = 1;
    }
    if (blockIdx.x == 0) write_alignment();
    for (int x = tid; x < PQ * 16; x += kF1Threads) s_slot[x] = 0.0f;  // the K-split partials are done
    lds_barrier();
    const bool failed = s_failed != 0;  // uniform
    if (tid == 0 && a.status) a.status[blockIdx.x] = failed ? 1 : 0;
    if (failed) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the FC2 stages issued above
      for (int c = cb; c < n_cb; c += G)
        for (int x = tid; x < t_live * 2; x += kF1Threads) {
          const uint4 nan = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
          *reinterpret_cast<uint4*>(q.out + static_cast<int64_t>(x >> 1) * H + c * 16 + 8 * (x & 1)) = nan;
        }
      return;
    }

    // ---- 5. this wave's FC2 input rows, read at device scope (other
    // workgroups wrote them), then the rest of the stream start
    if (has_cb) {
      fc2_quant_rows<FMT, true>(t, wave, lane, p.act_out, I, s_tok, s_sa, blockIdx.x == 0, q.hq, q.hs,
                                q.row_cap, nullptr, nullptr, nullptr, q.rounding);
      st.start(cb * 16, kDecPreStages, DEPTH - 1);
    }
    // ---- 6. stream and combine per column block
    for (; cb < n_cb; cb += G) {
      const int n0 = cb * 16;
      if (cb != static_cast<int>(blockIdx.x)) {
        for (int x = tid; x < PQ * 16; x += kF1Threads) s_slot[x] = 0.0f;
        lds_barrier();  // zeroed slots visible
        st.start(n0, 0, DEPTH - 1);
      }
      fc2_stream_block<DEPTH>(st, n0, t, s_tok, s_sa, s_slot, lane);
      lds_barrier();  // every slot of this column block written
      fc2_combine(t, s_slot, t_live, TK, p.row_cap, H, n0, q.out, q.y, tid);
      lds_barrier();  // slots free for the next column block
    }
  }
}

}  // namespace

hipError_t launch_fc1_decode(const DecodeFc1Args& a, hipStream_t stream) {
  if (a.t_cap == 0) return hipSuccess;
  if (!fc1_decode_fits(a.t_cap, a.topk, a.hidden, a.inter) || a.num_experts > kMaxExperts ||
      a.num_experts < 1 || a.align_rows < 1)
    return hipErrorInvalidValue;
  DecodeLayerArgs l{};
  l.f1 = a;
  const dim3 grid(static_cast<unsigned>(device_cu_count()));
  if (a.weight_fmt != kWeightE4m3) return hipErrorInvalidValue;  // FC1 alone: FP8 weights
  if (a.fmt == kFp32)
    hipLaunchKernelGGL((fc1_decode_kernel<kFp32, false, kDecDepth, false>), grid, dim3(kF1Threads), 0, stream, l);
  else if (a.fmt == kFp32Pow2)
    hipLaunchKernelGGL((fc1_decode_kernel<kFp32Pow2, false, kDecDepth, false>), grid, dim3(kF1Threads), 0, stream, l);
  else
    hipLaunchKernelGGL((fc1_decode_kernel<kUe8m0, false, kDecDepth, false>), grid, dim3(kF1Threads), 0, stream, l);
  return hipGetLastError();
}

// The grid barrier needs every workgroup resident at once: one per CU, at
// most kDlMaxGrid, and the same grid on every launch on a device (the
// epochs count launches per workgroup; both variants use that grid).
int decode_layer_grid(bool wide) {
  static std::atomic<int> cache[2][64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[wide][dev].load(std::memory_order_relaxed);
  if (v != 0) return v > 0 ? v : 0;
  int cus = 0, occ = 0;
  const hipError_t e =
      wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fc1_decode_kernel<kFp32, true, 4, false>, kF1Threads, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fc1_decode_kernel<kFp32, true, kDecDepth, false>, kF1Threads, 0);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      e != hipSuccess || cus < 1 || cus > kDlMaxGrid || occ < 1)
    v = -1;
  else
    v = cus;
  cache[wide][dev].store(v, std::memory_order_relaxed);
  return v > 0 ? v : 0;
}

hipError_t launch_decode_layer(const DecodeLayerArgs& a, hipStream_t stream) {
  if (a.f1.t_cap == 0) return hipSuccess;
  const bool wide = decode_layer_wide(a.f1.t_cap, a.f1.hidden);
  const int grid = decode_layer_grid(wide);
  if (!decode_layer_fits_fmt(a.f1.t_cap, a.f1.topk, a.f1.hidden, a.f1.inter, a.f1.weight_fmt) ||
      grid < 1 || a.f1.num_experts > kMaxExperts || a.f1.num_experts < 1 || a.f1.align_rows < 1)
    return hipErrorInvalidValue;
  auto launch = [&](auto depth, auto w4) {
    constexpr int D = decltype(depth)::value;
    constexpr bool W = decltype(w4)::value;
    if (a.f1.fmt == kFp32)
      hipLaunchKernelGGL((fc1_decode_kernel<kFp32, true, D, W>), dim3(grid), dim3(kF1Threads), 0, stream, a);
    else if (a.f1.fmt == kFp32Pow2)
      hipLaunchKernelGGL((fc1_decode_kernel<kFp32Pow2, true, D, W>), dim3(grid), dim3(kF1Threads), 0, stream, a);
    else
      hipLaunchKernelGGL((fc1_decode_kernel<kUe8m0, true, D, W>), dim3(grid), dim3(kF1Threads), 0, stream, a);
  };
  auto by_depth = [&](auto w4) {
    if (wide)
      launch(std::integral_constant<int, 4>{}, w4);
    else
      launch(std::integral_constant<int, kDecDepth>{}, w4);
  };
  if (a.f1.weight_fmt == kWeightMxfp4)
    by_depth(std::true_type{});
  else
    by_depth(std::false_type{});
  return hipGetLastError();
}

namespace {
std::atomic<int> g_spin_limit{kDlSpinDefault};
}  // namespace

void set_decode_layer_spin_limit(int polls) { g_spin_limit.store(polls, std::memory_order_relaxed); }
int decode_layer_spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

hipError_t decode_layer_timeouts(uint32_t* out) {
  return hipMemcpyFromSymbol(out, HIP_SYMBOL(g_dl_timeouts), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
}

}  // namespace moe
