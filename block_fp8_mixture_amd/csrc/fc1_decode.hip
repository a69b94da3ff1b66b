// FC1 of a decode-sized layer, with the routing alignment and the activation
// quantization in its prologue: one launch instead of two.
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
//     Token fragments come from the resident LDS copy.
//  3. Epilogue of a task. One cross-lane swap pairs gate and up values; C1
//     gets both BF16 halves, and act the fp32 SiLU(gate) * up of the
//     BF16-rounded pair (fp64 inside, rounded once).
#include "device_common.h"
#include "gemm_device.h"
#include "kernels.h"
#include "quant_device.h"

namespace moe {
namespace {

constexpr int kF1Threads = 512;
constexpr int kF1Waves = kF1Threads / 64;
constexpr int kF1Depth = 6;                  // stages in a wave's ring
constexpr int kF1StageW = 16 * kGroup;       // 8 gate + 8 up rows x 128 bytes
constexpr int kF1Stage = kF1StageW + 256;    // + the two weight scales (64 x 4-byte slots)
constexpr int kF1Loads = 3;                  // loads per wave and stage
constexpr int kF1XLoads = kF1TokBytes / 8 / kF1Threads;  // 16-byte (8-value) activation loads per thread

__device__ __forceinline__ uint32_t lds_addr(const void* q) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(q));
}

// A stage's reads: weight fragments, token fragments and both scales, in
// flight together under one wait (assembly: the compiler neither sees reads
// that might alias the direct-to-LDS loads in flight nor uses a result early).
__device__ __forceinline__ void f1_read_stage(uint32_t w0, uint32_t w1, uint32_t t0, uint32_t t1,
                                              uint32_t sa, uint32_t sw, uint4& rw0, uint4& rw1,
                                              uint4& rt0, uint4& rt1, float& fsa, float& fsw) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %8\n\t"
      "ds_read_b128 %3, %9\n\t"
      "ds_read_b32 %4, %10\n\t"
      "ds_read_b32 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(rw0), "=&v"(rw1), "=&v"(rt0), "=&v"(rt1), "=&v"(fsa), "=&v"(fsw)
      : "v"(w0), "v"(w1), "v"(t0), "v"(t1), "v"(sa), "v"(sw));
}

template <int FMT>
__global__ __launch_bounds__(kF1Threads, 1) void fc1_decode_kernel(DecodeFc1Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kF1Waves * kF1Depth * kF1Stage];
  __shared__ __attribute__((aligned(16))) uint8_t s_x[kF1TokBytes];  // codes, row stride H + 16
  __shared__ float s_xs[kF1MaxScales];    // token scale of (token, K block) at t * KB + kb
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int TK = p.topk, E = p.num_experts, H = p.hidden, I = p.inter, N = 2 * I;
  const int KB = H / kGroup, XS = H + 16, A = p.align_rows;
  const int PQ = p.t_cap * TK;  // <= kDcMaxPairs
  const int gpr = H / kGroup;   // activation groups per token

  // ---- 1. everything the prologue reads, issued together
  const int my_id = tid < PQ ? p.ids[tid] : -1;
  const int t_live = p.t_live_dev ? min(max(scalar_load(p.t_live_dev), 0), p.t_cap) : p.t_cap;
  const int n_chunks = p.t_cap * H / 8;  // 16-byte chunks of x
  uint4 xr[kF1XLoads];
#pragma unroll
  for (int k = 0; k < kF1XLoads; ++k) {
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
  // The first entry whose expert is >= e (n_live if none).
  auto entry_ge = [&](int e) {
    int lo = 0, hi = n_live;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_e[mid] < e) lo = mid + 1; else hi = mid;
    }
    return lo;
  };

  // ---- the alignment to the workspace (workgroup 0), as moe_align writes it
  if (blockIdx.x == 0) {
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
  }

  // ---- per-wave task stream. With few tasks (1 token: one per 16 weight
  // rows of each live expert) S waves of a workgroup share each task, each
  // over its own 1/S of K; S is the largest power of two up to 8 that still
  // leaves at most one task per group of S waves and divides the K blocks.
  const int n_rb = I / 8;  // 16-row blocks (8 gate + 8 up rows)
  const int n_tasks = s_tp[n_live] * n_rb;
  const int NW = gridDim.x * kF1Waves;
  int S = 1;
  while (S < kF1Waves && n_tasks * (2 * S) <= NW && KB % (2 * S) == 0) S *= 2;
  S = __builtin_amdgcn_readfirstlane(S);
  const int NG = NW / S;                                   // groups of S waves
  const int gidx = blockIdx.x * (kF1Waves / S) + wave / S;  // this wave's group
  const int kbs = KB / S;                                  // K blocks of a share
  const int kb_lo = (wave % S) * kbs, kb_hi = kb_lo + kbs;
  const int my_tasks = gidx < n_tasks ? (n_tasks - 1 - gidx) / NG + 1 : 0;
  const int total = my_tasks * kbs;  // stages of this wave
  uint8_t* ring = s_ring + wave * (kF1Depth * kF1Stage);
  const int grow = lane >> 3;
  const int chunk_lo = ((lane & 7) ^ ((grow >> 1) & 7)) << 4;        // slab row grow
  const int chunk_hi = ((lane & 7) ^ (((grow + 8) >> 1) & 7)) << 4;  // slab row grow + 8
  struct Task {
    int ent, rb, mt;
  };
  auto decode_task = [&](int t) {
    const int key = t / n_rb;
    int lo = 0, hi = n_live - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tp[mid] <= key) lo = mid; else hi = mid - 1;
    }
    Task k;
    k.ent = __builtin_amdgcn_readfirstlane(lo);
    const int tiles = __builtin_amdgcn_readfirstlane(s_tp[lo + 1] - s_tp[lo]);
    const int local = t - __builtin_amdgcn_readfirstlane(s_tp[lo]) * n_rb;
    k.rb = local / tiles;
    k.mt = local % tiles;
    return k;
  };
  // Issue side: stage pointers of the current task. Stand-ins (valid
  // addresses) serve the stages past a wave's last one that the stream start
  // issues so that it always issues the same number of loads.
  int i_task = gidx, i_kb = kb_lo;
  const uint8_t* i_w0 = p.w + lane * 16;
  const uint8_t* i_w1 = p.w + lane * 16;
  const uint8_t* i_s = reinterpret_cast<const uint8_t*>(p.w_scales);
  auto i_set = [&]() {
    const Task k = decode_task(i_task);
    const int e = __builtin_amdgcn_readfirstlane(s_e[k.ent]);
    const int jg = k.rb * 8;  // first gate column
    const uint8_t* we = p.w + static_cast<int64_t>(e) * N * H;
    i_w0 = we + static_cast<int64_t>(jg + grow) * H + chunk_lo;
    i_w1 = we + static_cast<int64_t>(I + jg + grow) * H + chunk_hi;
    // Lane 1 loads the up rows' block scale, every other lane the gate rows'.
    const int sb = lane == 1 ? (I + jg) / kGroup : jg / kGroup;
    i_s = reinterpret_cast<const uint8_t*>(p.w_scales + (static_cast<int64_t>(e) * (N / kGroup) + sb) * KB);
  };
  auto issue_stage = [&](uint8_t* st) {
    __builtin_amdgcn_global_load_lds(i_w0 + i_kb * kGroup, (lds_void*)(st), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(i_w1 + i_kb * kGroup, (lds_void*)(st + 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(i_s + i_kb * 4, (lds_void*)(st + kF1StageW), 4, 0, 0);
  };
  auto advance = [&]() {
    if (++i_kb == kb_hi) {
      i_kb = kb_lo;
      i_task += NG;
      if (i_task < n_tasks) i_set();
    }
  };
  if (total > 0) i_set();
  // Stream start: always kF1Depth - 1 stages; past the wave's last stage the
  // stand-ins repeat it (or the initial addresses) and are never read.
#pragma unroll
  for (int d = 0; d < kF1Depth - 1; ++d) {
    issue_stage(ring + d * kF1Stage);
    if (d + 1 < total) advance();
  }

  // ---- 2. all tokens' codes and scales into LDS (workgroup 0 also stores
  // them to the workspace); 16 lanes per group, as moe_act_quant
  const int l16 = tid & 15;
#pragma unroll
  for (int k = 0; k < kF1XLoads; ++k) {
    const int ci = tid + k * kF1Threads;
    if (ci >= n_chunks) break;  // whole 16-lane groups (512 is a multiple of 16)
    const int gid = ci >> 4;
    const int t = gid / gpr, g = gid % gpr;
    if (t >= t_live) continue;  // tokens past the live count: not written
    float sc;
    const uint2 codes = quantize8<FMT>(unpack_bf16x8(xr[k]), &sc);
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
  const int c0f = 2 * (lane >> 4);  // fragment chunks c0f, c0f + 1 of a 128-byte K block
  const uint32_t x_base = lds_addr(s_x) + c0f * 16;
  const uint32_t xs_base = lds_addr(s_xs);
  int c_task = gidx, c_kb = kb_lo, slot = 0, c_iter = 0;
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
    if (s + kF1Depth - 2 >= total)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kF1Loads * (kF1Depth - 2)));
    const int prev = slot == 0 ? kF1Depth - 1 : slot - 1;
    if (s + kF1Depth - 1 < total) {
      issue_stage(ring + prev * kF1Stage);
      advance();
    }
    const uint32_t st = lds_addr(ring + slot * kF1Stage);
    union {
      uint4 u[2];
      v8i v;
    } wf, af;
    float sa, sw;
    const uint32_t ta = x_base + c_t * XS + c_kb * kGroup;
    f1_read_stage(st + swz128(tok, c0f), st + swz128(tok, c0f + 1), ta, ta + 16,
                  xs_base + (c_t * KB + c_kb) * 4, st + kF1StageW + ((lane >> 5) << 2), wf.u[0],
                  wf.u[1], af.u[0], af.u[1], sa, sw);
    acc = fma4(mfma_fp8(wf.v, af.v), sa * sw, acc);
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
          float4 a;
          a.x = swiglu_any(p.act, bf16_to_f32(packed.x & 0xFFFFu), bf16_to_f32(other.x & 0xFFFFu), lim);
          a.y = swiglu_any(p.act, bf16_to_f32(packed.x >> 16), bf16_to_f32(other.x >> 16), lim);
          a.z = swiglu_any(p.act, bf16_to_f32(packed.y & 0xFFFFu), bf16_to_f32(other.y & 0xFFFFu), lim);
          a.w = swiglu_any(p.act, bf16_to_f32(packed.y >> 16), bf16_to_f32(other.y >> 16), lim);
          *reinterpret_cast<float4*>(p.act_out + row * I + col) = a;
        }
      }
      acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      c_kb = kb_lo;
      c_task += NG;
      ++c_iter;
      if (c_task < n_tasks) c_set();
    }
    slot = slot == kF1Depth - 1 ? 0 : slot + 1;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // stand-in stages of a wave with few stages
}

}  // namespace

hipError_t launch_fc1_decode(const DecodeFc1Args& a, hipStream_t stream) {
  if (a.t_cap == 0) return hipSuccess;
  if (!fc1_decode_fits(a.t_cap, a.topk, a.hidden, a.inter) || a.num_experts > kMaxExperts ||
      a.num_experts < 1 || a.align_rows < 1)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(device_cu_count()));
  if (a.fmt == kFp32)
    hipLaunchKernelGGL(fc1_decode_kernel<kFp32>, grid, dim3(kF1Threads), 0, stream, a);
  else if (a.fmt == kFp32Pow2)
    hipLaunchKernelGGL(fc1_decode_kernel<kFp32Pow2>, grid, dim3(kF1Threads), 0, stream, a);
  else
    hipLaunchKernelGGL(fc1_decode_kernel<kUe8m0>, grid, dim3(kF1Threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
