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
//  1. Prologue: the live experts are compacted from the endpoints, and the
//     FC2 input rows of all live pairs (fp32, written by the gated FC1) are
//     quantized into LDS with the 1x128 rule. Workgroup 0 also stores codes
//     and scales to the workspace, bit-identical to moe_silu_mul_quant.
//  2. Each wave streams the 16 x I weight slab of every 8th listed expert
//     through a private ring of 2 KB stages (16 rows x one 128-wide K block)
//     by direct-to-LDS loads of whole 128-byte lines. A wave only waits for
//     its own loads, so the loop has no workgroup barrier. Per stage and
//     16-token tile: one v_mfma_f32_16x16x128_f8f6f4 (token = lane % 16,
//     weight row = 4 * (lane / 16) + v) and acc += t * (sa * sw). After the
//     last K block each live row's BF16-rounded result goes to the LDS slot
//     of its (token, k) pair.
//  3. Epilogue: out[t, cols] = BF16(sum over ascending k of w[t, k] * slot)
//     with fp32 FMAs -- the arithmetic and order of moe_topk_combine -- and
//     the rows to the workspace's FC2 output.
#include "device_common.h"
#include "gemm_device.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kDcThreads = 512;
constexpr int kDcWaves = kDcThreads / 64;
constexpr int kDcDepth = 6;               // stages in a wave's ring
constexpr int kDcStageW = 16 * kGroup;    // 16 weight rows x 128 bytes
constexpr int kDcStage = kDcStageW + 256; // + the stage's weight block scale (64 x 4-byte slots)
constexpr int kDcLoads = 3;               // loads per wave and stage
constexpr int kDcTiles = kDcMaxPairs / kStreamTileM;  // token tiles of one expert, at most

template <int FMT>
__global__ __launch_bounds__(kDcThreads, 1) void down_combine_kernel(DownCombineArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kDcWaves * kDcDepth * kDcStage];
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
  __shared__ int s_wn[kDcWaves], s_wr[kDcWaves];
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
    if (c == 1 && E <= kDcThreads) break;  // uniform
    const int e = tid + c * kDcThreads;
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
  for (int x = tid; x < PQ * 16; x += kDcThreads) s_slot[x] = 0.0f;  // ordered by the barriers below
  int run_n = 0, run_r = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c == 1 && E <= kDcThreads) break;  // uniform
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
    for (int w = 0; w < kDcWaves; ++w) {
      bn += w < wave ? s_wn[w] : 0;
      br += w < wave ? s_wr[w] : 0;
    }
    const int i = bn + pos, c0 = br + incl - cnt;
    if (flag && i < list_cap && c0 + cnt <= row_cap_lds) {  // the valid entries form a prefix
      s_e[i] = tid + c * kDcThreads;
      s_cnt[i] = cnt;
      s_c0[i] = c0;
      s_r0[i] = row0_c[c];
      atomicMax(&s_nlist, i + 1);
      atomicMax(&s_nrows, c0 + cnt);
    }
#pragma unroll
    for (int w = 0; w < kDcWaves; ++w) {
      run_n += s_wn[w];
      run_r += s_wr[w];
    }
    __syncthreads();
  }
  // Nothing is in flight yet; an explicit wait here also tells the compiler
  // that the endpoint loads are done on every path, so it does not wait for
  // them (and with them for the prefetch below) when it reuses their registers.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  const int n_list = __builtin_amdgcn_readfirstlane(s_nlist);
  const int n_rows = __builtin_amdgcn_readfirstlane(s_nrows);

  // Compact row c of list entry `ent`: a search over the entries' first rows.
  auto entry_of = [&](int c) {
    int lo = 0, hi = n_list - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_c0[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  // ---- per-wave weight stream of column block n0
  const int my_n = wave < n_list ? (n_list - 1 - wave) / kDcWaves + 1 : 0;
  const int total = my_n * KB;  // stages of this wave
  uint8_t* ring = s_ring + wave * (kDcDepth * kDcStage);
  const int grow = lane >> 3;
  const int chunk_lo = ((lane & 7) ^ ((grow >> 1) & 7)) << 4;        // slab row grow
  const int chunk_hi = ((lane & 7) ^ (((grow + 8) >> 1) & 7)) << 4;  // slab row grow + 8
  int i_ent = wave, i_kb = 0;
  // Stand-ins (valid addresses) for the stages past a wave's last one that
  // the stream start issues so that it always issues the same number.
  const uint8_t* i_w0 = p.w + lane * 16;
  const uint8_t* i_w1 = p.w + lane * 16;
  const uint8_t* i_s = reinterpret_cast<const uint8_t*>(p.w_scales);
  auto i_set = [&](int n0) {
    const int e = __builtin_amdgcn_readfirstlane(s_e[i_ent]);
    const uint8_t* wb = p.w + (static_cast<int64_t>(e) * N + n0) * I;
    i_w0 = wb + static_cast<int64_t>(grow) * I + chunk_lo;
    i_w1 = wb + static_cast<int64_t>(grow + 8) * I + chunk_hi;
    i_s = reinterpret_cast<const uint8_t*>(p.w_scales + (static_cast<int64_t>(e) * (N / kGroup) + n0 / kGroup) * KB);
  };
  auto issue = [&](uint8_t* st, int n0) {
    __builtin_amdgcn_global_load_lds(i_w0 + i_kb * kGroup, (lds_void*)(st), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(i_w1 + i_kb * kGroup, (lds_void*)(st + 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(i_s + i_kb * 4, (lds_void*)(st + kDcStageW), 4, 0, 0);
    if (++i_kb == KB) {
      i_kb = 0;
      i_ent += kDcWaves;
      if (i_ent < n_list) i_set(n0);
    }
  };
  // Always kDcDepth - 1 stages (kDcLoads loads each), so the compiler knows how
  // many loads follow anything issued before, and a wave with fewer stages
  // fills the rest of its ring with stand-in loads that are never read.
  auto start_stream = [&](int n0) {
    i_ent = wave;
    i_kb = 0;
    if (total > 0) i_set(n0);
#pragma unroll
    for (int d = 0; d < kDcDepth - 1; ++d) {
      __builtin_amdgcn_global_load_lds(i_w0 + i_kb * kGroup, (lds_void*)(ring + d * kDcStage), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(i_w1 + i_kb * kGroup, (lds_void*)(ring + d * kDcStage + 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(i_s + i_kb * 4, (lds_void*)(ring + d * kDcStage + kDcStageW), 4, 0, 0);
      // Advance to stage d + 1 if it exists: the loop's issues then
      // continue from stage kDcDepth - 1, and past the last stage the
      // stand-ins repeat it.
      if (d + 1 < total && ++i_kb == KB) {
        i_kb = 0;
        i_ent += kDcWaves;
        i_set(n0);
      }
    }
  };
  // ---- 1b. FC2 input rows of this wave's experts (every 8th listed one).
  // 16 lanes per row, 4 rows per pass; lanes l16 and chunks u cover columns
  // 4 * (16 u + l16) of a 512-column chunk, so a 128-column group is u = 2g,
  // 2g + 1 over the 16 lanes. A wave's MFMAs read only the rows it quantizes
  // itself, so no workgroup barrier separates this from its weight stream.
  const int l16 = lane & 15, lg = lane >> 4;
  const bool writer = blockIdx.x == 0;
  int my_rows = 0;
  for (int i = wave; i < n_list; i += kDcWaves) my_rows += s_cnt[i];
  my_rows = __builtin_amdgcn_readfirstlane(my_rows);
  // Compact and source row of this wave's k-th row (k < my_rows).
  auto wave_row = [&](int k, int* c, int* r) {
    for (int i = wave; i < n_list; i += kDcWaves) {
      const int cnt = s_cnt[i];
      if (k < cnt) {
        *c = s_c0[i] + k;
        *r = s_r0[i] + k;
        return;
      }
      k -= cnt;
    }
    *c = 0;
    *r = 0;
  };
  auto load_chunk = [&](float4* v, int r, int col0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // columns past I (unused) load a valid stand-in
      const int col = min(col0 + 4 * (16 * u + l16), I - 4);
      v[u] = *reinterpret_cast<const float4*>(p.act + static_cast<int64_t>(r) * I + col);
    }
  };
  // Quantizes chunk col0 of compact row c (source row r) into LDS, and for
  // workgroup 0 into the workspace.
  auto quant_chunk = [&](const float4* v, bool row_ok, int c, int r, int col0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int colg = col0 + g * kGroup;
      if (colg >= I) break;  // uniform
      const float4 a = v[2 * g], b = v[2 * g + 1];
      float amax = fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
      amax = group_max<16>(amax);
      const float sc = group_scale(amax, FMT);
      const float inv = 1.0f / sc;  // IEEE division, once per group
      const uint32_t qa = cvt_pk_e4m3(scale_div(a.x, sc, inv, FMT), scale_div(a.y, sc, inv, FMT)) |
                          (cvt_pk_e4m3(scale_div(a.z, sc, inv, FMT), scale_div(a.w, sc, inv, FMT)) << 16);
      const uint32_t qb = cvt_pk_e4m3(scale_div(b.x, sc, inv, FMT), scale_div(b.y, sc, inv, FMT)) |
                          (cvt_pk_e4m3(scale_div(b.z, sc, inv, FMT), scale_div(b.w, sc, inv, FMT)) << 16);
      const int ca = col0 + 4 * (32 * g + l16), cbb = ca + 64;
      if (row_ok) {
        *reinterpret_cast<uint32_t*>(s_tok + c * TS + ca) = qa;
        *reinterpret_cast<uint32_t*>(s_tok + c * TS + cbb) = qb;
        if (l16 == 0) s_sa[c * KB + colg / kGroup] = sc;
        if (writer) {
          *reinterpret_cast<uint32_t*>(p.hq + static_cast<int64_t>(r) * I + ca) = qa;
          *reinterpret_cast<uint32_t*>(p.hq + static_cast<int64_t>(r) * I + cbb) = qb;
          if (l16 == 0) store_scale(p.hs, FMT, static_cast<int64_t>(colg / kGroup) * p.row_cap + r, sc);
        }
      }
    }
  };
  // Prefetch of the first pass (4 rows, first 512 columns) and its row-map
  // entries as untracked loads, then the stream start's kDcLoads * (kDcDepth
  // - 1) loads; waiting until only those remain waits for the prefetch and
  // nothing of the stream.
  float4 v[8];
  u32x4 vr[8];
  uint32_t pair_first = 0;
  int c_first = 0, r_first = 0;
  const bool row_first = lg < my_rows;
  if (my_rows > 0) {  // uniform
    wave_row(lg, &c_first, &r_first);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      vr[u] = gload_b128(p.act + static_cast<int64_t>(r_first) * I + min(4 * (16 * u + l16), I - 4));
    pair_first = gload_b32(p.row_to_pair + r_first);
  }
  int cb = blockIdx.x;  // < n_cb: the grid has at most n_cb workgroups
  start_stream(cb * 16);
  if (my_rows > 0) {
    static_assert(kDcLoads * (kDcDepth - 1) == 15, "wait immediate below");
    asm volatile("s_waitcnt vmcnt(15)"
                 : "+v"(vr[0]), "+v"(vr[1]), "+v"(vr[2]), "+v"(vr[3]), "+v"(vr[4]), "+v"(vr[5]),
                   "+v"(vr[6]), "+v"(vr[7]), "+v"(pair_first));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u].x = __uint_as_float(vr[u][0]);
      v[u].y = __uint_as_float(vr[u][1]);
      v[u].z = __uint_as_float(vr[u][2]);
      v[u].w = __uint_as_float(vr[u][3]);
    }
    if (row_first && l16 == 0) {
      s_row[c_first] = r_first;
      s_pair[c_first] = static_cast<int>(pair_first);
    }
    quant_chunk(v, row_first, c_first, r_first, 0);
  }
  // Further chunks and rows (beyond the decode sizes).
  for (int k0 = 0; k0 < my_rows; k0 += 4) {
    const bool row_ok = k0 + lg < my_rows;
    int c = 0, r = 0;
    wave_row(row_ok ? k0 + lg : 0, &c, &r);
    if (k0 > 0 && row_ok && l16 == 0) {
      s_row[c] = r;
      s_pair[c] = p.row_to_pair[r];
    }
    for (int col0 = k0 == 0 ? 512 : 0; col0 < I; col0 += 512) {
      load_chunk(v, r, col0);
      quant_chunk(v, row_ok, c, r, col0);
    }
    // Tells the compiler these loads are done on every path out of the loop
    // (they are: their values were used), so code after it does not wait.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  // The loop below reads these rows through assembly the compiler does not
  // see; keep the stores above it.
  asm volatile("" ::: "memory");

  const int tok = lane & 15;
  const int c0 = 2 * (lane >> 4);  // fragment chunks c0, c0 + 1 of a 128-byte K block
  const uint32_t tok_base = lds_addr(s_tok) + c0 * 16;
  const uint32_t sa_base = lds_addr(s_sa);

  for (; cb < n_cb; cb += G) {
    const int n0 = cb * 16;
    if (cb != static_cast<int>(blockIdx.x)) {
      for (int x = tid; x < PQ * 16; x += kDcThreads) s_slot[x] = 0.0f;
      lds_barrier();  // zeroed slots visible
      start_stream(n0);
    }

    // ---- 2. stream: wait for stage s, refill the slot of stage s - 1, compute s.
    int c_ent = wave, c_kb = 0, slot = 0;
    int e_cnt = 0, e_c0 = 0;
    if (c_ent < n_list) {
      e_cnt = __builtin_amdgcn_readfirstlane(s_cnt[c_ent]);
      e_c0 = __builtin_amdgcn_readfirstlane(s_c0[c_ent]);
    }
    v4f acc[kDcTiles];
#pragma unroll
    for (int m = 0; m < kDcTiles; ++m) acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < total; ++s) {
      if (s + kDcDepth - 2 >= total)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDcLoads * (kDcDepth - 2)));
      const int prev = slot == 0 ? kDcDepth - 1 : slot - 1;
      if (s + kDcDepth - 1 < total) issue(ring + prev * kDcStage, n0);
      const uint32_t st = lds_addr(ring + slot * kDcStage);
      union {
        uint4 u[2];
        v8i v;
      } wf, af;
      const int n_mt = (e_cnt + kStreamTileM - 1) / kStreamTileM;
      float sa, sw;
      {
        const int row = min(e_c0 + tok, n_rows - 1);
        const uint32_t ta = tok_base + row * TS + c_kb * kGroup;
        lds_read_stage(st + swz128(tok, c0), st + swz128(tok, c0 + 1), ta, ta + 16,
                       sa_base + (row * KB + c_kb) * 4, st + kDcStageW, wf.u[0], wf.u[1], af.u[0],
                       af.u[1], sa, sw);
        acc[0] = fma4(mfma_fp8(wf.v, af.v), sa * sw, acc[0]);
      }
#pragma unroll
      for (int m = 1; m < kDcTiles; ++m) {
        if (m < n_mt) {
          const int row = min(e_c0 + m * kStreamTileM + tok, n_rows - 1);
          const uint32_t ta = tok_base + row * TS + c_kb * kGroup;
          lds_read_tile(ta, ta + 16, sa_base + (row * KB + c_kb) * 4, af.u[0], af.u[1], sa);
          acc[m] = fma4(mfma_fp8(wf.v, af.v), sa * sw, acc[m]);
        }
      }
      if (++c_kb == KB) {  // expert done: BF16-rounded rows to their pairs' slots
#pragma unroll
        for (int m = 0; m < kDcTiles; ++m) {
          const int j = m * kStreamTileM + tok;
          if (m < n_mt && j < e_cnt) {
            const int q = s_pair[e_c0 + j];
            if (static_cast<unsigned>(q) < static_cast<unsigned>(PQ)) {
              float4 o;
              o.x = bf16_to_f32(f32_to_bf16(acc[m][0]));
              o.y = bf16_to_f32(f32_to_bf16(acc[m][1]));
              o.z = bf16_to_f32(f32_to_bf16(acc[m][2]));
              o.w = bf16_to_f32(f32_to_bf16(acc[m][3]));
              *reinterpret_cast<float4*>(s_slot + q * 16 + 4 * (lane >> 4)) = o;
            }
          }
          acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
        c_kb = 0;
        c_ent += kDcWaves;
        if (c_ent < n_list) {
          e_cnt = __builtin_amdgcn_readfirstlane(s_cnt[c_ent]);
          e_c0 = __builtin_amdgcn_readfirstlane(s_c0[c_ent]);
        }
      }
      slot = slot == kDcDepth - 1 ? 0 : slot + 1;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // stand-in stages of a wave with few stages
    lds_barrier();  // every slot of this column block written

    // ---- 3. top-k sum of the 16 columns (two threads per token), then the
    // FC2 output rows (two threads per compact row).
    for (int x = tid; x < t_live * 2; x += kDcThreads) {
      const int t = x >> 1, h = x & 1;
      float a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = 0.0f;
      for (int k0 = 0; k0 < TK; k0 += 8) {
        bool ok[8];
        float w[8];
        float4 lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int q = t * TK + min(k0 + j, TK - 1);
          ok[j] = k0 + j < TK && static_cast<unsigned>(s_p2r[q]) < static_cast<unsigned>(p.row_cap);
          w[j] = s_tw[q];
          lo[j] = *reinterpret_cast<const float4*>(s_slot + q * 16 + 8 * h);
          hi[j] = *reinterpret_cast<const float4*>(s_slot + q * 16 + 8 * h + 4);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (!ok[j]) continue;
          a[0] = fmaf(w[j], lo[j].x, a[0]);
          a[1] = fmaf(w[j], lo[j].y, a[1]);
          a[2] = fmaf(w[j], lo[j].z, a[2]);
          a[3] = fmaf(w[j], lo[j].w, a[3]);
          a[4] = fmaf(w[j], hi[j].x, a[4]);
          a[5] = fmaf(w[j], hi[j].y, a[5]);
          a[6] = fmaf(w[j], hi[j].z, a[6]);
          a[7] = fmaf(w[j], hi[j].w, a[7]);
        }
      }
      uint4 o;
      o.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
      o.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
      o.z = f32_to_bf16(a[4]) | (f32_to_bf16(a[5]) << 16);
      o.w = f32_to_bf16(a[6]) | (f32_to_bf16(a[7]) << 16);
      *reinterpret_cast<uint4*>(p.out + static_cast<int64_t>(t) * N + n0 + 8 * h) = o;
    }
    for (int x = tid; x < n_rows * 2; x += kDcThreads) {
      const int c = x >> 1, h = x & 1;
      const int q = s_pair[c];
      if (static_cast<unsigned>(q) >= static_cast<unsigned>(PQ)) continue;
      const float* v = s_slot + q * 16 + 8 * h;
      uint4 o;
      o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
      o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
      *reinterpret_cast<uint4*>(p.y + static_cast<int64_t>(s_row[c]) * N + n0 + 8 * h) = o;
    }
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
    hipLaunchKernelGGL(down_combine_kernel<kFp32>, dim3(grid), dim3(kDcThreads), 0, stream, a);
  else if (a.fmt == kFp32Pow2)
    hipLaunchKernelGGL(down_combine_kernel<kFp32Pow2>, dim3(grid), dim3(kDcThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(down_combine_kernel<kUe8m0>, dim3(grid), dim3(kDcThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
