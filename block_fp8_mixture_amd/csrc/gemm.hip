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
// Both kernels compute C^T tiles with v_mfma_f32_16x16x128_f8f6f4: the MFMA
// "A" operand is 16 weight rows x 128 K, "B" is 16 token rows x 128 K, so one
// MFMA covers exactly one 128-wide scale block. Its 16x16 fp32 result sits
// with token = lane % 16 and weight row = 4 * (lane / 16) + v, which makes the
// weight block scale uniform over the wave and the activation scale a single
// value per lane: each K block costs one MFMA into a zeroed temporary and four
// FMAs acc += temp * (sa * sw). Both operands carry 32 consecutive K bytes
// per lane (lane / 16 selects which 32).
//
// Work is found on the device: every workgroup compacts the experts it owns
// (by row count) from expert_counts into LDS, then walks its share of the
// resulting item list, so padded capacity and empty experts cost nothing.
//
//  * gemm_stream_kernel -- experts with 1..64 rows. An item is (expert, 16*WN
//    weight rows); the 4 waves split the item as WN row blocks x KSPLIT K
//    ranges. Weight fragments are loaded once into registers and reused for
//    every 16-row token tile of the expert; K-split partial sums are added in
//    a fixed order through LDS. This is the weight-streaming (HBM-bound) path.
//  * gemm_tiled_kernel -- experts with more rows. 128 token x 128 weight
//    tiles, K step 128, both operands staged through double-buffered LDS with
//    an XOR swizzle of 16-byte chunks (conflict-free fragment reads); 2x2
//    waves of 64x64.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ v4f fma4(v4f t, float s, v4f acc) {
  v4f r;
  r[0] = __builtin_fmaf(t[0], s, acc[0]);
  r[1] = __builtin_fmaf(t[1], s, acc[1]);
  r[2] = __builtin_fmaf(t[2], s, acc[2]);
  r[3] = __builtin_fmaf(t[3], s, acc[3]);
  return r;
}

__device__ __forceinline__ v4f mfma_fp8(v8i w, v8i x) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint2 pack_bf16x4(v4f v) {
  uint2 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  return o;
}

// Live rows of expert e, or 0 when its endpoints do not describe a segment
// inside [0, row_cap): metadata that is not what moe_align produces can make
// results meaningless but never makes a kernel touch memory out of bounds.
__device__ __forceinline__ int expert_rows(const GemmArgs& p, int e) {
  const int o0 = p.offsets[e], o1 = p.offsets[e + 1], c = p.counts[e];
  if (o0 < 0 || o1 < o0 || o1 > p.row_cap || c <= 0) return 0;
  return c < o1 - o0 ? c : o1 - o0;
}

// A row feeding output row r, or -1 when the map points outside A.
__device__ __forceinline__ int a_source_row(const GemmArgs& p, int r) {
  const int ar = p.a_row_map ? p.a_row_map[r] / p.a_row_div : r;
  return static_cast<unsigned>(ar) < static_cast<unsigned>(p.a_rows) ? ar : -1;
}

// Ordered compaction of the experts whose row count satisfies `want`, into
// s_list[0..n). s_pref[i] gets the exclusive prefix sum of units(count) over
// the listed experts and s_pref[n] the total. Returns n. All threads call it.
template <typename Want, typename Units>
__device__ int build_expert_list(const GemmArgs& p, Want want, Units units, int* s_list,
                                 int* s_pref, int* s_tmp) {
  const int num_experts = p.num_experts;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kW = kThreads / 64;
  int run_n = 0, run_u = 0;
  for (int base = 0; base < num_experts; base += kThreads) {
    const int e = base + tid;
    const int cnt = e < num_experts ? expert_rows(p, e) : 0;
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
      s_list[bn + pos] = e;
      s_pref[bn + pos] = bu + incl - u;
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

template <int WN, int KSPLIT>
__global__ __launch_bounds__(kThreads) void gemm_stream_kernel(GemmArgs p) {
  static_assert(WN * KSPLIT == kThreads / 64, "4 waves per item");
  constexpr int KCH = 8;                               // K blocks per register chunk
  __shared__ int s_list[kMaxExperts];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_tmp[2 * kThreads / 64];
  __shared__ v4f s_red[KSPLIT > 1 ? (KSPLIT - 1) * WN * 64 : 1];

  const int n_list = build_expert_list(p, WantSmall(), NoUnits(), s_list, s_pref, s_tmp);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % WN;
  const int ks = wave / WN;
  constexpr int NB = 16 * WN;
  const int N = p.n, K = p.k, KB = K / kGroup;
  const int n_blocks = N / NB;
  const int total = n_list * n_blocks;
  const int kb0 = ks * KB / KSPLIT;
  const int kb1 = (ks + 1) * KB / KSPLIT;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int e = s_list[item / n_blocks];
    const int nb = item % n_blocks;
    const int cnt = expert_rows(p, e);
    const int row0 = p.offsets[e];
    const int n_mt = (cnt + kStreamTileM - 1) / kStreamTileM;
    const int n0 = nb * NB + wn * 16;
    const uint8_t* wp = p.w + (static_cast<int64_t>(e) * N + n0 + (lane & 15)) * K + (lane >> 4) * 32;
    const float* wsp = p.w_scales + (static_cast<int64_t>(e) * (N / kGroup) + n0 / kGroup) * KB;

    // One token tile at a time (decode experts have one); a second tile of
    // the same expert re-reads this wave's weight slice, which is in L2.
    for (int mt = 0; mt < n_mt; ++mt) {
      const int j = mt * kStreamTileM + (lane & 15);
      const int src = j < cnt ? a_source_row(p, row0 + j) : -1;
      const bool rv = src >= 0;
      const int arow = rv ? src : 0;
      const uint8_t* ap = p.a + static_cast<int64_t>(arow) * K + (lane >> 4) * 32;
      v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      for (int kc = kb0; kc < kb1; kc += KCH) {
        v8i wf[KCH], af[KCH];
        float sa[KCH];
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
          if (kc + q < kb1) {
            wf[q] = *reinterpret_cast<const v8i*>(wp + static_cast<int64_t>(kc + q) * kGroup);
            if (rv) {
              af[q] = *reinterpret_cast<const v8i*>(ap + (kc + q) * kGroup);
              sa[q] = load_scale(p.a_scales, p.fmt, static_cast<int64_t>(kc + q) * p.a_rows + arow);
            } else {
              af[q] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
              sa[q] = 0.0f;
            }
          }
        }
#pragma unroll
        for (int q = 0; q < KCH; ++q)
          if (kc + q < kb1) acc = fma4(mfma_fp8(wf[q], af[q]), sa[q] * wsp[kc + q], acc);
      }
      if constexpr (KSPLIT > 1) {
        if (ks > 0) s_red[((ks - 1) * WN + wn) * 64 + lane] = acc;
        __syncthreads();
        if (ks == 0)
          for (int s = 1; s < KSPLIT; ++s) acc = acc + s_red[((s - 1) * WN + wn) * 64 + lane];
        __syncthreads();
      }
      if (ks == 0 && j < cnt)
        *reinterpret_cast<uint2*>(p.c + static_cast<int64_t>(row0 + j) * N + n0 + 4 * (lane >> 4)) =
            pack_bf16x4(acc);
    }
    if (tid == 0 && p.tiles_visited && (nb * NB) % kColTile == 0) atomicAdd(p.tiles_visited, n_mt);
  }
}

// ---------------------------------------------------------------- tiled

constexpr int BM = kTiledTileM;  // token rows per tile
constexpr int BN = kColTile;     // weight rows per tile
constexpr int BK = kGroup;

// Byte offset of 16-byte chunk c of tile row `row` in a [rows][128 B] LDS tile.
__device__ __forceinline__ int swz(int row, int c) { return row * BK + ((c ^ (row & 7)) << 4); }

union Frag {
  uint4 u[2];
  v8i v;
};

__global__ __launch_bounds__(kThreads, 2) void gemm_tiled_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][BN * BK];
  __shared__ float s_sa[2][BM];
  __shared__ int s_list[kMaxExperts];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ int s_tmp[2 * kThreads / 64];

  const int n_list = build_expert_list(p, WantLarge(), TiledUnits(), s_list, s_pref, s_tmp);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;   // token half of the tile
  const int wn = wave >> 1;  // weight half of the tile
  const int N = p.n, K = p.k, KB = K / BK;
  const int n_tn = N / BN;
  const int total = s_pref[n_list] * n_tn;
  const int lrow = tid >> 3;  // load row within a 32-row slab
  const int lc = tid & 7;     // load chunk (16 bytes) within the row

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt_all = tile / n_tn;
    const int nt = tile % n_tn;
    int lo = 0, hi = n_list - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= mt_all) lo = mid; else hi = mid - 1;
    }
    const int e = s_list[lo];
    const int mt = mt_all - s_pref[lo];
    const int cnt = expert_rows(p, e);
    const int rows_here = min(BM, cnt - mt * BM);
    const int row0 = p.offsets[e] + mt * BM;
    const int n0 = nt * BN;

    const uint8_t* asrc[4];
    bool aval[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lrow + 32 * i;
      const int ar = row < rows_here ? a_source_row(p, row0 + row) : -1;
      aval[i] = ar >= 0;
      asrc[i] = p.a + static_cast<int64_t>(aval[i] ? ar : 0) * K + lc * 16;
    }
    const uint8_t* wsrc = p.w + (static_cast<int64_t>(e) * N + n0 + lrow) * K + lc * 16;
    const int sa_row = tid < rows_here ? a_source_row(p, row0 + tid) : -1;
    const float* wsp = p.w_scales + (static_cast<int64_t>(e) * (N / kGroup) + nt) * KB;

    uint4 ra[4], rw[4];
    float rs = 0.0f;
    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = aval[i] ? *reinterpret_cast<const uint4*>(asrc[i] + kb * BK) : uint4{0, 0, 0, 0};
        rw[i] = *reinterpret_cast<const uint4*>(wsrc + static_cast<int64_t>(32 * i) * K + kb * BK);
      }
      if (tid < BM)
        rs = sa_row >= 0 ? load_scale(p.a_scales, p.fmt, static_cast<int64_t>(kb) * p.a_rows + sa_row) : 0.0f;
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int off = swz(lrow + 32 * i, lc);
        *reinterpret_cast<uint4*>(&s_a[buf][off]) = ra[i];
        *reinterpret_cast<uint4*>(&s_w[buf][off]) = rw[i];
      }
      if (tid < BM) s_sa[buf][tid] = rs;
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kb = 0; kb < KB; ++kb) {
      const int cur = kb & 1;
      if (kb + 1 < KB) gload(kb + 1);
      const float sw = wsp[kb];
      float sc[4];
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) sc[ts] = s_sa[cur][wm * 64 + ts * 16 + (lane & 15)] * sw;
      Frag wf[4], af[4];
      const int c0 = 2 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rw_ = wn * 64 + i * 16 + (lane & 15);
        wf[i].u[0] = *reinterpret_cast<const uint4*>(&s_w[cur][swz(rw_, c0)]);
        wf[i].u[1] = *reinterpret_cast<const uint4*>(&s_w[cur][swz(rw_, c0 + 1)]);
        const int ra_ = wm * 64 + i * 16 + (lane & 15);
        af[i].u[0] = *reinterpret_cast<const uint4*>(&s_a[cur][swz(ra_, c0)]);
        af[i].u[1] = *reinterpret_cast<const uint4*>(&s_a[cur][swz(ra_, c0 + 1)]);
      }
#pragma unroll
      for (int ws = 0; ws < 4; ++ws)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
          acc[ws][ts] = fma4(mfma_fp8(wf[ws].v, af[ts].v), sc[ts], acc[ws][ts]);
      if (kb + 1 < KB) lstore(cur ^ 1);
      __syncthreads();
    }

#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      const int j = wm * 64 + ts * 16 + (lane & 15);
      if (j < rows_here) {
        uint16_t* crow = p.c + static_cast<int64_t>(row0 + j) * N + n0 + wn * 64 + 4 * (lane >> 4);
#pragma unroll
        for (int ws = 0; ws < 4; ++ws)
          *reinterpret_cast<uint2*>(crow + ws * 16) = pack_bf16x4(acc[ws][ts]);
      }
    }
    if (tid == 0 && p.tiles_visited) atomicAdd(p.tiles_visited, 1);
  }
}

template <int WN, int KSPLIT>
hipError_t launch_stream(const GemmArgs& g, int live_bound, hipStream_t stream) {
  const int n_blocks = g.n / (16 * WN);
  const int64_t items = static_cast<int64_t>(live_bound) * n_blocks;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  const int grid = static_cast<int>(items < cap ? items : cap);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_stream_kernel<WN, KSPLIT>), dim3(grid), dim3(kThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t stream) {
  const int live_bound = g.max_live_experts < g.num_experts ? g.max_live_experts : g.num_experts;
  if (live_bound <= 0) return hipSuccess;
  const int kb = g.k / kGroup;
  hipError_t err;
  if (kb >= 16) err = launch_stream<1, 4>(g, live_bound, stream);
  else if (kb >= 8) err = launch_stream<2, 2>(g, live_bound, stream);
  else err = launch_stream<4, 1>(g, live_bound, stream);
  if (err != hipSuccess) return err;
  if (g.max_rows_per_expert > kStreamMaxRows) {
    // Row tiles of the large experts: at most ceil(rows / BM) + one partial
    // tile per expert that can be large.
    const int64_t rows = g.row_cap;
    const int64_t large_experts = rows / (kStreamMaxRows + 1) < live_bound ? rows / (kStreamMaxRows + 1) : live_bound;
    const int64_t tiles = ((rows + BM - 1) / BM + large_experts) * (g.n / BN);
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 2;
    const int grid = static_cast<int>(tiles < cap ? tiles : cap);
    if (grid > 0) {
      hipLaunchKernelGGL(gemm_tiled_kernel, dim3(grid), dim3(kThreads), 0, stream, g);
      err = hipGetLastError();
    }
  }
  return err;
}

}  // namespace moe
