// FC2 and the top-k combine of a decode-sized layer for one workgroup that
// owns 16 output columns: the steps shared by the FC2 + combine kernel and
// the one-launch decode layer.
//
// TensorRT-LLM PR #21250 (description; rounding-fix commit): at decode sizes
// FC2 streams the weights of the few live experts, and the top-k sum scales
// the BF16 expert outputs by the routing weights in fp32. vLLM PR #65794
// (Details): the FC2 input is SiLU(gate) * up quantized per 1x128 group.
//
// A workgroup of 8 waves owns output columns n0..n0+15, i.e. 16 W2 rows of
// every live expert, so the whole top-k sum of those columns forms in its
// LDS. Wave w handles every 8th live expert ("entry", in expert order):
//  - it quantizes those experts' FC2 input rows into LDS (only it reads
//    them, so no workgroup barrier is needed before its stream);
//  - it streams their 16 x I weight slabs through a private ring of stages
//    (16 rows x one 128-wide K block + the block scale) by direct-to-LDS
//    loads of whole 128-byte lines, waiting only for its own loads;
//  - per stage and 16-token tile one v_mfma_f32_16x16x128_f8f6f4 (token =
//    lane % 16, weight row = 4 (lane / 16) + v), acc += t * (sa * sw);
//  - after an expert's last K block each live row's BF16-rounded result
//    goes to the LDS slot of its (token, k) pair.
// Then out[t, cols] = BF16(sum over ascending k of w[t, k] * slot), with
// fp32 FMAs in the arithmetic and order of moe_topk_combine.
//
// MXFP4 weights (vLLM PR #59128's description names FP4 weights; read as
// OCP MXFP4: E2M1 codes, two per byte with the even K element in the low
// nibble, one E8M0 scale byte per 32 along K) keep the stage geometry: 16
// weight rows x 128 packed bytes are two 128-wide K blocks, and the third
// load brings the rows' 8 scale bytes of those 256 K values. Per K block one
// v_mfma_scale_f32_16x16x128_f8f6f4 applies the weight scales in the matrix
// core; then acc += t * sa.
#pragma once

#include "device_common.h"
#include "gemm_device.h"
#include "kernels.h"

namespace moe {

constexpr int kDecThreads = 512;                       // decode-path workgroup: 8 waves, one per CU
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecDepth = 6;                           // stages in a wave's ring
constexpr int kDecStageW = 16 * kGroup;                // 16 weight rows x 128 bytes
constexpr int kDecStage = kDecStageW + 256;            // + block scale(s): 64 x 4-byte slots
constexpr int kDecLoads = 3;                           // direct-to-LDS loads per wave and stage
constexpr int kDecTiles = kDcMaxPairs / kStreamTileM;  // 16-token tiles of one expert, at most
constexpr int kDecPreStages = 2;  // stream-start stages issued before the FC2 input rows are loaded

// One 128-wide K block with MXFP4 weights on v_mfma_scale_f32_16x16x128_f8f6f4
// (operand layout measured on gfx950 with in-bounds probes): the E2M1 weights
// are operand A (format 4): lane l holds weight row l % 16 and the K values
// [32 g, 32 g + 32) of the block (g = l / 16), i.e. 16-byte chunk g of the
// row's 64 packed bytes, with that MX block's scale byte as its A scale. The
// E4M3 tokens are operand B: lane l holds token l % 16 and, in that K order,
// the block's values [16 g, 16 g + 16) and [64 + 16 g, 80 + 16 g): 16-byte
// chunks g and 4 + g of its 128 codes (not the chunks 2g, 2g + 1 that the
// FP8 x FP8 instruction pairs). The B scale is 1.0 (E8M0 127). The output
// layout is the FP8 instruction's: token l % 16, weight row 4 (l / 16) + v.
__device__ __forceinline__ v4f mfma_w4(uint4 w, uint4 x0, uint4 x1, uint32_t sc) {
  const v8i a = {static_cast<int>(w.x), static_cast<int>(w.y), static_cast<int>(w.z),
                 static_cast<int>(w.w), 0, 0, 0, 0};
  const v8i b = {static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                 static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                 static_cast<int>(x1.z), static_cast<int>(x1.w)};
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 0, 0, static_cast<int>(sc), 0, 127);
}

// Reads of an MXFP4 stage for one token tile, all under one wait (assembly,
// as lds_read_stage): per K block h = 0, 1 of the stage the weight fragment
// (at w0, w1) and its scale byte (at sb + 4 h), the token fragments (at t,
// t + 64 for h = 0; t + 128, t + 192 for h = 1) and the two token scales
// (adjacent floats at sa, 8-byte aligned).
struct W4Frags {
  uint4 w0, w1, x00, x01, x10, x11;
  uint32_t s0, s1;
  uint2 sa;  // the two token scales' bits
};
__device__ __forceinline__ void lds_read_stage_w4(uint32_t w0, uint32_t w1, uint32_t sb, uint32_t t,
                                                  uint32_t sa, W4Frags& f) {
  asm volatile(
      "ds_read_b128 %0, %9\n\t"
      "ds_read_b128 %1, %10\n\t"
      "ds_read_u8 %2, %11\n\t"
      "ds_read_u8 %3, %11 offset:4\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %12 offset:64\n\t"
      "ds_read_b128 %6, %12 offset:128\n\t"
      "ds_read_b128 %7, %12 offset:192\n\t"
      "ds_read_b64 %8, %13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.w0), "=&v"(f.w1), "=&v"(f.s0), "=&v"(f.s1), "=&v"(f.x00), "=&v"(f.x01), "=&v"(f.x10),
        "=&v"(f.x11), "=&v"(f.sa)
      : "v"(w0), "v"(w1), "v"(sb), "v"(t), "v"(sa));
}
// Token fragments and scales of a further token tile of an MXFP4 stage.
__device__ __forceinline__ void lds_read_tile_w4(uint32_t t, uint32_t sa, W4Frags& f) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:64\n\t"
      "ds_read_b128 %2, %5 offset:128\n\t"
      "ds_read_b128 %3, %5 offset:192\n\t"
      "ds_read_b64 %4, %6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.x00), "=&v"(f.x01), "=&v"(f.x10), "=&v"(f.x11), "=&v"(f.sa)
      : "v"(t), "v"(sa));
}
// The two K blocks of an MXFP4 stage, ascending, into acc.
__device__ __forceinline__ v4f w4_stage_step(const W4Frags& f, v4f acc) {
  acc = fma4(mfma_w4(f.w0, f.x00, f.x01, f.s0), __uint_as_float(f.sa.x), acc);
  return fma4(mfma_w4(f.w1, f.x10, f.x11, f.s1), __uint_as_float(f.sa.y), acc);
}

// A workgroup's live experts ("entries", in expert order) and their rows
// ("compact rows", entry after entry), in LDS.
struct DecodeTables {
  const int* e;     // entry -> expert
  const int* cnt;   // entry -> live rows
  const int* c0;    // entry -> first compact row
  const int* r0;    // entry -> first source row (its aligned rows in the workspace)
  const int* row;   // compact row -> source row
  const int* pair;  // compact row -> pair
  const int* p2r;   // pair -> source row (a pair without one holds a value >= row_cap)
  const float* tw;  // pair -> routing weight
  int n_list;
  int n_rows;
  int n_pairs;      // pairs of capacity (t_cap * topk): the slots in use
};

// One wave's FC2 weight stream over a column block: the 16 x I slab of every
// kDecWaves-th entry, one stage per 128-wide K block (per two with MXFP4
// weights, W4). Stand-ins (valid addresses) fill the stages past the wave's
// last one that the stream start issues, so that it always issues (ring
// depth) - 1 stages.
template <bool W4>
struct Fc2Stream {
  const uint8_t* w;       // [E, H, I] E4M3, or [E, H, I/2] MXFP4
  const void* w_scales;   // fp32 [E, H/128, I/128], or E8M0 bytes [E, H, I/32]
  const int* list_e;
  uint8_t* ring;
  int H, I, KB, n_list, wave, total;  // KB: stages per entry
  int grow, chunk_lo, chunk_hi;
  int srow, shalf;  // MXFP4: slab row and half of this lane's 4 scale bytes (lanes 32..63 repeat 0..31)
  int ent, kb;
  const uint8_t* w0;
  const uint8_t* w1;
  const uint8_t* s;

  __device__ __forceinline__ void init(const uint8_t* w_, const void* ws_, const DecodeTables& t,
                                       uint8_t* ring_, int H_, int I_, int wave_, int lane) {
    w = w_;
    w_scales = ws_;
    list_e = t.e;
    ring = ring_;
    H = H_;
    I = I_;
    KB = W4 ? I_ / (2 * kGroup) : I_ / kGroup;
    srow = (lane & 31) >> 1;
    shalf = lane & 1;
    n_list = t.n_list;
    wave = wave_;
    const int my_n = wave < n_list ? (n_list - 1 - wave) / kDecWaves + 1 : 0;
    total = my_n * KB;
    grow = lane >> 3;
    chunk_lo = ((lane & 7) ^ ((grow >> 1) & 7)) << 4;        // slab row grow
    chunk_hi = ((lane & 7) ^ (((grow + 8) >> 1) & 7)) << 4;  // slab row grow + 8
    ent = wave;
    kb = 0;
    w0 = w + lane * 16;
    w1 = w + lane * 16;
    s = reinterpret_cast<const uint8_t*>(w_scales);
  }
  __device__ __forceinline__ void set(int n0) {
    const int e = __builtin_amdgcn_readfirstlane(list_e[ent]);
    const int64_t rs = W4 ? I / 2 : I;  // bytes per weight row
    const uint8_t* wb = w + (static_cast<int64_t>(e) * H + n0) * rs;
    w0 = wb + static_cast<int64_t>(grow) * rs + chunk_lo;
    w1 = wb + static_cast<int64_t>(grow + 8) * rs + chunk_hi;
    if constexpr (W4)
      s = static_cast<const uint8_t*>(w_scales) + (static_cast<int64_t>(e) * H + n0 + srow) * (I / kMxBlock) + shalf * 4;
    else
      s = reinterpret_cast<const uint8_t*>(static_cast<const float*>(w_scales) +
                                           (static_cast<int64_t>(e) * (H / kGroup) + n0 / kGroup) * (I / kGroup));
  }
  // A stage: two loads of 8 rows x 128 bytes and the scales (FP8: the block
  // scale, every lane; MXFP4: the 16 rows' 8 scale bytes, lane 2r + h
  // bringing bytes 4h..4h+3 of row r to slot 2r + h).
  __device__ __forceinline__ void issue(uint8_t* st) {
    __builtin_amdgcn_global_load_lds(w0 + kb * kGroup, (lds_void*)(st), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(w1 + kb * kGroup, (lds_void*)(st + 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(s + kb * (W4 ? 8 : 4), (lds_void*)(st + kDecStageW), 4, 0, 0);
  }
  __device__ __forceinline__ void advance(int n0) {
    if (++kb == KB) {
      kb = 0;
      ent += kDecWaves;
      if (ent < n_list) set(n0);
    }
  }
  // Stages d0..d1-1 of the stream start of column block n0 (d0 == 0 resets
  // the stream); the start as a whole issues stages 0..DEPTH-2 of the ring
  // it runs on (kDecDepth, or 4 in the wide one-launch layer).
  __device__ __forceinline__ void start(int n0, int d0, int d1) {
    if (d0 == 0) {
      ent = wave;
      kb = 0;
      if (total > 0) set(n0);
    }
    for (int d = d0; d < d1; ++d) {
      issue(ring + d * kDecStage);
      if (d + 1 < total) advance(n0);
    }
  }
};

// This wave's compact rows: the rows of entries wave, wave + kDecWaves, ...
__device__ __forceinline__ int wave_rows(const DecodeTables& t, int wave) {
  int n = 0;
  for (int i = wave; i < t.n_list; i += kDecWaves) n += t.cnt[i];
  return __builtin_amdgcn_readfirstlane(n);
}

// Compact row and source row of this wave's k-th row (k < wave_rows).
__device__ __forceinline__ void wave_row(const DecodeTables& t, int wave, int k, int* c, int* r) {
  for (int i = wave; i < t.n_list; i += kDecWaves) {
    const int cnt = t.cnt[i];
    if (k < cnt) {
      *c = t.c0[i] + k;
      *r = t.r0[i] + k;
      return;
    }
    k -= cnt;
  }
  *c = 0;
  *r = 0;
}

// Quantizes this wave's FC2 input rows (fp32 act, one row of I values per
// source row) into LDS codes (row stride I + 16) and scales (at c * KB + kb)
// with the 1x128 rule; `writer` also stores them to the workspace (hq, hs)
// bit-identical to moe_silu_mul_quant. 16 lanes per row, 4 rows per pass;
// lanes l16 and loads u cover columns 4 (16 u + l16) of a 512-column chunk,
// so a 128-column group is u = 2g, 2g + 1 over the 16 lanes. DEVICE_SCOPE
// reads act at device scope (rows written by other workgroups in the same
// launch). With row_to_pair, the rows' pairs are loaded with them and the
// compact-row tables row[] and pair[] filled.
template <int FMT, bool DEVICE_SCOPE>
__device__ __forceinline__ void fc2_quant_rows(const DecodeTables& t, int wave, int lane, const float* act,
                                               int I, uint8_t* tok, float* sa, bool writer, uint8_t* hq,
                                               void* hs, int row_cap, const int32_t* row_to_pair,
                                               int* row, int* pair, int rnd) {
  const int KB = I / kGroup, TS = I + 16;
  const int l16 = lane & 15, lg = lane >> 4;
  const int my_rows = wave_rows(t, wave);
  for (int k0 = 0; k0 < my_rows; k0 += 4) {
    const bool row_ok = k0 + lg < my_rows;
    int c = 0, r = 0;
    wave_row(t, wave, row_ok ? k0 + lg : 0, &c, &r);
    for (int col0 = 0; col0 < I; col0 += 512) {
      u32x4 vr[8];
      uint32_t pr = 0;
      const void* av[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)  // columns past I (unused) load a valid stand-in
        av[u] = act + static_cast<int64_t>(r) * I + min(col0 + 4 * (16 * u + l16), I - 4);
      // The row's pair, or a stand-in (the row's first value, never used).
      const void* pv = row_to_pair && col0 == 0 ? static_cast<const void*>(row_to_pair + r) : av[0];
      gload9_wait<DEVICE_SCOPE>(av, pv, vr, pr);
      if (row_to_pair && col0 == 0 && row_ok && l16 == 0) {
        row[c] = r;
        pair[c] = static_cast<int>(pr);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int colg = col0 + g * kGroup;
        const bool g_ok = colg < I;  // uniform; past I the loads hold stand-ins, never stored
        const u32x4 ra = vr[2 * g], rb = vr[2 * g + 1];
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = __uint_as_float(ra[j]);
          x[4 + j] = __uint_as_float(rb[j]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
        amax = group_max<16>(amax);
        float inv;
        const float sc = group_scale_inv(amax, FMT, rnd, &inv);  // IEEE divisions, once per group
        auto q = [&](int j) { return scale_apply(x[j], sc, inv, FMT, rnd); };
        const uint32_t qa = cvt_pk_e4m3(q(0), q(1)) | (cvt_pk_e4m3(q(2), q(3)) << 16);
        const uint32_t qb = cvt_pk_e4m3(q(4), q(5)) | (cvt_pk_e4m3(q(6), q(7)) << 16);
        const int ca = col0 + 4 * (32 * g + l16), cb = ca + 64;
        if (row_ok && g_ok) {
          *reinterpret_cast<uint32_t*>(tok + c * TS + ca) = qa;
          *reinterpret_cast<uint32_t*>(tok + c * TS + cb) = qb;
          if (l16 == 0) sa[c * KB + colg / kGroup] = sc;
          if (writer) {
            *reinterpret_cast<uint32_t*>(hq + static_cast<int64_t>(r) * I + ca) = qa;
            *reinterpret_cast<uint32_t*>(hq + static_cast<int64_t>(r) * I + cb) = qb;
            if (l16 == 0) store_scale(hs, FMT, static_cast<int64_t>(colg / kGroup) * row_cap + r, sc);
          }
        }
      }
    }
  }
  // The stream reads these rows through assembly the compiler does not see;
  // keep the stores above it.
  asm volatile("" ::: "memory");
}

// The stream of one column block (started with Fc2Stream::start on a ring of
// DEPTH stages, so the start issued DEPTH - 1 of them): wait for
// stage s, refill the slot of stage s - 1, compute s; after an entry's last
// K block its live rows' BF16-rounded results go to their pairs' slots.
// Ends with the wave's loads drained.
template <int DEPTH, bool W4>
__device__ __forceinline__ void fc2_stream_block(Fc2Stream<W4>& st, int n0, const DecodeTables& t,
                                                 const uint8_t* tok, const float* sa, float* slot,
                                                 int lane) {
  const int KB = st.KB, TS = st.I + 16;
  const int KG = st.I / kGroup;  // token scales per row
  const int tok16 = lane & 15;
  // fragment chunks cf, cf + 1 of a 128-byte K block (MXFP4: token chunks g, g + 4)
  const int cf = W4 ? (lane >> 4) : 2 * (lane >> 4);
  const uint32_t tok_base = lds_addr(tok) + cf * 16;
  const uint32_t sa_base = lds_addr(sa);
  int e_ent = st.wave, e_kb = 0, slotn = 0;
  int e_cnt = 0, e_c0 = 0;
  if (e_ent < t.n_list) {
    e_cnt = __builtin_amdgcn_readfirstlane(t.cnt[e_ent]);
    e_c0 = __builtin_amdgcn_readfirstlane(t.c0[e_ent]);
  }
  v4f acc[kDecTiles];
#pragma unroll
  for (int m = 0; m < kDecTiles; ++m) acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < st.total; ++s) {
    // The start issued DEPTH - 1 stages (stand-ins past the end) and
    // every step one more while any remain, so the stages issued after s
    // number DEPTH - 2 in the steady state and max(DEPTH - 2,
    // total - 1) - s near the end; operations issued among them only make
    // the wait stricter (they retire in order).
    if (s + DEPTH - 2 >= st.total)
      wait_stages<kDecLoads>(max(DEPTH - 2, st.total - 1) - s);
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDecLoads * (DEPTH - 2)));
    const int prev = slotn == 0 ? DEPTH - 1 : slotn - 1;
    if (s + DEPTH - 1 < st.total) {
      st.issue(st.ring + prev * kDecStage);
      st.advance(n0);
    }
    const uint32_t stg = lds_addr(st.ring + slotn * kDecStage);
    const int n_mt = (e_cnt + kStreamTileM - 1) / kStreamTileM;
    if constexpr (W4) {
      // stage e_kb holds K blocks 2 e_kb and 2 e_kb + 1
      W4Frags f;
      {
        const int row = min(e_c0 + tok16, t.n_rows - 1);
        lds_read_stage_w4(stg + swz128(tok16, cf), stg + swz128(tok16, 4 + cf),
                          stg + kDecStageW + 8 * tok16 + cf, tok_base + row * TS + e_kb * 2 * kGroup,
                          sa_base + (row * KG + 2 * e_kb) * 4, f);
        acc[0] = w4_stage_step(f, acc[0]);
      }
#pragma unroll
      for (int m = 1; m < kDecTiles; ++m) {
        if (m < n_mt) {
          const int row = min(e_c0 + m * kStreamTileM + tok16, t.n_rows - 1);
          lds_read_tile_w4(tok_base + row * TS + e_kb * 2 * kGroup, sa_base + (row * KG + 2 * e_kb) * 4, f);
          acc[m] = w4_stage_step(f, acc[m]);
        }
      }
    } else {
    union {
      uint4 u[2];
      v8i v;
    } wf, af;
    float fsa, fsw;
    {
      const int row = min(e_c0 + tok16, t.n_rows - 1);
      const uint32_t ta = tok_base + row * TS + e_kb * kGroup;
      lds_read_stage(stg + swz128(tok16, cf), stg + swz128(tok16, cf + 1), ta, ta + 16,
                     sa_base + (row * KB + e_kb) * 4, stg + kDecStageW, wf.u[0], wf.u[1], af.u[0],
                     af.u[1], fsa, fsw);
      acc[0] = fma4(mfma_fp8(wf.v, af.v), fsa * fsw, acc[0]);
    }
#pragma unroll
    for (int m = 1; m < kDecTiles; ++m) {
      if (m < n_mt) {
        const int row = min(e_c0 + m * kStreamTileM + tok16, t.n_rows - 1);
        const uint32_t ta = tok_base + row * TS + e_kb * kGroup;
        lds_read_tile(ta, ta + 16, sa_base + (row * KB + e_kb) * 4, af.u[0], af.u[1], fsa);
        acc[m] = fma4(mfma_fp8(wf.v, af.v), fsa * fsw, acc[m]);
      }
    }
    }
    if (++e_kb == KB) {  // entry done: BF16-rounded rows to their pairs' slots
#pragma unroll
      for (int m = 0; m < kDecTiles; ++m) {
        const int j = m * kStreamTileM + tok16;
        if (m < n_mt && j < e_cnt) {
          const int q = t.pair[e_c0 + j];
          if (static_cast<unsigned>(q) < static_cast<unsigned>(t.n_pairs)) {
            float4 o;
            o.x = bf16_to_f32(f32_to_bf16(acc[m][0]));
            o.y = bf16_to_f32(f32_to_bf16(acc[m][1]));
            o.z = bf16_to_f32(f32_to_bf16(acc[m][2]));
            o.w = bf16_to_f32(f32_to_bf16(acc[m][3]));
            *reinterpret_cast<float4*>(slot + q * 16 + 4 * (lane >> 4)) = o;
          }
        }
        acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      }
      e_kb = 0;
      e_ent += kDecWaves;
      if (e_ent < t.n_list) {
        e_cnt = __builtin_amdgcn_readfirstlane(t.cnt[e_ent]);
        e_c0 = __builtin_amdgcn_readfirstlane(t.c0[e_ent]);
      }
    }
    slotn = slotn == DEPTH - 1 ? 0 : slotn + 1;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // stand-in stages of a wave with few stages
}

// Top-k sum of a column block's 16 columns (two threads per token) for the
// live tokens, then the FC2 output rows of the compact rows (two threads per
// row). All threads of the workgroup, after the slots are complete.
__device__ __forceinline__ void fc2_combine(const DecodeTables& t, const float* slot, int t_live, int TK,
                                           int row_cap, int H, int n0, uint16_t* out, uint16_t* y,
                                           int tid) {
  for (int x = tid; x < t_live * 2; x += kDecThreads) {
    const int tk = x >> 1, h = x & 1;
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0.0f;
    for (int k0 = 0; k0 < TK; k0 += 8) {
      bool ok[8];
      float w[8];
      float4 lo[8], hi[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = tk * TK + min(k0 + j, TK - 1);
        ok[j] = k0 + j < TK && static_cast<unsigned>(t.p2r[q]) < static_cast<unsigned>(row_cap);
        w[j] = t.tw[q];
        lo[j] = *reinterpret_cast<const float4*>(slot + q * 16 + 8 * h);
        hi[j] = *reinterpret_cast<const float4*>(slot + q * 16 + 8 * h + 4);
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
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(tk) * H + n0 + 8 * h) = o;
  }
  for (int x = tid; x < t.n_rows * 2; x += kDecThreads) {
    const int c = x >> 1, h = x & 1;
    const int q = t.pair[c];
    if (static_cast<unsigned>(q) >= static_cast<unsigned>(t.n_pairs)) continue;
    const float* v = slot + q * 16 + 8 * h;
    uint4 o;
    o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
    o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4*>(y + static_cast<int64_t>(t.row[c]) * H + n0 + 8 * h) = o;
  }
}

}  // namespace moe
