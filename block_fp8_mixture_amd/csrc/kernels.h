// Host-side launchers of the gfx950 kernels (internal to libmoefp8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 1024;     // LDS tables in align and the GEMM schedulers
constexpr int kStreamTileM = 16;      // row tile of the weight-streaming GEMM
constexpr int kStreamMaxRows = 64;    // experts with at most this many rows stream
constexpr int kTiledTileM = 256;      // row tile of the MFMA-tiled GEMM
constexpr int kColTile = 128;         // column tile (= weight block rows)

// How routed ids become rows: local ids id - expert_start (other ids are
// dropped); batch_cap > 0 selects the batched layout of batch_cap rows per
// expert, whose pairs past the capacity are dropped and counted into
// *overflow (when given).
struct AlignMode {
  int expert_start = 0;
  int batch_cap = 0;
  int32_t* overflow = nullptr;
};

hipError_t launch_align(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                        int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                        int32_t* row_to_pair, int32_t* pair_to_row, AlignMode mode,
                        hipStream_t stream);

// moe_align and moe_act_quant of one layer in a single launch.
// `rounding` below is the quantizers' convention (Rounding in device_common.h).
hipError_t launch_prep(const int32_t* ids, int t_cap, const int32_t* t_live_dev, int topk,
                       int num_experts, int align_rows, int32_t* counts, int32_t* offsets,
                       int32_t* row_to_pair, int32_t* pair_to_row, const uint16_t* x, int hidden,
                       int fmt, int rounding, uint8_t* xq, void* xs, AlignMode mode,
                       hipStream_t stream);

hipError_t launch_act_quant(const uint16_t* x, int t_cap, const int32_t* t_live_dev, int hidden,
                            int fmt, int rounding, uint8_t* xq, void* xs, hipStream_t stream);

// seg_cap > 0: the batched layout, expert e's rows starting at e*seg_cap
// (offsets is then not read).
hipError_t launch_silu_mul_quant(const uint16_t* gate_up, int inter, const int32_t* counts,
                                 const int32_t* offsets, int num_experts, int row_cap, int act,
                                 float clamp_limit, int fmt, int rounding, uint8_t* hq, void* hs,
                                 int seg_cap, hipStream_t stream);

hipError_t launch_topk_combine(const uint16_t* y, int row_cap, const int32_t* pair_to_row,
                               const float* topk_w, int t_cap, const int32_t* t_live_dev,
                               int topk, int hidden, uint16_t* out, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a;
  const void* a_scales;
  int fmt;
  int a_rows;             // leading dimension of a_scales
  const int32_t* a_row_map;
  int a_row_div;
  const uint8_t* w;
  const float* w_scales;
  const int32_t* counts;
  const int32_t* offsets;   // not read when seg_cap > 0
  int num_experts;
  int row_cap;
  int max_rows_per_expert;  // host bound on counts[e]
  int max_live_experts;     // host bound on experts with rows
  int n;
  int k;
  uint16_t* c;
  int32_t* tiles_visited;
  // Gated FC1 (decode layers): when act_out is set, the weight rows are
  // gate rows [0, n/2) and up rows [n/2, n); every 16-row block the kernel
  // visits pairs 8 gate rows with the 8 up rows of the same columns, and
  // besides C it writes act_out[row, j] = act(gate, up) in fp32 ([row_cap,
  // n/2]) from the BF16-rounded C values. Needs a row map and experts of at
  // most kStreamMaxRows rows.
  float* act_out = nullptr;
  int act = 0;
  float act_limit = 0.0f;
  int rounding = 0;  // act_out is BF16-rounded under the reciprocal convention
  // The batched layout: expert e's segment is rows [e*seg_cap, (e+1)*seg_cap)
  // (0: the segments come from offsets).
  int seg_cap = 0;
  // MXFP4 weights (launch_tiled_w4 only): w holds [E, n, k/2] E2M1 codes and
  // w_mx [E, n, k/32] E8M0 bytes; w_scales is not read.
  const uint8_t* w_mx = nullptr;
};

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t stream);

// The 256 x 256 tiled kernel with MXFP4 weights for the experts of more than
// kStreamMaxRows rows, when the launch's bound on its tiles is at least twice
// the CU count; otherwise launches nothing and returns false (*err
// untouched). g.w_mx must be set.
bool launch_tiled_w4(const GemmArgs& g, hipStream_t stream, hipError_t* err);

// The grouped GEMM with MXFP4 weights: w [num_experts, n, k/2] packed E2M1
// codes (the even K element in the low nibble), w_scales [num_experts, n,
// k/32] E8M0 bytes; everything else as GemmArgs.
constexpr int kMxBlock = 32;  // weights per E8M0 scale along K
enum WeightFmt : int { kWeightE4m3 = 0, kWeightMxfp4 = 1 };  // the values of moe_weight_fmt
struct W4Args {
  const uint8_t* a;
  const void* a_scales;
  int fmt;
  int a_rows;
  const int32_t* a_row_map;
  int a_row_div;
  const uint8_t* w;
  const uint8_t* w_scales;
  const int32_t* counts;
  const int32_t* offsets;  // not read when seg_cap > 0
  int seg_cap;
  int num_experts;
  int row_cap;
  int max_rows_per_expert;  // host bound on counts[e]: selects the kernels, never the result
  int n;
  int k;
  uint16_t* c;
};
hipError_t launch_grouped_gemm_w4(const W4Args& g, hipStream_t stream);

// FC2 and the top-k combine of a decode-sized layer in one launch: a
// workgroup owns 16 output columns of every live expert. Limits of its LDS
// tables: at most kDcMaxPairs routed pairs of capacity, their quantized
// rows (I + 16 bytes each) within kDcTokBytes, and pairs x I/128 within
// kDcMaxScales.
constexpr int kDcMaxPairs = 64;
constexpr int kDcTokBytes = 24576;
constexpr int kDcMaxScales = 256;

inline bool down_combine_fits(int64_t t_cap, int64_t topk, int64_t inter) {
  const int64_t pairs = t_cap * topk;
  return pairs >= 1 && pairs <= kDcMaxPairs && pairs * (inter + 16) <= kDcTokBytes &&
         pairs * (inter / 128) <= kDcMaxScales;
}

struct DownCombineArgs {
  const float* act;           // [row_cap, I] fp32 FC2 input before quantization
  int fmt;
  const uint8_t* w;           // [E, H, I] E4M3, or [E, H, I/2] MXFP4 (decode layer only)
  const void* w_scales;       // fp32 [E, H/128, I/128], or E8M0 bytes [E, H, I/32]
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* row_to_pair;
  const int32_t* pair_to_row;
  const float* topk_w;        // [t_cap, topk]
  const int32_t* t_live_dev;  // nullable: t_cap
  int num_experts;
  int row_cap;
  int t_cap;
  int topk;
  int hidden;
  int inter;
  uint8_t* hq;                // [row_cap, I] quantized FC2 input (workspace copy)
  void* hs;                   // [I/128][row_cap] its scales
  uint16_t* y;                // [row_cap, H] FC2 output rows (workspace copy)
  uint16_t* out;              // [t_cap, H]
  int rounding;               // quantizer convention of the FC2 input
};

hipError_t launch_down_combine(const DownCombineArgs& a, hipStream_t stream);

// FC1 of a decode-sized layer with the routing alignment and the activation
// quantization in its prologue (one launch instead of two). Needs the
// decode-path limits above plus all t_cap tokens' codes within kF1TokBytes
// of LDS (row stride H + 16) and t_cap x H/128 scales within kF1MaxScales.
constexpr int kF1TokBytes = 24576;
constexpr int kF1MaxScales = 256;

inline bool fc1_decode_fits(int64_t t_cap, int64_t topk, int64_t hidden, int64_t inter) {
  return down_combine_fits(t_cap, topk, inter) && t_cap * (hidden + 16) <= kF1TokBytes &&
         t_cap * (hidden / 128) <= kF1MaxScales;
}

struct DecodeFc1Args {
  const int32_t* ids;         // [t_cap, topk]
  const int32_t* t_live_dev;  // nullable: t_cap
  int t_cap;
  int topk;
  int num_experts;
  int align_rows;
  int row_cap;
  int expert_start;           // local ids are ids - expert_start
  const uint16_t* x;          // [t_cap, H] BF16
  int hidden;
  int inter;
  int fmt;
  const uint8_t* w;           // [E, 2I, H] E4M3: gate rows [0, I), up rows [I, 2I); MXFP4: [E, 2I, H/2]
  const void* w_scales;       // fp32 [E, 2I/128, H/128], or E8M0 bytes [E, 2I, H/32]
  int weight_fmt;             // kWeightE4m3, or kWeightMxfp4 (one-launch layer only; both halves)
  int act;
  float act_limit;
  int32_t* counts;            // workspace copies, as moe_align writes them
  int32_t* offsets;
  int32_t* row_to_pair;
  int32_t* pair_to_row;
  uint8_t* xq;                // workspace copies, as moe_act_quant writes them
  void* xs;
  uint16_t* c1;               // [row_cap, 2I] BF16
  float* act_out;             // [row_cap, I] fp32 SiLU(gate) * up
  int rounding;               // quantizer convention (and BF16-rounded act when reciprocal)
};

hipError_t launch_fc1_decode(const DecodeFc1Args& a, hipStream_t stream);

// The whole decode layer in one launch: the FC1 kernel above, a barrier
// across the grid (one workgroup per CU, all resident), then FC2 and the
// top-k combine as launch_down_combine computes them. f2's act is f1's
// act_out; its counts, offsets and row maps are not read (the routing is
// the launch's own). Launches on one device must not overlap in time: the
// barrier's epochs live in device globals.
constexpr int kDlMaxGrid = 1024;

// Its variant for more token bytes: a 4-deep weight ring per wave instead
// of 6 leaves room for t_cap x (H + 16) codes within kF1TokBytesWide and
// t_cap x H/128 scales within kF1MaxScalesWide (e.g. 8 tokens of H = 7168).
constexpr int kF1TokBytesWide = 61440;
constexpr int kF1MaxScalesWide = 512;

inline bool decode_layer_wide(int64_t t_cap, int64_t hidden) {
  return t_cap * (hidden + 16) > kF1TokBytes || t_cap * (hidden / 128) > kF1MaxScales;
}

inline bool decode_layer_fits(int64_t t_cap, int64_t topk, int64_t hidden, int64_t inter) {
  return down_combine_fits(t_cap, topk, inter) && hidden % 16 == 0 &&
         t_cap * (hidden + 16) <= kF1TokBytesWide && t_cap * (hidden / 128) <= kF1MaxScalesWide;
}
// With MXFP4 weights a weight stage holds two 128-wide K blocks (16 rows x
// 128 packed bytes), so both K dimensions must be multiples of 256.
inline bool decode_layer_fits_fmt(int64_t t_cap, int64_t topk, int64_t hidden, int64_t inter,
                                  int weight_fmt) {
  if (weight_fmt == kWeightMxfp4 && (hidden % 256 != 0 || inter % 256 != 0)) return false;
  return (weight_fmt == kWeightE4m3 || weight_fmt == kWeightMxfp4) &&
         decode_layer_fits(t_cap, topk, hidden, inter);
}

struct DecodeLayerArgs {
  DecodeFc1Args f1;
  DownCombineArgs f2;
  // Per-workgroup outcome of the grid barrier ([grid] int32, the workspace's
  // status slots): 0 = it opened, 1 = a wait gave up and the workgroup wrote
  // NaN to its output columns instead of computing them.
  int32_t* status;
  // Polls per barrier wait before it gives up; below 0: give up at once
  // (a host-forced timeout, for tests).
  int spin_limit;
};

// Polls per wait of the one-launch layer's grid barrier (about a microsecond
// each) used by subsequent launches in this process; below 0, every wait
// gives up at once. Default kDlSpinDefault.
constexpr int kDlSpinDefault = 1 << 21;
void set_decode_layer_spin_limit(int polls);
int decode_layer_spin_limit();

hipError_t launch_decode_layer(const DecodeLayerArgs& a, hipStream_t stream);
// Grid of launch_decode_layer on the current device (one workgroup per CU),
// or 0 where its workgroups cannot all be resident; `wide`: the variant
// decode_layer_wide selects.
int decode_layer_grid(bool wide);
// Waits at the grid barrier that gave up (sticky, per device).
hipError_t decode_layer_timeouts(uint32_t* out);

int device_cu_count();

}  // namespace moe
