// Device helpers of the 1x128 FP8 quantization and of the gated activation,
// shared by the quantization kernels and the fused kernels of the layer.
//
// Rule (vLLM PR #65794, Details): scale = max(amax / 448, 1 / (448 * 512)),
// codes = E4M3(x / scale); power-of-two scales round up. 16 lanes own one
// 128-element group, 8 consecutive elements each (one 16-byte BF16 load);
// the group amax is a 4-step xor-shuffle reduction inside the 16 lanes.
#pragma once

#include "device_common.h"

namespace moe {

struct Vals8 {
  float v[8];
};

__device__ __forceinline__ Vals8 unpack_bf16x8(uint4 raw) {
  Vals8 r;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    r.v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  return r;
}

// Quantizes the 8 values this lane holds against the group's scale; returns
// the 8 codes packed little-endian and writes the stored scale when asked.
template <int FMT>
__device__ __forceinline__ uint2 quantize8(const Vals8& x, float* scale_out, int rnd) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x.v[i]));
  amax = group_max<16>(amax);
  float inv;
  const float s = group_scale_inv(amax, FMT, rnd, &inv);  // IEEE divisions, once per group
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = scale_apply(x.v[i], s, inv, FMT, rnd);
  uint2 out;
  out.x = cvt_pk_e4m3(q[0], q[1]) | (cvt_pk_e4m3(q[2], q[3]) << 16);
  out.y = cvt_pk_e4m3(q[4], q[5]) | (cvt_pk_e4m3(q[6], q[7]) << 16);
  *scale_out = s;
  return out;
}

// Quantizes group gid (token gid / (hidden / 128), group gid % (hidden / 128))
// of x with the 16 lanes l16 = 0..15 that call it. Groups past t_cap exit;
// groups of tokens past the live count are not written.
template <int FMT>
__device__ __forceinline__ void act_quant_group(const uint16_t* __restrict__ x, int t_cap,
                                                const int32_t* __restrict__ t_live_dev, int hidden,
                                                uint8_t* __restrict__ xq, void* __restrict__ xs,
                                                int64_t gid, int l16, int rnd) {
  const int groups = hidden / kGroup;
  if (gid >= static_cast<int64_t>(t_cap) * groups) return;  // whole 16-lane groups exit
  const int t = static_cast<int>(gid / groups);
  const int g = static_cast<int>(gid % groups);
  const int64_t base = static_cast<int64_t>(t) * hidden + g * kGroup + l16 * 8;
  // The row is inside x whether or not the token is live, so its load is
  // issued together with the live-count load instead of after it.
  const uint4 raw = *reinterpret_cast<const uint4*>(x + base);
  if (t >= clamp_live(t_live_dev, t_cap)) return;
  const Vals8 v = unpack_bf16x8(raw);
  float s;
  const uint2 codes = quantize8<FMT>(v, &s, rnd);
  *reinterpret_cast<uint2*>(xq + base) = codes;
  if (l16 == 0) store_scale(xs, FMT, static_cast<int64_t>(g) * t_cap + t, s);
}

enum Act : int { kSwiglu = 0, kSwigluClamp = 1, kSwigluClampAfterSilu = 2 };

// SiLU(g) * u in double, rounded once to float (vLLM PR #65794, Details: no
// intermediate BF16 rounding). Clamp variants as TensorRT-LLM PR #21250's
// test coverage names them, with limit L: clamp gate above and up to [-L, L]
// before SiLU, or clamp SiLU's output above and up to [-L, L].
__device__ __forceinline__ double silu_f64(double g) { return g / (1.0 + exp(-g)); }

template <int ACT>
__device__ __forceinline__ float swiglu(float gf, float uf, double lim) {
  double g = gf, u = uf;
  if (ACT == kSwigluClamp) {
    g = fmin(g, lim);
    u = fmin(fmax(u, -lim), lim);
  }
  double s = silu_f64(g);
  if (ACT == kSwigluClampAfterSilu) {
    s = fmin(s, lim);
    u = fmin(fmax(u, -lim), lim);
  }
  return static_cast<float>(s * u);
}

// SiLU of BF16 gates by table. A gate is a BF16 value, so silu_f64 of every
// gate with |g| in [2^-12, 2^4) -- where nearly all of them fall -- fits in a
// 32 KB table that a workgroup fills once in LDS with silu_f64 itself; a gate
// outside that range (zero, tiny, huge, not finite, or a clamp limit that is
// not a BF16 value) takes silu_f64 directly. Either way the double is the one
// swiglu() computes, so the results are bit-identical to it; the table only
// replaces an fp64 exp and division per element by an LDS read.
constexpr int kSiluLutLo = 127 - 12;              // biased exponent of 2^-12
constexpr int kSiluLutExps = 16;                  // 2^-12 <= |g| < 2^4
constexpr int kSiluLutSize = kSiluLutExps * 256;  // 128 mantissas x 2 signs per exponent

// Entry i holds the BF16 value with magnitude bits (i >> 1) + (kSiluLutLo << 7)
// and sign i & 1.
__device__ __forceinline__ void fill_silu_lut(double* lut, int tid, int nthreads) {
  for (int i = tid; i < kSiluLutSize; i += nthreads) {
    const uint32_t bits = ((static_cast<uint32_t>(i) & 1u) << 15) |
                          ((static_cast<uint32_t>(i) >> 1) + (kSiluLutLo << 7));
    lut[i] = silu_f64(static_cast<double>(bf16_to_f32(bits)));
  }
}

// Table entry of gate g, or -1 when g is not a tabulated BF16 value.
__device__ __forceinline__ int silu_lut_index(float g) {
  const uint32_t b = __float_as_uint(g);
  const uint32_t mag = ((b >> 16) & 0x7FFFu) - static_cast<uint32_t>(kSiluLutLo << 7);
  return ((b & 0xFFFFu) == 0 && mag < static_cast<uint32_t>(kSiluLutExps * 128))
             ? static_cast<int>(mag * 2 + (b >> 31))
             : -1;
}

// swiglu<ACT> with the SiLU from `lut` (filled by fill_silu_lut) where it
// has the gate.
template <int ACT>
__device__ __forceinline__ float swiglu_lut(float gf, float uf, double lim, const double* lut) {
  float g = gf;
  double u = uf;
  if (ACT == kSwigluClamp) {
    g = static_cast<float>(fmin(static_cast<double>(gf), lim));  // gf or the limit, both floats
    u = fmin(fmax(u, -lim), lim);
  }
  const int i = silu_lut_index(g);
  double s;
  if (i >= 0)
    s = lut[i];
  else
    s = silu_f64(g);
  if (ACT == kSwigluClampAfterSilu) {
    s = fmin(s, lim);
    u = fmin(fmax(u, -lim), lim);
  }
  return static_cast<float>(s * u);
}

// The activation chosen at run time (a uniform branch); under the
// reciprocal convention the result is rounded to BF16 (TensorRT-LLM PR
// #21250, rounding-fix commit message: the fused op's epilogue rounds the
// SwiGLU output to BF16 before its FP8 quantization).
__device__ __forceinline__ float swiglu_any(int act, float g, float u, double lim, int rnd) {
  float y;
  if (act == kSwigluClamp)
    y = swiglu<kSwigluClamp>(g, u, lim);
  else if (act == kSwigluClampAfterSilu)
    y = swiglu<kSwigluClampAfterSilu>(g, u, lim);
  else
    y = swiglu<kSwiglu>(g, u, lim);
  return rnd == kReciprocal ? round_bf16(y) : y;
}

}  // namespace moe
