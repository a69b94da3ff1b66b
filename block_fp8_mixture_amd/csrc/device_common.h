// Device helpers shared by the gfx950 kernels of the FP8 expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;  // activation quantization group and weight block edge

// ---- BF16 -----------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even; inputs are finite by contract.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- activation scale (vLLM PR #65794, Details: max(amax/448, 1/(448*512))) ----

enum ScaleFmt : int { kFp32 = 0, kFp32Pow2 = 1, kUe8m0 = 2 };

// The float32 scale a group is divided by. amax/448 is an IEEE division (the
// library is built without fast-math, so it is correctly rounded); the floor
// constant 1/229376 is folded by the compiler with correct rounding. The
// power-of-two forms round up: a non-zero mantissa bumps the exponent.
__device__ __forceinline__ float group_scale(float amax, int fmt) {
  float s = fmaxf(amax / 448.0f, 1.0f / 229376.0f);
  if (fmt != kFp32) {
    uint32_t u = __float_as_uint(s);
    if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
    s = __uint_as_float(u);
  }
  return s;
}

// Stored scale -> float (UE8M0 byte b is 2^(b-127); b >= 1 here).
__device__ __forceinline__ float load_scale(const void* base, int fmt, int64_t idx) {
  if (fmt == kUe8m0) {
    uint32_t b = static_cast<const uint8_t*>(base)[idx];
    return __uint_as_float(b << 23);
  }
  return static_cast<const float*>(base)[idx];
}

__device__ __forceinline__ void store_scale(void* base, int fmt, int64_t idx, float s) {
  if (fmt == kUe8m0)
    static_cast<uint8_t*>(base)[idx] = static_cast<uint8_t>(__float_as_uint(s) >> 23);
  else
    static_cast<float*>(base)[idx] = s;
}

// x / s for one element, as the rule states it. For power-of-two scales the
// reciprocal is exact, so multiplying by it gives the same correctly rounded
// quotient with one instruction.
__device__ __forceinline__ float scale_div(float x, float s, float inv_pow2, int fmt) {
  return fmt == kFp32 ? x / s : x * inv_pow2;
}

// Two float32 values -> two E4M3 codes (low 16 bits: a in byte 0, b in byte 1).
// gfx950's v_cvt_pk_fp8_f32 rounds to nearest even in the OCP E4M3 format and
// agrees with that rounding for every |x| <= 464; quotients here never exceed
// 448*(1+2^-22), and the clamp keeps even out-of-contract inputs from
// producing the NaN code.
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// ---- wave helpers ------------------------------------------------------------

// Max over aligned groups of `width` lanes (width a power of two <= 64).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ int clamp_live(const int32_t* t_live_dev, int t_cap) {
  if (t_live_dev == nullptr) return t_cap;
  int t = *t_live_dev;
  return t < 0 ? 0 : (t > t_cap ? t_cap : t);
}

// Expert owning aligned row r: the last e with offsets[e] <= r (offsets has
// E+1 non-decreasing entries, offsets[0] = 0). Requires r < offsets[E].
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int num_experts, int r) {
  int lo = 0, hi = num_experts - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
