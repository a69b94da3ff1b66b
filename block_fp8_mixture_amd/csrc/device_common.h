// Device helpers shared by the gfx950 kernels of the FP8 expert layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Rounding conventions of the quantizers. kDivide: the rule above, scale =
// max(fl32(amax/448), fl32(1/229376)) and codes from fl32(x / scale).
// kReciprocal: the fused CUTLASS op's convention that TensorRT-LLM PR #21250
// follows (rounding-fix commit message): multiply by inv = fl32(448 / amax),
// store fl32(1 / inv), with amax floored at 2^-9 (= 448 / (448*512), where the
// divide rule's floor starts to bind) so that an all-zero group stays finite;
// the SwiGLU output is rounded to BF16 before its quantization.
enum Rounding : int { kDivide = 0, kReciprocal = 1 };

// Rounds a power-of-two format's scale up: a non-zero mantissa bumps the exponent.
__device__ __forceinline__ float pow2_ceil(float s) {
  uint32_t u = __float_as_uint(s);
  if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
  return __uint_as_float(u);
}

// The stored (float) scale of a group with this amax, and in *inv the factor
// its elements are multiplied by. Divisions are IEEE (the library is built
// without fast-math, so they are correctly rounded); the constants are folded
// by the compiler with correct rounding. Under kDivide *inv = 1/s, which
// scale_apply refines to the correctly rounded quotient; under kReciprocal
// with fp32 scales *inv is the convention's multiplier itself. Power-of-two
// scales give an exact *inv either way.
__device__ __forceinline__ float group_scale_inv(float amax, int fmt, int rnd, float* inv) {
  float s;
  if (rnd == kReciprocal) {
    const float m = 448.0f / fmaxf(amax, 0x1p-9f);
    s = 1.0f / m;
    if (fmt == kFp32) {
      *inv = m;
      return s;
    }
  } else {
    s = fmaxf(amax / 448.0f, 1.0f / 229376.0f);
  }
  if (fmt != kFp32) s = pow2_ceil(s);
  *inv = 1.0f / s;
  return s;
}

// The divide convention's scale alone.
__device__ __forceinline__ float group_scale(float amax, int fmt) {
  float inv;
  return group_scale_inv(amax, fmt, kDivide, &inv);
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

// x / s for one element, correctly rounded as the rule states it, given
// inv = 1 / s (an IEEE division, once per group). For power-of-two scales inv
// is exact and so is x * inv. Otherwise Markstein's correction: with
// q0 = RN(x * inv) and the exact remainder r = x - q0 * s (one FMA), RN(q0 +
// r * inv) is the correctly rounded quotient when inv is the correctly rounded
// reciprocal and nothing underflows (P. Markstein, IBM J. Res. Dev. 34(1),
// 1990). Here |x / s| <= 448 and s >= 1/229376, and a remainder can only
// underflow for |x / s| far below half the smallest E4M3 subnormal, whose
// code is zero either way. The sign is copied back so that -0 stays -0.
__device__ __forceinline__ float scale_div(float x, float s, float inv, int fmt) {
  const float q0 = x * inv;
  if (fmt != kFp32) return q0;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, inv, q0), x);
}

// One element's value before its E4M3 rounding, as the convention defines it
// (s and inv from group_scale_inv): fl32(x / s) under kDivide, fl32(x * inv)
// under kReciprocal.
__device__ __forceinline__ float scale_apply(float x, float s, float inv, int fmt, int rnd) {
  return rnd == kReciprocal ? x * inv : scale_div(x, s, inv, fmt);
}

// A float rounded to the nearest BF16 value (ties to even), kept as float.
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

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

// Max over aligned groups of `width` lanes (16, 32 or 64). Inside a 16-lane
// row with DPP moves (no LDS round trip): swap neighbours, swap pairs, mirror
// each half row, mirror the row; then across rows through lane reads.
template <int width>
__device__ __forceinline__ float group_max(float v) {
  static_assert(width == 16 || width == 32 || width == 64, "group width");
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xF, 0xF, false));
  };
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
  v = fmaxf(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
  if constexpr (width > 16) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    if constexpr (width == 32) {
      const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      v = lane < 32 ? fmaxf(r0, r1) : fmaxf(r2, r3);
    } else {
      v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
    }
  }
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
