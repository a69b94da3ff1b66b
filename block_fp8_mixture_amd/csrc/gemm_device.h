// Device helpers shared by the FP8 GEMM kernels: MFMA and scale steps,
// direct-to-LDS bookkeeping (wait immediates, barrier without a fence,
// swizzled 128-byte rows) and segment checks of the expert endpoints.
#pragma once

#include "device_common.h"

namespace moe {

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

// Four values to BF16 (round to nearest even, as f32_to_bf16 for finite
// values), two per v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint2 pack_bf16x4(v4f v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2);
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Live rows of expert e, or 0 when its endpoints do not describe a segment
// inside [0, row_cap): metadata that is not what moe_align produces can make
// results meaningless but never makes a kernel touch memory out of bounds.
__device__ __forceinline__ int segment_rows(int o0, int o1, int c, int row_cap) {
  if (o0 < 0 || o1 < o0 || o1 > row_cap || c <= 0) return 0;
  return c < o1 - o0 ? c : o1 - o0;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(4))) const int const_int;

// Load through the scalar data cache (a uniform address). Scalar loads are
// counted by lgkmcnt, apart from the vector-memory queue, so waiting for one
// never waits for the direct-to-LDS loads in flight.
__device__ __forceinline__ int scalar_load(const int* q) { return *(const const_int*)(q); }

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (gfx9 layout: vmcnt bits [3:0] and [15:14], expcnt and
// lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Waits until at most n (uniform, 0..4) stages of L vector-memory operations
// each are outstanding; s_waitcnt takes only an immediate.
template <int L>
__device__ __forceinline__ void wait_stages(int n) {
  static_assert(4 * L <= 63, "vmcnt range");
  if (n >= 4)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * L));
  else if (n == 3)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * L));
  else if (n == 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L));
  else if (n == 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Byte offset of 16-byte chunk c of row `row` in a slab of 128-byte rows.
// Rows are written whole (8 lanes x 16 bytes each); chunk c of a row sits in
// slot c ^ ((row >> 1) & 7), which gives the 16 lanes one ds_read_b128 cycle
// serves (16 consecutive rows, the same chunk) distinct bank groups on the
// 64 four-byte banks of gfx950's LDS.
__device__ __forceinline__ uint32_t swz128(int row, int c) {
  return static_cast<uint32_t>(row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
}

// Workgroup barrier for the pipelined K loop. A fence (as in
// __syncthreads()) would make the compiler wait for every vector-memory
// operation in flight, including the direct-to-LDS loads of later stages, and
// so collapse the pipeline. Instead the caller waits for exactly the data the
// next stage needs (explicit vmcnt), this waits for the wave's own LDS
// writes, and the "memory" clobber keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// LDS byte address of a __shared__ object (for assembly operands).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// A stage's reads for the first token tile: weight and token fragments and
// the two scales, all in flight together under one wait. Assembly: the
// compiler then neither sees reads that might alias the direct-to-LDS loads
// in flight (which would make it wait for all of them) nor uses a result
// early.
__device__ __forceinline__ void lds_read_stage(uint32_t w0, uint32_t w1, uint32_t t0, uint32_t t1,
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

// Token fragments and scale of a further token tile.
__device__ __forceinline__ void lds_read_tile(uint32_t t0, uint32_t t1, uint32_t sa, uint4& rt0,
                                              uint4& rt1, float& fsa) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(rt0), "=&v"(rt1), "=&v"(fsa)
      : "v"(t0), "v"(t1), "v"(sa));
}

// Global loads the compiler does not track. Its wait insertion does not
// count direct-to-LDS loads as later vector-memory operations, so a register
// load issued before them would be waited for with vmcnt(0), draining the
// weight stream; these are issued and waited for inside assembly instead.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Eight 16-byte loads and one 4-byte load that have all landed when the
// statement ends: issued and waited for (vmcnt(0)) in one assembly
// statement, so no compiler-scheduled code can move or reuse their
// registers while they are in flight. DEVICE: read at device scope (sc1).
template <bool DEVICE>
__device__ __forceinline__ void gload9_wait(const void* const (&a)[8], const void* b, u32x4 (&v)[8],
                                            uint32_t& w) {
  if constexpr (DEVICE)
    asm volatile(
        "global_load_dwordx4 %0, %9, off sc1\n\t"
        "global_load_dwordx4 %1, %10, off sc1\n\t"
        "global_load_dwordx4 %2, %11, off sc1\n\t"
        "global_load_dwordx4 %3, %12, off sc1\n\t"
        "global_load_dwordx4 %4, %13, off sc1\n\t"
        "global_load_dwordx4 %5, %14, off sc1\n\t"
        "global_load_dwordx4 %6, %15, off sc1\n\t"
        "global_load_dwordx4 %7, %16, off sc1\n\t"
        "global_load_dword %8, %17, off\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7]), "=&v"(w)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(b)
        : "memory");
  else
    asm volatile(
        "global_load_dwordx4 %0, %9, off\n\t"
        "global_load_dwordx4 %1, %10, off\n\t"
        "global_load_dwordx4 %2, %11, off\n\t"
        "global_load_dwordx4 %3, %12, off\n\t"
        "global_load_dwordx4 %4, %13, off\n\t"
        "global_load_dwordx4 %5, %14, off\n\t"
        "global_load_dwordx4 %6, %15, off\n\t"
        "global_load_dwordx4 %7, %16, off\n\t"
        "global_load_dword %8, %17, off\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7]), "=&v"(w)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(b)
        : "memory");
}

// Data handed from one workgroup to another inside a launch, across XCDs
// whose L2 caches are not coherent with each other: the store writes
// through to memory (system scope), the reader loads at device scope
// (gload9_wait<true>) -- the cache bits of relaxed atomics of those scopes.
// Untracked: the writer waits for it explicitly.
__device__ __forceinline__ void gstore_b128_wt(void* a, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(a), "v"(v) : "memory");
}

}  // namespace moe
