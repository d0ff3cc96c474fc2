// Device helpers shared by the MFMA attention kernels (not part of the ABI).
//
// Layout conventions of every bf16 attention kernel here: a 64-key tile of
// K is staged in LDS token-major (one 2*D-byte row per key), a tile of V^T
// d-major (one 128-byte row of 64 keys per head dim); 16-byte chunks of a
// row are XOR-swizzled by the row index so that the rows read together by
// one MFMA operand load fall in distinct LDS banks.
#pragma once

#include "bca_internal.h"

namespace bca {
namespace attn {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kSlowSum = 1099511627776.0f;   // 2^40: a tile row sum above it raises the overflow flag

// Key order on the rows of a 32-row MFMA block: row m holds key sigma32(m),
// so that each 32-lane half of the S^T accumulator holds 8 consecutive keys
// per 16-key chunk -- the B-operand layout of the following PV MFMA.
__device__ __forceinline__ int sigma32(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// 16-byte chunk swizzle for LDS rows of R chunks (R = 8 or 16).
template <int R>
__device__ __forceinline__ int swz(int row) {
  if constexpr (R == 16) {
    return (row & 3) | ((row >> 1) & 4) | ((row << 1) & 8);
  } else {
    return ((row >> 1) & 1) | ((row >> 2) & 2) | (((row ^ (row >> 2)) & 1) << 2);
  }
}

// max / sum of the two 32-lane halves (lane l and l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Page-table entry through the scalar cache: the table is read-only for the
// whole launch and the index is uniform, so the physical page (and every
// tile base address derived from it) lives in scalar registers.
__device__ __forceinline__ int64_t page_of(const int32_t* pt, int64_t lp) {
  return ((const __attribute__((address_space(4))) int32_t*)(const void*)pt)[lp];
}

// fp8 E4M3FN -> bf16 bits for 4 codes packed in a u32.  Exact (3 mantissa
// bits fit in bf16's 7; the E4M3 exponent range fits bf16's).
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  uint32_t a = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
  uint32_t b = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
  return make_uint2(a, b);
}

// Workgroup barrier that waits only for this wave's LDS traffic, not for
// global loads still in flight (they land in registers and are waited for
// at their use).  The asm clobber keeps the compiler from moving memory
// accesses across it.
// The scheduling barriers keep register-only work (e.g. a softmax whose
// inputs are already in registers) on its side of the barrier, which is
// what makes two wave groups alternate between matrix and vector work.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unchanged
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace attn
}  // namespace bca
