// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // raw bfloat16 storage

#define DITATTN_LDS __attribute__((address_space(3)))

// Workgroup id -> logical tile id so that each XCD (hardware hands workgroup
// i to XCD i % 8) receives one contiguous range of logical ids.  Consecutive
// logical ids share a head, so the 32 CUs of an XCD stream the same K/V
// through their common L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int per = nwg >> 3, rem = nwg & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// v_permlane32_swap exchanges lanes 32-63 of one register with lanes 0-31 of
// another.  With both operands equal to x, the first result holds x[l % 32]
// and the second x[32 + l % 32] in every lane l, so combining them reduces
// over the two wave halves (lanes l and l ^ 32).
__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier without a memory fence (the caller waits for its own
// memory counters first); the empty asm statements keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace ditattn
