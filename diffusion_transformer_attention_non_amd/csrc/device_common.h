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

// Raw buffer resource (stride 0) over [base, base + num_records): loads at
// offsets past num_records return zero.  Every field is made wave-uniform so
// the descriptor lives in scalar registers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = 0x00020000;   // 32-bit data format, no swizzle
  return r;
}

// buffer_load_dwordx4 ... lds: lane l reads 16 bytes at voffset and the wave
// writes them to LDS bytes [lds_addr + 16 l, lds_addr + 16 l + 16).  Issued
// as inline assembly, so the compiler tracks no LDS dependency for it and
// inserts no wait of its own; the caller orders it against LDS reads with an
// explicit s_waitcnt vmcnt and a barrier.  lds_addr must be wave-uniform.
// (m0 is a reserved register: the compiler sets it before each of its own
// uses, so clobbering it here is safe; the warning about that is silenced.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t lds_addr, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

// As buffer_load_lds16 with the LDS address given as base + offset, added in
// the instruction stream: only the base needs to stay in a register across a
// loop, the offset (a constant at the call site) is rematerialized.
__device__ __forceinline__ void buffer_load_lds16_at(i32x4 rsrc, uint32_t lds_base, uint32_t lds_off,
                                                     uint32_t voffset) {
  asm volatile(
      "s_add_u32 m0, %0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds"
      :
      : "s"(lds_base), "s"(lds_off), "v"(voffset), "s"(rsrc)
      : "memory", "m0", "scc");
}

// As buffer_load_lds16 with 4 bytes per lane: LDS bytes [lds_addr + 4 l, lds_addr + 4 l + 4).
__device__ __forceinline__ void buffer_load_lds4(i32x4 rsrc, uint32_t lds_addr, uint32_t voffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((DITATTN_LDS T*)p);
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// v_permlane32_swap exchanges lanes 32-63 of one register with lanes 0-31 of
// another.  With both operands equal to x, the first result holds x[l % 32]
// and the second x[32 + l % 32] in every lane l, so combining them reduces
// over the two wave halves (lanes l and l ^ 32).
// Maxima as single v_max / v_max3 instructions.  fmaxf would first quiet
// signalling NaNs (an extra canonicalizing v_max per operand that is not
// known to be canonical); no NaN reaches these maxima.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
