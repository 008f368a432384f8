// Instruction-issue probes for gfx950: how fast a SIMD issues the VALU
// instructions of the attention softmax, and how VALU work and E4M3 MFMAs
// share a SIMD.  Measurement infrastructure for the benchmark
// (`bench.py --issue-probe`), built into the probe library beside the MFMA
// peak probe, not part of the attention library's interface.
//
// Every kernel runs one workgroup per CU with 4 * wps wavefronts (wps per
// SIMD); each wavefront records the span of its timed loop in shader cycles
// (clock64), which the caller turns into SIMD cycles per unit of work.
// Results are summed into one value per lane and written, so nothing is dead
// code; the values themselves are meaningless.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;   // independent dependency chains per lane

// ---- VALU issue rate: 4 x kChains instructions of one kind per iteration.
//   op 0 v_add_f32, 1 v_fma_f32, 2 v_max3_f32, 3 v_exp_f32,
//   4 v_cvt_pk_fp8_f32, 5 v_pk_fma_f16 (two f16 lanes per register).
template <int kOp>
__device__ __forceinline__ void valu_step(float (&x)[kChains]) {
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    if constexpr (kOp == 0) asm volatile("v_add_f32 %0, 1.0, %0" : "+v"(x[c]));
    else if constexpr (kOp == 1) asm volatile("v_fma_f32 %0, %0, %0, 1.0" : "+v"(x[c]));
    else if constexpr (kOp == 2) asm volatile("v_max3_f32 %0, %0, 1.0, %0" : "+v"(x[c]));
    else if constexpr (kOp == 3) asm volatile("v_exp_f32 %0, %0" : "+v"(x[c]));
    else if constexpr (kOp == 4) asm volatile("v_cvt_pk_fp8_f32 %0, %0, %0" : "+v"(x[c]));
    else asm volatile("v_pk_fma_f16 %0, %0, %0, %0" : "+v"(x[c]));
  }
}

template <int kOp>
__global__ __launch_bounds__(768) void valu_issue_kernel(int iters, unsigned long long* cycles, float* sink) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = 1e-3f * (float)(threadIdx.x + c);
  const unsigned long long c0 = clock64();
  for (int it = 0; it < iters; ++it) {
    valu_step<kOp>(x);
    valu_step<kOp>(x);
    valu_step<kOp>(x);
    valu_step<kOp>(x);
  }
  const unsigned long long c1 = clock64();
  float t = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) t += x[c];
  const int wave = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  sink[(size_t)wave * 64 + (threadIdx.x & 63)] = t;
  if ((threadIdx.x & 63) == 0) cycles[wave] = c1 - c0;
}

// ---- E4M3 MFMAs and VALU work on one SIMD.  One step of a wavefront is one
// v_mfma_scale_f32_32x32x64_f8f6f4 (64 cycles at the full rate) and/or its
// VALU share:
//   mode 0: MFMAs only (four independent accumulators);
//   mode 1: split: the first 4 * (wps / 2) wavefronts run MFMAs, the others
//           16 v_fma_f32 per step;
//   mode 2: 16 v_fma_f32 issued right after each MFMA of the same wavefront;
//   mode 3: softmax mix after each MFMA: four logits through fma -> exp2,
//           their sum, two maxima and two E4M3 packs, as the low-precision
//           attention kernel issues them per MFMA;
//   mode 4: the same mix issued as a burst of four groups after four MFMAs.
struct Mix {
  float s[16];
  float mx, sum, f, nb;
  int pk[4];
};

__device__ __forceinline__ void mix_group(Mix& m, int g) {
  const int base = (4 * g) & 15;
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(m.s[base + j], m.f, m.nb));
  m.mx = fmaxf(fmaxf(m.mx, m.s[base]), m.s[base + 1]);
  m.mx = fmaxf(fmaxf(m.mx, m.s[base + 2]), m.s[base + 3]);
  m.sum += (x[0] + x[1]) + (x[2] + x[3]);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], m.pk[g & 3], false);
  m.pk[g & 3] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w, true);
#pragma unroll
  for (int j = 0; j < 4; ++j) m.s[base + j] += 1e-7f * x[j];   // the next group depends on this one
}

template <int kMode>
__global__ __launch_bounds__(768) void coexec_kernel(int iters, unsigned long long* cycles, float* sink) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wps = (int)(blockDim.x >> 8);
  i32x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // E4M3 bytes in [0x30, 0x3f]: finite, no overflow
    a[i] = (int)(0x30313233u + 0x01010101u * (unsigned)((lane + i) & 7));
    b[i] = (int)(0x38393a3bu + 0x01010101u * (unsigned)(i & 3));
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  float y[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) y[c] = 1e-3f * (float)(lane + c);
  Mix m;
#pragma unroll
  for (int i = 0; i < 16; ++i) m.s[i] = -0.01f * (float)(i + lane);
  m.mx = -1e30f;
  m.sum = 0.0f;
  m.f = 0.37f + 1e-4f * (float)lane;
  m.nb = -3.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) m.pk[i] = 0;
  const bool mfma_wave = kMode != 1 || wid < 4 * (wps / 2);
  const bool fma_wave = kMode == 2 || (kMode == 1 && !mfma_wave);
  __syncthreads();
  const unsigned long long c0 = clock64();
  for (int it = 0; it < iters; ++it) {
    if constexpr (kMode == 4) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) mix_group(m, g);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (mfma_wave) acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
        if (fma_wave) {
#pragma unroll
          for (int j = 0; j < 16; ++j) asm volatile("v_fma_f32 %0, %0, %0, 1.0" : "+v"(y[j & (kChains - 1)]));
        }
        if constexpr (kMode == 3) mix_group(m, c);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  const unsigned long long c1 = clock64();
  float t = m.mx + m.sum + (float)(m.pk[0] + m.pk[1] + m.pk[2] + m.pk[3]);
#pragma unroll
  for (int c = 0; c < kChains; ++c) t += y[c];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[c][r];
  const int wave = blockIdx.x * (blockDim.x / 64) + wid;
  sink[(size_t)wave * 64 + lane] = t;
  if (lane == 0) cycles[wave] = c1 - c0;
}

}  // namespace

extern "C" {

// Number of VALU kinds and co-execution modes the probes know.
int issue_probe_valu_kinds(void) { return 6; }
int issue_probe_coexec_modes(void) { return 5; }

// Instructions (VALU probe) or MFMAs (co-execution probe) one wavefront
// issues per iteration of its timed loop.
int issue_probe_per_iter(int probe) { return probe == 0 ? 4 * kChains : 4; }

// Launch a probe on `stream`: probe 0 = VALU issue rate of `kind` (0..5),
// probe 1 = co-execution mode `kind` (0..4); `workgroups` workgroups of
// 4 * wps wavefronts (wps = 1..3 per SIMD; the split mode needs wps = 2).
// cycles: device, one uint64 per wavefront; sink: device, 64 floats per
// wavefront.  Returns 0, or -1 for a bad argument, -8 for a launch failure.
int issue_probe_launch(int probe, int kind, int wps, int workgroups, int iters, unsigned long long* cycles, float* sink,
                       void* stream) {
  if (probe < 0 || probe > 1 || wps < 1 || wps > 3 || workgroups <= 0 || iters <= 0 || cycles == nullptr ||
      sink == nullptr)
    return -1;
  if ((probe == 0 && (kind < 0 || kind > 5)) || (probe == 1 && (kind < 0 || kind > 4)) ||
      (probe == 1 && kind == 1 && wps != 2))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)workgroups), block((unsigned)(256 * wps));
  if (probe == 0) {
    switch (kind) {
      case 0: hipLaunchKernelGGL(valu_issue_kernel<0>, grid, block, 0, st, iters, cycles, sink); break;
      case 1: hipLaunchKernelGGL(valu_issue_kernel<1>, grid, block, 0, st, iters, cycles, sink); break;
      case 2: hipLaunchKernelGGL(valu_issue_kernel<2>, grid, block, 0, st, iters, cycles, sink); break;
      case 3: hipLaunchKernelGGL(valu_issue_kernel<3>, grid, block, 0, st, iters, cycles, sink); break;
      case 4: hipLaunchKernelGGL(valu_issue_kernel<4>, grid, block, 0, st, iters, cycles, sink); break;
      default: hipLaunchKernelGGL(valu_issue_kernel<5>, grid, block, 0, st, iters, cycles, sink); break;
    }
  } else {
    switch (kind) {
      case 0: hipLaunchKernelGGL(coexec_kernel<0>, grid, block, 0, st, iters, cycles, sink); break;
      case 1: hipLaunchKernelGGL(coexec_kernel<1>, grid, block, 0, st, iters, cycles, sink); break;
      case 2: hipLaunchKernelGGL(coexec_kernel<2>, grid, block, 0, st, iters, cycles, sink); break;
      case 3: hipLaunchKernelGGL(coexec_kernel<3>, grid, block, 0, st, iters, cycles, sink); break;
      default: hipLaunchKernelGGL(coexec_kernel<4>, grid, block, 0, st, iters, cycles, sink); break;
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
