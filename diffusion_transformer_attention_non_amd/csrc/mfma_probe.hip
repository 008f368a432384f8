// Matrix-core peak probe for gfx950: back-to-back dense MFMAs of one type on
// every SIMD, timed by the caller with events on the launch stream, plus the
// shader clock the waves ran at (the shader cycle counter against the
// constant-rate wall clock, read by every wave at its start and end).
//
// Measurement infrastructure for the benchmark, not part of the attention
// library's interface: it lives in its own shared object.
//
// Work: each wavefront issues `iters` rounds of four independent MFMAs (four
// accumulator chains, so no MFMA waits on the previous one's result):
//   kind 0: v_mfma_f32_32x32x16_bf16          (32 x 32 x 16 MACs,  32,768 flop)
//   kind 1: v_mfma_f32_32x32x64_f8f6f4, E4M3  (32 x 32 x 64 MACs, 131,072 flop)
//   kind 2: v_mfma_i32_32x32x32_i8            (32 x 32 x 32 MACs,  65,536 op)
// Operands are lane-dependent non-zero bit patterns, so the datapath toggles.
// Each wavefront writes four 64-bit words: clock64 and wall_clock64 at its
// start and end.  The results are summed into one value per lane and written
// too, so the MFMAs are not dead code.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;   // wavefronts per workgroup

template <int kKind>
__global__ __launch_bounds__(kWaves * 64) void mfma_probe_kernel(int iters, unsigned long long* clocks, float* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  float total = 0.0f;
  if constexpr (kKind == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(0.5f + 0.03125f * (float)((lane + i) & 15));
      b[i] = (__bf16)(1.0f - 0.0625f * (float)((lane * 3 + i) & 7));
    }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += acc[c][r];
  } else if constexpr (kKind == 1) {
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {   // E4M3 bytes in [0x30, 0x3f] (0.5 .. 0.94): no overflow
      a[i] = (int)(0x30313233u + 0x01010101u * (unsigned)((lane + i) & 7));
      b[i] = (int)(0x38393a3bu + 0x01010101u * (unsigned)((lane * 5 + i) & 3));
    }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += acc[c][r];
  } else {
    i32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // int8 bytes in [1, 16]: int32 sums stay far from overflow
      a[i] = (int)(0x01020304u + 0x01010101u * (unsigned)((lane + i) & 7));
      b[i] = (int)(0x05060708u + 0x01010101u * (unsigned)((lane * 7 + i) & 7));
    }
    i32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += (float)acc[c][r];
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  sink[(size_t)wave * 64 + lane] = total;
  if (lane == 0) {
    clocks[4 * (size_t)wave + 0] = c0;
    clocks[4 * (size_t)wave + 1] = c1;
    clocks[4 * (size_t)wave + 2] = w0;
    clocks[4 * (size_t)wave + 3] = w1;
  }
}

}  // namespace

extern "C" {

// Flop (or op) count of one MFMA of `kind`, 0 for an unknown kind.
double mfma_probe_flops_per_mfma(int kind) {
  return kind == 0 ? 32768.0 : kind == 1 ? 131072.0 : kind == 2 ? 65536.0 : 0.0;
}

// Frequency of wall_clock64 on the current device, in kHz (0 on error).
int mfma_probe_wall_rate_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

// Launch the probe of `kind` with `workgroups` workgroups of four wavefronts
// on `stream`.  clocks: device, 4 * workgroups * 4 uint64; sink: device,
// workgroups * 4 * 64 floats.  Returns 0, or -1 for a bad argument, -8 for a
// launch failure.
int mfma_probe_launch(int kind, int workgroups, int iters, unsigned long long* clocks, float* sink, void* stream) {
  if (kind < 0 || kind > 2 || workgroups <= 0 || iters <= 0 || clocks == nullptr || sink == nullptr) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)workgroups), block(kWaves * 64);
  if (kind == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, st, iters, clocks, sink);
  else if (kind == 1) hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, st, iters, clocks, sink);
  else hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, st, iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
