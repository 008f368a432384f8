// Quantization kernels for gfx950: K-smoothing mean, per-block Q/K codes,
// per-channel E4M3 V codes ("TRTLLM Attention", section "SAGE quantization";
// "VisualGen Quantized Attention", section "SageAttention in the TRTLLM
// backend"), and for the other recipes of that page's section "Recipes"
// MXFP8 Q/K codes with E8M0 block scales and a tensor-wide V scale.  All of
// these are HBM-bound streaming kernels.
//
// Pipeline (one stream, three launches; QK16PV8 quantizes V only):
//   1. kv_stats:  per (b, kv head, 256-token chunk, channel) the binary32 sum of
//                 K over the chunk in ascending token order, and max |V| per
//                 (b, kv head, channel) via an integer atomic max on the float
//                 bits (exact and order-free).
//   2. kv_finish: mu = (sum of the chunk sums in ascending chunk order) / S_kv
//                 and the V scale max|V| / 448 (1 when the channel is all zero).
//   3. quantize:  Q and K_hat = K - mu per token block (absmax reduced across
//                 lanes), or Q and K in MXFP8 (32-channel blocks), and V
//                 written transposed (d-major), the layout the attention
//                 kernel reads as the BMM2 A operand.
// Without K-smoothing (MXFP8, QK16PV8) mu is 0 and K is not summed; with a
// tensor-wide V scale one more launch reduces the channel maxima.
// Divisions are correctly rounded binary32 (the default HIP division); the
// E4M3 conversion is the hardware v_cvt_pk_fp8_f32 (OCP E4M3, round to
// nearest even, subnormals kept) applied after clamping to +-448, which makes
// it saturating.
#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr int kChunksPerWG = 16;
constexpr float kE4M3Max = 448.0f;
constexpr float kInt8Max = 127.0f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ void unpack8(const uint4 u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
    x[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
  }
}

// Two E4M3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t int8_code(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -kInt8Max), kInt8Max);
  return (uint32_t)((int)r) & 0xFFu;
}

// Thread (chunk c = blockIdx.x * 16 + tid / 16, channels 8 * (tid % 16) + 0..7).
__global__ __launch_bounds__(256) void kv_stats_kernel(SageQuantArgs a) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int c = blockIdx.x * kChunksPerWG + (tid >> 4);
  const int d0 = 8 * (tid & 15);
  const int nchunks = (a.Skv + kMeanChunk - 1) / kMeanChunk;
  if (c >= nchunks) return;
  const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.ks[0] + g * a.ks[2] + d0;
  const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.vs[0] + g * a.vs[2] + d0;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float vmax[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int s_end = min(a.Skv, (c + 1) * kMeanChunk);
  const bool smooth = a.smooth != 0;
  // Unrolled so that several rows' loads are in flight at once; the sums still
  // run in token order.
#pragma unroll 8
  for (int s = c * kMeanChunk; s < s_end; ++s) {
    float kx[8], vx[8];
    if (smooth) unpack8(ldg16(kp + (int64_t)s * a.ks[1]), kx);
    unpack8(ldg16(vp + (int64_t)s * a.vs[1]), vx);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (smooth) acc[j] = acc[j] + kx[j];
      vmax[j] = fmaxf(vmax[j], fabsf(vx[j]));
    }
  }
  float* part = a.k_partial + (((int64_t)b * a.Hkv + g) * nchunks + c) * kHeadDim + d0;
  unsigned* vm = a.v_absmax + ((int64_t)b * a.Hkv + g) * kHeadDim + d0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    part[j] = acc[j];
    atomicMax(vm + j, __float_as_uint(vmax[j]));
  }
}

__global__ void zero_absmax_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// One thread per (b, kv head, channel).
__global__ __launch_bounds__(128) void kv_finish_kernel(SageQuantArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int nchunks = (a.Skv + kMeanChunk - 1) / kMeanChunk;
  const float* part = a.k_partial + ((int64_t)b * a.Hkv + g) * nchunks * kHeadDim + d;
  float tot = 0.0f;
#pragma unroll 8   // loads run ahead; the sum keeps chunk order
  for (int c = 0; c < nchunks; ++c) tot = tot + part[(int64_t)c * kHeadDim];
  const int64_t idx = ((int64_t)b * a.Hkv + g) * kHeadDim + d;
  a.k_mean[idx] = a.smooth ? tot / (float)a.Skv : 0.0f;
  const float vmax = __uint_as_float(a.v_absmax[idx]);
  a.v_scale[idx] = vmax == 0.0f ? 1.0f : vmax / kE4M3Max;
}

// Tensor-wide V scale: max over every channel maximum (one workgroup), then
// the same scale max / 448 in every v_scale entry.
__global__ __launch_bounds__(1024) void v_tensor_scale_kernel(SageQuantArgs a) {
  __shared__ unsigned red[1024];
  const int n = a.B * a.Hkv * kHeadDim;
  unsigned m = 0u;
  for (int i = threadIdx.x; i < n; i += 1024) m = max(m, a.v_absmax[i]);   // non-negative floats order as integers
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float vmax = __uint_as_float(red[0]);
  const float scale = vmax == 0.0f ? 1.0f : vmax / kE4M3Max;
  for (int i = threadIdx.x; i < n; i += 1024) a.v_scale[i] = scale;
}

// MXFP8 Q/K: OCP MX with E4M3 elements, one E8M0 scale per 32 channels of a
// token.  Thread (row 16 wave-groups..): 16 lanes per token row, 8 channels
// per lane, 4 lanes per 32-channel block.  X = 2^e with e = floor(log2 amax)
// - 8 (8: exponent of E4M3's largest binade), clamped to [-127, 127]
// (-127 for an all-zero block); code = E4M3(x / X) saturated at 448.  The
// E8M0 byte is e + 127.  Rows past S (up to s_pad) get zero codes and byte 0.
__global__ __launch_bounds__(256) void mx_quant_kernel(SageQuantArgs a) {
  const int head = blockIdx.y, b = blockIdx.z;
  const bool is_q = head < a.Hq;
  const int hh = is_q ? head : head - a.Hq;
  const int S = is_q ? a.Sq : a.Skv;
  const int64_t* st = is_q ? a.qs : a.ks;
  const bf16_t* src = static_cast<const bf16_t*>(is_q ? a.q : a.k) + b * st[0] + hh * st[2];
  const int H = is_q ? a.Hq : a.Hkv;
  uint8_t* codes = (is_q ? a.q_codes : a.k_codes) + ((int64_t)b * H + hh) * a.s_pad * kHeadDim;
  uint8_t* mx = (is_q ? a.q_mx : a.k_mx) + ((int64_t)b * H + hh) * a.s_pad * 4;
  const int s = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (s >= a.s_pad) return;
  const int d0 = 8 * (threadIdx.x & 15);
  float x[8];
  if (s < S) {
    unpack8(ldg16(src + (int64_t)s * st[1] + d0), x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.0f;
  }
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
  am = fmaxf(am, __shfl_xor(am, 1, 64));
  am = fmaxf(am, __shfl_xor(am, 2, 64));
  // floor(log2 am) from the binary32 exponent field (a subnormal am is below
  // 2^-126, where the clamp to -127 applies anyway).
  const int ebits = (int)((__float_as_uint(am) >> 23) & 0xFF);
  int e = ebits - 127 - 8;
  e = am == 0.0f ? -127 : (e < -127 ? -127 : (e > 127 ? 127 : e));
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact (e <= 126 here)
  uint32_t w0, w1;
  w0 = e4m3_pair(x[0] * inv, x[1] * inv) | e4m3_pair(x[2] * inv, x[3] * inv) << 16;
  w1 = e4m3_pair(x[4] * inv, x[5] * inv) | e4m3_pair(x[6] * inv, x[7] * inv) << 16;
  *reinterpret_cast<uint2*>(codes + (int64_t)s * kHeadDim + d0) = make_uint2(w0, w1);
  if ((threadIdx.x & 3) == 0) mx[(int64_t)s * 4 + ((threadIdx.x & 15) >> 2)] = (uint8_t)(e + 127);
}

// Q / K_hat block quantization.  One wavefront per 16-token group of one
// head: lane l covers tokens 4*i + l/16 (i = 0..3) of the group and channels
// 8*(l%16) + 0..7.  A block of 1 token is 16 lanes, of 4 tokens one i over
// the whole wavefront, of 16 tokens the whole group.
template <bool kInt8>
__global__ __launch_bounds__(256) void qk_quant_kernel(SageQuantArgs a) {
  const int head = blockIdx.y, b = blockIdx.z;
  const bool is_q = head < a.Hq;
  const int hh = is_q ? head : head - a.Hq;
  const int S = is_q ? a.Sq : a.Skv;
  const int blk = is_q ? a.q_block : a.k_block;
  const int64_t* st = is_q ? a.qs : a.ks;
  const bf16_t* src = static_cast<const bf16_t*>(is_q ? a.q : a.k) + b * st[0] + hh * st[2];
  const int H = is_q ? a.Hq : a.Hkv;
  uint8_t* codes = (is_q ? a.q_codes : a.k_codes) + ((int64_t)b * H + hh) * a.s_pad * kHeadDim;
  float* scales = (is_q ? a.q_scale : a.k_scale) + ((int64_t)b * H + hh) * (is_q ? a.n_qblk : a.n_kblk);
  const int64_t nblk = is_q ? a.n_qblk : a.n_kblk;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s0 = (blockIdx.x * 4 + wave) * 16;  // first token of this wave's group
  if (s0 >= a.s_pad) return;
  const int d0 = 8 * (lane & 15);
  float mu[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (!is_q) {
    const float* m = a.k_mean + ((int64_t)b * a.Hkv + hh) * kHeadDim + d0;
#pragma unroll
    for (int j = 0; j < 8; ++j) mu[j] = m[j];
  }

  float x[4][8];
  float am[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = s0 + 4 * i + (lane >> 4);
    if (s < S) {
      unpack8(ldg16(src + (int64_t)s * st[1] + d0), x[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!is_q && s < S) x[i][j] = x[i][j] - mu[j];   // K_hat = K - mu, binary32
      m = fmaxf(m, fabsf(x[i][j]));
    }
    am[i] = m;
  }
  // Reduce |x| maxima over the lanes (and token rows) of each block.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) am[i] = fmaxf(am[i], __shfl_xor(am[i], off, 64));
  }
  if (blk >= 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      am[i] = fmaxf(am[i], __shfl_xor(am[i], 16, 64));
      am[i] = fmaxf(am[i], __shfl_xor(am[i], 32, 64));
    }
  }
  if (blk == 16) {
    const float m = fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) am[i] = m;
  }
  const float qmax = kInt8 ? kInt8Max : kE4M3Max;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = s0 + 4 * i + (lane >> 4);
    const float scale = am[i] == 0.0f ? 1.0f : am[i] / qmax;
    uint32_t w0 = 0, w1 = 0;
    if (s < S) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = x[i][j] / scale;
      if constexpr (kInt8) {
        w0 = int8_code(y[0]) | int8_code(y[1]) << 8 | int8_code(y[2]) << 16 | int8_code(y[3]) << 24;
        w1 = int8_code(y[4]) | int8_code(y[5]) << 8 | int8_code(y[6]) << 16 | int8_code(y[7]) << 24;
      } else {
        w0 = e4m3_pair(y[0], y[1]) | e4m3_pair(y[2], y[3]) << 16;
        w1 = e4m3_pair(y[4], y[5]) | e4m3_pair(y[6], y[7]) << 16;
      }
      // one lane per block writes its scale
      const int sb = s / blk;
      const bool writer = (lane & 15) == 0 && (s % blk == 0) && sb < nblk;
      if (writer) scales[sb] = scale;
    }
    *reinterpret_cast<uint2*>(codes + (int64_t)s * kHeadDim + d0) = make_uint2(w0, w1);
  }
}

// V codes, transposed.  Workgroup = 128 tokens x 128 channels of one
// (b, kv head).  Thread t covers channels 8 (t % 16) + 0..7 of tokens
// 4 (t / 16) + 0..3 (plus 64 in the second pass): 16-byte reads of V rows,
// and per channel the codes of its four tokens form one 32-bit word of the
// [channel][token] LDS tile.  The tile leaves as 128-byte rows (whole cache
// lines) of v_codes[b, g, d, :].  Tokens at or past S_kv get zero codes.
constexpr int kVqTokens = 128;
constexpr int kVqPitch = kVqTokens + 16;   // bytes per LDS row (16-byte aligned rows)

__global__ __launch_bounds__(256) void v_quant_kernel(SageQuantArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kHeadDim * kVqPitch];
  const int g = blockIdx.y, b = blockIdx.z;
  const int s0 = blockIdx.x * kVqTokens;
  const int tid = threadIdx.x;
  const int cg = tid & 15, tg = tid >> 4;
  const int d0 = 8 * cg;
  const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.vs[0] + g * a.vs[2] + d0;
  const float* sv = a.v_scale + ((int64_t)b * a.Hkv + g) * kHeadDim + d0;
  float scale[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) scale[j] = sv[j];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int t0 = 64 * pass + 4 * tg;   // first of this thread's four tokens within the tile
    float x[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + t0 + i;
      if (s < a.Skv) {
        unpack8(ldg16(vp + (int64_t)s * a.vs[1]), x[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = e4m3_pair(x[0][j] / scale[j], x[1][j] / scale[j]);
      const uint32_t hi = e4m3_pair(x[2][j] / scale[j], x[3][j] / scale[j]);
      *reinterpret_cast<uint32_t*>(&tile[(d0 + j) * kVqPitch + t0]) = lo | hi << 16;
    }
  }
  __syncthreads();
  uint8_t* out = a.v_codes + ((int64_t)b * a.Hkv + g) * kHeadDim * a.s_pad + s0;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int idx = pass * 256 + tid;   // 1024 chunks of 16 bytes: channel idx / 8, part idx % 8
    const int d = idx >> 3, part = idx & 7;
    if (s0 + 16 * part < a.s_pad) {     // s_pad is a multiple of 64: the last tile may be half
      const uint4 w = *reinterpret_cast<const uint4*>(&tile[d * kVqPitch + 16 * part]);
      *reinterpret_cast<uint4*>(out + (int64_t)d * a.s_pad + 16 * part) = w;
    }
  }
}

}  // namespace

hipError_t launch_sage_quantize(const SageQuantArgs& a, hipStream_t stream) {
  const int nabs = a.B * a.Hkv * kHeadDim;
  hipLaunchKernelGGL(zero_absmax_kernel, dim3((nabs + 255) / 256), dim3(256), 0, stream, a.v_absmax, nabs);
  if (a.Skv > 0) {
    const int nchunks = (a.Skv + kMeanChunk - 1) / kMeanChunk;
    hipLaunchKernelGGL(kv_stats_kernel, dim3((nchunks + kChunksPerWG - 1) / kChunksPerWG, a.Hkv, a.B), dim3(256), 0,
                       stream, a);
  }
  hipLaunchKernelGGL(kv_finish_kernel, dim3(a.Hkv, a.B), dim3(128), 0, stream, a);
  if (a.v_tensor) hipLaunchKernelGGL(v_tensor_scale_kernel, dim3(1), dim3(1024), 0, stream, a);
  const unsigned groups = (unsigned)((a.s_pad / 16 + 3) / 4);
  if (a.qk_fmt == kQkInt8)
    hipLaunchKernelGGL(qk_quant_kernel<true>, dim3(groups, a.Hq + a.Hkv, a.B), dim3(256), 0, stream, a);
  else if (a.qk_fmt == kQkFp8)
    hipLaunchKernelGGL(qk_quant_kernel<false>, dim3(groups, a.Hq + a.Hkv, a.B), dim3(256), 0, stream, a);
  else if (a.qk_fmt == kQkMxfp8)
    hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)(a.s_pad / 16), a.Hq + a.Hkv, a.B), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(v_quant_kernel, dim3((unsigned)((a.s_pad + kVqTokens - 1) / kVqTokens), a.Hkv, a.B), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace ditattn
