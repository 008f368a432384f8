// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

// Tile geometry shared by the attention kernels and the host layer.
constexpr int kHeadDim = 128;
constexpr int kWaveRows = 32;    // query rows per wavefront in the low-precision (SAGE) kernel,
                                  // its Skip-Softmax vote rows (its workgroup: 12 wavefronts, 384 rows)
constexpr int kBlockM = 256;      // query rows per workgroup of the BF16 kernels (4 wavefronts x 64),
                                  // the most workgroups any attention launch uses per head
constexpr int kBlockN = 64;       // keys per KV tile (LDS stage)
constexpr int kSkipBlockM = 64;   // BF16 kernels: query rows per wavefront = rows per Skip-Softmax vote
constexpr int kSkipBlockN = 32;   // keys per BF16 Skip-Softmax vote (half a KV tile)
constexpr int kMeanChunk = 256;   // tokens per partial sum of the K mean

struct FmhaBf16Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides (b, s, h)
  int B, Sq, Skv, Hq, Hkv;
  float sm_scale;
  int o_fp32;
  float log2_lambda;                // skip threshold in log2 units (skip kernel only)
  uint8_t* bitmap;                  // nullable
  unsigned long long* counter;      // nullable
  float* lse;                       // nullable, [B, Hq, Sq] natural-log row log-sum-exp
};

hipError_t launch_fmha_bf16(const FmhaBf16Args& a, hipStream_t stream);        // dense
hipError_t launch_fmha_bf16_skip(const FmhaBf16Args& a, hipStream_t stream);   // Skip-Softmax
hipError_t launch_zero_u64(unsigned long long* p, hipStream_t stream);
hipError_t launch_fill_u8(uint8_t* p, size_t n, uint8_t value, hipStream_t stream);

// Q/K formats of the low-precision attention path.
constexpr int kQkInt8 = 0, kQkFp8 = 1, kQkMxfp8 = 2, kQkBf16 = 3;

struct SageQuantArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs[3], ks[3], vs[3];
  int B, Sq, Skv, Hq, Hkv;
  int qk_fmt;           // kQk*
  int smooth;           // 1 = K-smoothing (SageAttention recipes)
  int v_tensor;         // 1 = one tensor-wide V scale, 0 = one per (b, kv head, channel)
  int q_block, k_block;
  int64_t s_pad, n_qblk, n_kblk;
  uint8_t* q_codes;     // [B, Hq, s_pad, 128]
  uint8_t* k_codes;     // [B, Hkv, s_pad, 128]
  uint8_t* v_codes;     // [B, Hkv, 128, s_pad]
  float* q_scale;       // [B, Hq, n_qblk]
  float* k_scale;       // [B, Hkv, n_kblk]
  float* v_scale;       // [B, Hkv, 128]
  float* k_mean;        // [B, Hkv, 128]
  float* k_partial;     // [B, Hkv, n_chunks, 128]
  unsigned* v_absmax;   // [B, Hkv, 128] float bits
  uint8_t* q_mx;        // MXFP8: [B, Hq, s_pad, 4] E8M0 bytes (aliases q_scale's region)
  uint8_t* k_mx;        // MXFP8: [B, Hkv, s_pad, 4]
};

hipError_t launch_sage_quantize(const SageQuantArgs& a, hipStream_t stream);

struct FmhaSageArgs {
  const uint8_t* q_codes;
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* q_mx;    // MXFP8 E8M0 bytes [B, Hq, s_pad, 4]
  const uint8_t* k_mx;    // [B, Hkv, s_pad, 4]
  const void* q;          // BF16 Q and K (QK16PV8), element strides (b, s, h)
  const void* k;
  int64_t qs[3], ks[3];
  int qk_fmt;             // kQk*
  void* o;
  int64_t os[3];
  int B, Sq, Skv, Hq, Hkv;
  int64_t s_pad, n_qblk, n_kblk;
  int q_block, k_block;
  float sm_scale;
  int o_fp32;
  int skip;                         // 1 = Skip-Softmax tile test on (32 rows x one KV tile)
  float log2_lambda;                // skip threshold in log2 units
  uint8_t* bitmap;                  // nullable, [B, Hq, ceil(Sq / 32), ceil(Skv / 64)]
  unsigned long long* counter;      // nullable
};

hipError_t launch_fmha_sage(const FmhaSageArgs& a, hipStream_t stream);

}  // namespace ditattn
