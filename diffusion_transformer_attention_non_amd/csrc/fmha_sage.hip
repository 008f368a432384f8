// SAGE attention on quantized codes for gfx950 ("TRTLLM Attention", section
// "SAGE quantization": both attention matmuls in low precision; "VisualGen
// Quantized Attention", section "SageAttention in the TRTLLM backend").
//
// Same decomposition as the BF16 kernel (workgroup = 4 wavefronts x 64 query
// rows, KV tiles of 64 keys, transposed products so that each query stays in
// one lane), with:
//   BMM1  S^T = Kc Qc^T on int8 (v_mfma_i32_32x32x32_i8, exact int32) or
//         OCP E4M3 (v_mfma_f32_32x32x64_f8f6f4) codes; the logit is
//         s_ij = acc_ij * sq_i * sk_j * sm_scale (bmm1 scale);
//   softmax exact per tile: m' = max(m, tile max), alpha = 2^(m - m'),
//         e = 2^(s - m' + 8) = 2^8 p, l = alpha * l + sum e (unrounded);
//   BMM2  O^T += Vc^T E4M3(e)^T on E4M3 codes (v_mfma_f32_32x32x64_f8f6f4),
//         V^T codes read as written by the quantizer (d-major);
//   epilogue O = acc * sv_d / l (bmm2 scale), l holding the 2^8 factor.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// LDS stage (bytes): K codes 64 rows x 128 (+16 pad) in MFMA-row order,
// V^T codes 128 rows x 64 (+16 pad), the tile's 64 K scales.
constexpr int kKRowB = 144;
constexpr int kVRowB = 80;
constexpr int kKTileB = kBlockN * kKRowB;     // 9216
constexpr int kVTileB = kHeadDim * kVRowB;    // 10240
constexpr int kScaleB = kBlockN * 4;
constexpr int kStageB = kKTileB + kVTileB + kScaleB;

// The E4M3 BMM2 takes 64 keys per MFMA, 32 consecutive k per lane half.
// Register r of lane half h in S^T block kb must therefore hold key
// 32*h + 16*kb + r.  Accumulator register r of lane half h is MFMA row
// 8*(r/4) + 4*h + r%4, so block kb's MFMA row 8a + 4h + b reads key
// 32*h + 16*kb + 4a + b.  This maps a key (0..63) to its LDS row.
__device__ __forceinline__ int sage_row_of_key(int k) {
  const int h = k >> 5, kb = (k >> 4) & 1, a = (k >> 2) & 3, b = k & 3;
  return 32 * kb + 8 * a + 4 * h + b;
}

template <bool kInt8>
__global__ __launch_bounds__(256, 1) void fmha_sage_kernel(FmhaSageArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageB];

  const int nqt = (p.Sq + kBlockM - 1) / kBlockM;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % nqt;
  const int bh = wg / nqt;
  const int h = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * kBlockM + wave * kWaveRows;
  const int Sq = p.Sq, Skv = p.Skv;
  const int64_t s_pad = p.s_pad;

  // Q codes, B operand of BMM1.  int8: 4 k-steps of 32 channels, lane half h
  // holds 16 channels; E4M3: 2 k-steps of 64, lane half holds 32.
  constexpr int kQSteps = kInt8 ? 4 : 2;
  constexpr int kQBytes = kInt8 ? 16 : 32;
  typedef typename std::conditional<kInt8, i32x4, i32x8>::type qfrag_t;
  qfrag_t qf[2][kQSteps];
  float qsc[2];
  const float c = p.sm_scale * kLog2e;
  const uint8_t* qbase = p.q_codes + ((int64_t)b * p.Hq + h) * s_pad * kHeadDim;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 32 + l32;   // rows < s_pad hold codes (zero past S_q)
    const bool inb = row < s_pad;
    const uint8_t* qp = qbase + (int64_t)(inb ? row : 0) * kHeadDim + kQBytes * hh;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      if constexpr (kInt8) {
        qf[qb][ks] = __builtin_bit_cast(qfrag_t, inb ? ldg16(qp + 32 * ks) : z);
      } else {
        const uint4 lo = inb ? ldg16(qp + 64 * ks) : z, hi = inb ? ldg16(qp + 64 * ks + 16) : z;
        i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        qf[qb][ks] = __builtin_bit_cast(qfrag_t, v);
      }
    }
    const int qrow = row < Sq ? row : Sq - 1;
    qsc[qb] = p.q_scale[((int64_t)b * p.Hq + h) * p.n_qblk + qrow / p.q_block] * c;
  }

  // Loader: K tile = 64 rows x 128 B (two 16-byte chunks per thread),
  // V^T tile = 128 rows x 64 B (two chunks per thread), 64 K scales.
  const uint8_t* kg = p.k_codes + ((int64_t)b * p.Hkv + g) * s_pad * kHeadDim;
  const uint8_t* vg = p.v_codes + ((int64_t)b * p.Hkv + g) * kHeadDim * s_pad;
  const float* skg = p.k_scale + ((int64_t)b * p.Hkv + g) * p.n_kblk;
  int k_src[2], k_dst[2], v_src_row[2], v_src_col[2], v_dst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = i * 256 + tid;
    const int kr = idx >> 3, kc = idx & 7;          // key row, 16-byte chunk
    k_src[i] = kr * kHeadDim + 16 * kc;
    k_dst[i] = sage_row_of_key(kr) * kKRowB + 16 * kc;
    const int vr = idx >> 2, vc = idx & 3;          // channel row, 16-byte chunk
    v_src_row[i] = vr;
    v_src_col[i] = 16 * vc;
    v_dst[i] = kKTileB + vr * kVRowB + 16 * vc;
  }
  uint4 kreg[2], vreg[2];
  float sreg = 0.0f;
  auto gload = [&](int t) {
    const int key0 = t * kBlockN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kreg[i] = ldg16(kg + (int64_t)key0 * kHeadDim + k_src[i]);
      vreg[i] = ldg16(vg + (int64_t)v_src_row[i] * s_pad + key0 + v_src_col[i]);
    }
    if (tid < kBlockN) {
      const int key = key0 + tid;
      sreg = key < Skv ? skg[key / p.k_block] : 0.0f;
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* base = smem + stage * kStageB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(base + k_dst[i]) = kreg[i];
      *reinterpret_cast<uint4*>(base + v_dst[i]) = vreg[i];
    }
    if (tid < kBlockN) reinterpret_cast<float*>(base + kKTileB + kVTileB)[tid] = sreg;
  };

  const int ka_lane = l32 * kKRowB + kQBytes * hh;
  const int va_lane = kKTileB + l32 * kVRowB + 32 * hh;

  f32x16 o[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.0f;
  float m[2] = {kNegInf, kNegInf};
  float lsum[2] = {0.0f, 0.0f};
  const int nkt = (Skv + kBlockN - 1) / kBlockN;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < nkt; ++t) {
    const uint8_t* st = smem + (t & 1) * kStageB;
    if (t + 1 < nkt) gload(t + 1);

    // ---- BMM1 and dequantization to log2-scaled logits.
    f32x16 s[2][2];
    if constexpr (kInt8) {
      i32x16 acc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[kb][qb][r] = 0;
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const i32x4 a = *reinterpret_cast<const i32x4*>(st + ka_lane + kb * 32 * kKRowB + 32 * ks);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            acc[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, __builtin_bit_cast(i32x4, qf[qb][ks]),
                                                                acc[kb][qb], 0, 0, 0);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] = (float)acc[kb][qb][r];
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint4 lo = *reinterpret_cast<const uint4*>(st + ka_lane + kb * 32 * kKRowB + 64 * ks);
          const uint4 hi = *reinterpret_cast<const uint4*>(st + ka_lane + kb * 32 * kKRowB + 64 * ks + 16);
          const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                a, __builtin_bit_cast(i32x8, qf[qb][ks]), s[kb][qb], 0, 0, 0, 0, 0, 0);
        }
    }
    // Per-key scale: register r of block kb, lane half hh is key 32*hh + 16*kb + r.
    const float* sks = reinterpret_cast<const float*>(st + kKTileB + kVTileB) + 32 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 sk = *reinterpret_cast<const f32x4*>(sks + 16 * kb + 4 * r4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[kb][qb][4 * r4 + j] *= sk[j] * qsc[qb];
      }
    if ((t + 1) * kBlockN > Skv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * kBlockN + 32 * hh + 16 * kb + r;
          if (key >= Skv) {
            s[kb][0][r] = kNegInf;
            s[kb][1][r] = kNegInf;
          }
        }
    }

    // ---- Exact online softmax for the tile.
    float mnew[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mnew[qb] = fmaxf(m[qb], max_halves(mx));
    }
    if (__any(mnew[0] > m[0] || mnew[1] > m[1])) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float alpha = exp2_fast(m[qb] - mnew[qb]);
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
      }
    }
    i32x8 pf[2];   // E4M3(2^8 p): 32 keys of lane half hh, key order 16*kb + r
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      m[qb] = mnew[qb];
      const float nb = 8.0f - mnew[qb];
      float part = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            e[j] = exp2_fast(s[kb][qb][4 * r4 + j] + nb);
            part += e[j];
          }
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
          pf[qb][4 * kb + r4] = w;
        }
      lsum[qb] += part;
    }

    // ---- BMM2: O^T += Vc^T P^T, one 64-key MFMA per (d block, query block).
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const uint4 lo = *reinterpret_cast<const uint4*>(st + va_lane + 32 * db * kVRowB);
      const uint4 hi = *reinterpret_cast<const uint4*>(st + va_lane + 32 * db * kVRowB + 16);
      const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        o[db][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf[qb], o[db][qb], 0, 0, 0, 0, 0, 0);
    }

    if (t + 1 < nkt) lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- Epilogue: O = O^T * sv_d / l.
  const float* svp = p.v_scale + ((int64_t)b * p.Hkv + g) * kHeadDim;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = sum_halves(lsum[qb]);
    const float inv = 1.0f / l;
    const int row = q0 + qb * 32 + l32;
    if (row < Sq) {
      const int64_t obase = b * p.os[0] + (int64_t)row * p.os[1] + h * p.os[2];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * hh;
          const f32x4 sv = *reinterpret_cast<const f32x4*>(svp + d);
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = o[db][qb][4 * gq + j] * sv[j] * inv;
          if (p.o_fp32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + obase + d) = v;
          } else {
            const bf16x4 vb = __builtin_convertvector(v, bf16x4);
            *reinterpret_cast<bf16x4*>(static_cast<bf16_t*>(p.o) + obase + d) = vb;
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_fmha_sage(const FmhaSageArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBlockM - 1) / kBlockM;
  const int64_t nwg = nqt * a.Hq * a.B;
  if (nwg <= 0) return hipSuccess;
  if (a.qk_int8)
    hipLaunchKernelGGL(fmha_sage_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fmha_sage_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ditattn
