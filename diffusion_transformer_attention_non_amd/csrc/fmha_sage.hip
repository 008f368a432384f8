// Low-precision attention for gfx950: SageAttention on quantized codes
// ("TRTLLM Attention", section "SAGE quantization": both attention matmuls in
// low precision; "VisualGen Quantized Attention", section "SageAttention in
// the TRTLLM backend"), and the recipes of the same section "Recipes" that
// share its FP8 BMM2: QK16PV8 (BF16 Q/K, "QK16PV8 Attention Kernels in the
// CUTEDSL Backend") and MXFP8 Q/K ("MXFP8 and NVFP4 in the CUTEDSL and
// FlashInfer backends").
//
// Q/K formats (template kFmt):
//   kFmtI8   int8 codes, one fp32 scale per token block (SageAttention);
//   kFmtF8   OCP E4M3 codes, one fp32 scale per token block (SageAttention);
//   kFmtMX8  OCP MXFP8: E4M3 codes with an E8M0 scale per 32 channels of a
//            token, applied by the MFMA itself (v_mfma_scale A/B scales);
//   kFmtBF16 Q and K read as BF16 from the inputs (QK16PV8).
//
// Work decomposition
//   workgroup = 12 wavefronts = 384 query rows of one (batch, query head),
//   three wavefronts per SIMD (at most 168 VGPRs each); each wavefront owns
//   32 query rows and walks all KV tiles of 64 keys.  While one wavefront of
//   a SIMD issues its MFMAs the other two run softmax VALU work (a single
//   wavefront issues VALU at half rate while its own E4M3 MFMA executes), so
//   the SIMD's scheduler, not a fixed interleave in the code, overlaps the
//   two.  Per tile:
//   BMM1  S^T = Kc Qc^T on int8 (v_mfma_i32_32x32x32_i8, exact int32), OCP
//         E4M3 (v_mfma_scale_f32_32x32x64_f8f6f4, MXFP8 with its block
//         scales) or BF16 (v_mfma_f32_32x32x16_bf16); each lane holds one
//         query (lane % 32) and 32 keys of the tile; the logit in log2 units
//         is L_ij = acc_ij * sk_j * (sq_i * sm_scale * log2 e), sk = sq = 1
//         for MXFP8 and BF16;
//   online softmax against the exact running maximum m of L: m' = max(m,
//         tile max of L); if any row of the wavefront moved, O and the row
//         sums are rescaled by 2^(m - m') (a wavefront-uniform branch, taken
//         on few tiles once the maxima settle); P = E4M3(2^(L - m' + 8));
//         the row sum l adds the unrounded fp32 p = 2^(L - m'), per lane
//         over its 32 keys, the two lane halves combined in the epilogue;
//   BMM2  O^T += Vc^T P^T on E4M3 codes (v_mfma_f32_32x32x64_f8f6f4, V^T
//         codes d-major as the quantizer writes them).
//   Epilogue O = acc * sv_d / (2^8 l) (bmm2 scale).
//
// Skip-Softmax (kSkip; both options in one kernel, "TRTLLM Attention",
// section "Skip-Softmax", and "VisualGen Quantized Attention", section
// "Interaction With Other Features"): after BMM1 of a KV tile the wavefront
// drops the tile (no exponentials, no BMM2, no change of m) when every valid
// row i has 2^(M_it - m_i) < lambda, M_it being the row's largest L in the
// tile and m_i its running maximum over the tiles kept so far (the softmax
// reference itself); lambda = factor / S_kv.  The first tile is kept.
//
// K (codes, or BF16 rows for QK16PV8), V^T codes and the tile's 64 K scale
// words stream into a 4-stage LDS ring with buffer_load ... lds, three tiles
// ahead (out-of-range reads are zero), issued by the first eight wavefronts
// (one load round each); one barrier per tile.  LDS layouts
// (16-byte chunks, XOR-swizzled so that the 16 lanes an LDS cycle serves, 16
// consecutive rows at one logical chunk, hit 16 distinct 16-byte slots of the
// 64 four-byte banks):
//   K codes: 64 rows x 128 B in MFMA-row order, physical chunk = logical ^ ((row >> 1) & 7);
//   K BF16:  64 rows x 256 B in MFMA-row order, physical chunk = logical ^ (row & 15);
//   V^T:     128 rows (channel) x 64 B (keys), physical chunk = logical ^ ((row >> 2) & 3).
//
// E4M3 fragments (kFmtF8, kFmtMX8): the 32x32x64 MFMA reads byte b of lane
// half hh as k = 32 (b / 16) + 16 hh + b % 16, and its E8M0 scale for (row,
// 32-k block g) from lane row + 32 g.  Step ks puts channels 64 ks + 32 g +
// 16 hh + 0..15 into bytes 16 g.. of lane half hh, so hardware k block g is
// exactly MX block 2 ks + g, whose scale the lane of half hh = g supplies.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kSageWaves = 12;                // three wavefronts per SIMD
constexpr int kSageLoaders = 8;               // the first eight issue the tile loads
constexpr int kSageWaveRows = kWaveRows;   // 32 query rows per wavefront
constexpr int kSageBlockM = kSageWaveRows * kSageWaves;   // query rows per workgroup
constexpr int kVTileB = kHeadDim * kBlockN;   // 8 KB of V^T codes
constexpr int kLoadsPerTile = 3;              // per wavefront: K, V and scales (BF16: 2 K, 1 V)

constexpr int kFmtI8 = kQkInt8, kFmtF8 = kQkFp8, kFmtMX8 = kQkMxfp8, kFmtBF16 = kQkBf16;
// LDS stage: [K][V^T][64 K scale words] (no scales for BF16).
template <int kFmt> constexpr int k_tile_bytes() { return kFmt == kFmtBF16 ? kBlockN * kHeadDim * 2 : kBlockN * kHeadDim; }
template <int kFmt> constexpr int scale_off() { return k_tile_bytes<kFmt>() + kVTileB; }
template <int kFmt> constexpr int stage_bytes() { return scale_off<kFmt>() + (kFmt == kFmtBF16 ? 0 : kBlockN * 4); }

// s_waitcnt immediate for vmcnt(n) (lgkmcnt and expcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int N>
using IC = std::integral_constant<int, N>;

// Key (0..63 within the tile) held by LDS K row `row`.  The BMM2 B operand
// takes 64 keys per MFMA, 32 consecutive ones per lane half, so register r of
// lane half h in S^T block kb must hold key 32 h + 16 kb + r.  Accumulator
// register r of lane half h is MFMA row 8 (r / 4) + 4 h + r % 4; block kb
// reads LDS rows 32 kb + (MFMA row), hence row 32 kb + 8 a + 4 h + b holds key
// 32 h + 16 kb + 4 a + b.
__device__ __forceinline__ int sage_key_of_row(int row) {
  const int kb = row >> 5, a = (row >> 3) & 3, h = (row >> 2) & 1, b = row & 3;
  return 32 * h + 16 * kb + 4 * a + b;
}

// kBlock4: k_block >= 4, so each group of 4 keys (aligned) shares one K scale.
template <int kFmt, bool kBlock4, bool kSkip>
__global__ __launch_bounds__(kSageWaves * 64, 1) void fmha_sage_kernel(FmhaSageArgs p) {
  constexpr bool kInt8 = kFmt == kFmtI8;
  constexpr bool kMx = kFmt == kFmtMX8;
  constexpr bool kBf16 = kFmt == kFmtBF16;
  constexpr bool kTokScales = kFmt == kFmtI8 || kFmt == kFmtF8;   // fp32 scale per token block
  constexpr int kKTileB = k_tile_bytes<kFmt>();
  constexpr int kScaleOff = scale_off<kFmt>();
  constexpr int kStageB = stage_bytes<kFmt>();
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kStageB];
  auto stage = [&](auto s) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return st0; else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2; else return st3;
  };

  const int nqt = (p.Sq + kSageBlockM - 1) / kSageBlockM;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % nqt;
  const int bh = wg / nqt;
  const int h = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * kSageBlockM + wave * kSageWaveRows;
  const int Sq = p.Sq, Skv = p.Skv;
  const int64_t s_pad = p.s_pad;
  const int nkt = (Skv + kBlockN - 1) / kBlockN;
  const float c = p.sm_scale * kLog2e;

  // ---- Q of query q0 + l32, B operand of BMM1.  E4M3: 2 k-steps of 64
  // channels (byte assignment above); int8: 4 k-steps of 32, lane half holds
  // 32 ks + 16 hh + 0..15; BF16: 8 k-steps of 16, lane half holds 16 ks +
  // 8 hh + 0..7.  K fragments use the same assignment.
  i32x8 qf8[2];
  i32x4 qi8[4];
  bf16x8 qbf[8];
  float qsc = c;
  int qmx = 0;   // MXFP8: E8M0 scales of this lane's query, byte 2 ks = block 2 ks + hh
  {
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int row = q0 + l32;
    if constexpr (kBf16) {
      const bool ok = row < Sq;
      const bf16_t* qp = static_cast<const bf16_t*>(p.q) + b * p.qs[0] + (int64_t)(ok ? row : 0) * p.qs[1] +
                         h * p.qs[2] + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qbf[ks] = __builtin_bit_cast(bf16x8, ok ? ldg16(qp + 16 * ks) : z);
    } else {
      const uint8_t* qbase = p.q_codes + ((int64_t)b * p.Hq + h) * s_pad * kHeadDim;
      const bool inb = row < s_pad;   // rows < s_pad hold codes (zero past S_q)
      const uint8_t* qp = qbase + (int64_t)(inb ? row : 0) * kHeadDim;
      if constexpr (kInt8) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qi8[ks] = __builtin_bit_cast(i32x4, inb ? ldg16(qp + 32 * ks + 16 * hh) : z);
      } else {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 lo = inb ? ldg16(qp + 64 * ks + 16 * hh) : z;
          const uint4 hi = inb ? ldg16(qp + 64 * ks + 32 + 16 * hh) : z;
          qf8[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
      if constexpr (kTokScales) {
        const int qrow = row < Sq ? row : Sq - 1;
        qsc = p.q_scale[((int64_t)b * p.Hq + h) * p.n_qblk + qrow / p.q_block] * c;
      }
      if constexpr (kMx) {
        const uint32_t w = inb ? *reinterpret_cast<const uint32_t*>(p.q_mx + (((int64_t)b * p.Hq + h) * s_pad + row) * 4) : 0u;
        qmx = (int)(w >> (8 * hh));
      }
    }
  }

  // ---- Loads.  Round R (0..7) of a tile's K covers LDS rows 8R..8R+7 and
  // of its V^T rows 16R..16R+15; wavefront w issues round w of each, plus the
  // 64 scales (every loading wavefront writes the same 256 bytes); wavefronts
  // 8..11 issue no loads.
  const uint8_t* vg = p.v_codes + ((int64_t)b * p.Hkv + g) * kHeadDim * s_pad;
  const i32x4 vrsrc = make_rsrc(vg, (uint32_t)(s_pad * kHeadDim));
  const int vrow = 16 * wave + (lane >> 2);
  const uint32_t voff = (uint32_t)(vrow * s_pad + 16 * ((lane & 3) ^ ((vrow >> 2) & 3)));
  const uint32_t wave_slot = (uint32_t)__builtin_amdgcn_readfirstlane(1024 * wave);
  // K: codes from the workspace, or BF16 rows of the input (rows past S_kv read as zero).
  const char* kg;
  uint32_t kbytes, kstride_b;
  if constexpr (kBf16) {
    kstride_b = (uint32_t)(p.ks[1] * 2);
    kg = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.k) + b * p.ks[0] + g * p.ks[2]);
    kbytes = kstride_b * (uint32_t)Skv;
  } else {
    kstride_b = kHeadDim;
    kg = reinterpret_cast<const char*>(p.k_codes + ((int64_t)b * p.Hkv + g) * s_pad * kHeadDim);
    kbytes = (uint32_t)(s_pad * kHeadDim);
  }
  const i32x4 krsrc = make_rsrc(kg, kbytes);
  uint32_t koff[2];
  if constexpr (kBf16) {   // rounds i = 0, 1: LDS rows 8 wave + 4 i + lane / 16, 16-byte chunk lane % 16
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * wave + 4 * i + (lane >> 4);
      koff[i] = (uint32_t)sage_key_of_row(r) * kstride_b + 16u * (uint32_t)((lane & 15) ^ (r & 15));
    }
  } else {
    const int krow = 8 * wave + (lane >> 3);
    koff[0] = koff[1] = (uint32_t)(sage_key_of_row(krow) * kHeadDim + 16 * ((lane & 7) ^ ((krow >> 1) & 7)));
  }
  // K scale words: one 4-byte word per key of the tile (fp32 scale of its
  // token block, or its four MXFP8 E8M0 bytes).
  i32x4 srsrc = {0, 0, 0, 0};
  uint32_t soff = 0, sstep = 0;
  if constexpr (kTokScales) {
    const float* skg = p.k_scale + ((int64_t)b * p.Hkv + g) * p.n_kblk;
    srsrc = make_rsrc(skg, (uint32_t)(p.n_kblk * 4));
    soff = (uint32_t)(4 * (lane / p.k_block));
    sstep = (uint32_t)(4 * (kBlockN / p.k_block));
  } else if constexpr (kMx) {
    srsrc = make_rsrc(p.k_mx + ((int64_t)b * p.Hkv + g) * s_pad * 4, (uint32_t)(s_pad * 4));
    soff = (uint32_t)(4 * lane);
    sstep = (uint32_t)(4 * kBlockN);
  }
  auto issue_loads = [&](uint32_t sbase, int t) __attribute__((always_inline)) {
    if (wave_slot >= 1024u * kSageLoaders) return;   // scalar branch: wave_slot is uniform
    if constexpr (kBf16) {
      const uint32_t tk = (uint32_t)t * kBlockN * kstride_b;
      buffer_load_lds16(krsrc, sbase + 2 * wave_slot, koff[0] + tk);
      buffer_load_lds16(krsrc, sbase + 2 * wave_slot + 1024, koff[1] + tk);
    } else {
      buffer_load_lds16(krsrc, sbase + wave_slot, koff[0] + (uint32_t)t * kKTileB);
    }
    buffer_load_lds16(vrsrc, sbase + kKTileB + wave_slot, voff + (uint32_t)t * kBlockN);
    if constexpr (!kBf16) buffer_load_lds4(srsrc, sbase + kScaleOff, soff + (uint32_t)t * sstep);
  };

  // ---- LDS read addresses (lane constants; the rest is immediate).
  //   K: E4M3 fragment (kb, ks) = row 32 kb + l32, logical chunks 4 ks + 2 hh + e;
  //      int8 fragment (kb, ks) = logical chunk 2 ks + hh.
  //   V^T: fragment db = row 32 db + l32, logical chunks 2 hh + e.
  int ka[8], va[2];
  {
    if constexpr (kBf16) {   // fragment ks: row 32 kb + l32, logical chunk 2 ks + hh
#pragma unroll
      for (int i = 0; i < 8; ++i) ka[i] = l32 * 2 * kHeadDim + 16 * ((2 * i + hh) ^ (l32 & 15));
    } else {
      const int f = (l32 >> 1) & 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // int8: chunk 2 i + hh; E4M3: chunk 4 (i / 2) + 2 (i % 2) + hh
        const int lc = kInt8 ? 2 * i + hh : 4 * (i >> 1) + 2 * (i & 1) + hh;
        ka[i] = l32 * kHeadDim + 16 * (lc ^ f);
      }
#pragma unroll
      for (int i = 4; i < 8; ++i) ka[i] = 0;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) va[e] = kKTileB + l32 * kBlockN + 16 * ((2 * hh + e) ^ ((l32 >> 2) & 3));
  }
  const int sa = kScaleOff + 4 * 32 * hh;   // this lane half's 32 K scales

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  // Row sum of this lane's keys (its query, its lane half), in units of
  // 2^8 p relative to the current reference m; rescaled with O when m moves.
  float lsum = 0.0f;

  float m = kNegInf;   // running maximum of L over the (kept) tiles, log2 units

  // Skip-Softmax state: the wavefront's skipped-tile count and its bitmap row.
  unsigned skipped = 0;
  const bool qvalid = q0 + l32 < Sq;
  uint8_t* bitmap_row = nullptr;
  if (kSkip && p.bitmap != nullptr && q0 < Sq)
    bitmap_row = p.bitmap + ((int64_t)(b * p.Hq + h) * ((Sq + kSageWaveRows - 1) / kSageWaveRows) +
                             q0 / kSageWaveRows) * nkt;

  // BMM1 of the tile in stage sm into s: S^T of keys 32 hh + 16 kb + r
  // (register r of block kb); int8 accumulators are converted to float.
  auto bmm1 = [&](const uint8_t* sm, f32x16 (&s)[2]) __attribute__((always_inline)) {
    if constexpr (kBf16) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm + ka[ks] + kb * 32 * 2 * kHeadDim);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qbf[ks], s[kb], 0, 0, 0);
        }
    } else if constexpr (kInt8) {
      i32x16 acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kb][r] = 0;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const i32x4 a = *reinterpret_cast<const i32x4*>(sm + ka[ks] + kb * 32 * kHeadDim);
          acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qi8[ks], acc[kb], 0, 0, 0);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = (float)acc[kb][r];
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      int kmx[2] = {0, 0};   // MXFP8: E8M0 scales of this lane's key row, byte 2 ks = block 2 ks + hh
      if constexpr (kMx) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kmx[kb] = (int)(*reinterpret_cast<const uint32_t*>(sm + kScaleOff + 4 * sage_key_of_row(32 * kb + l32)) >>
                          (8 * hh));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(sm + ka[2 * ks] + kb * 32 * kHeadDim);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(sm + ka[2 * ks + 1] + kb * 32 * kHeadDim);
          const i32x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          if constexpr (kMx) {
            if (ks == 0)
              s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[0], s[kb], 0, 0, 0, kmx[kb], 0, qmx);
            else
              s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[1], s[kb], 0, 0, 2, kmx[kb], 2, qmx);
          } else {
            s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf8[ks], s[kb], 0, 0, 0, 0, 0, 0);
          }
        }
    }
  };
  // Softmax of S(tile) (keys key0..key0+63, scales and V^T in stage sm), then BMM2.
  auto softmax_bmm2 = [&](const uint8_t* sm, f32x16 (&s)[2], int key0) __attribute__((always_inline)) {
    // The exponent argument y = L - m + 8 with L = acc * sk * qsc.  With a
    // block of four or more keys per K scale (kFold) the per-key factor
    // sk * qsc is formed once per four keys and y comes from one fma with the
    // reference as it stands; if the tile then moves m, y is shifted by the
    // change.  Otherwise the K scale (SageAttention) is applied first and
    // y = fma(acc', qsc, 8 - m) once m is known.
    constexpr bool kFold = kTokScales && kBlock4;
    const float mt = m == kNegInf ? 0.0f : m;   // reference folded into y (kFold)
    if constexpr (kFold) {
      const float nb0 = 8.0f - mt;
#pragma unroll
      for (int gq = 0; gq < 8; ++gq) {
        const int kb = gq >> 2, r0 = 4 * (gq & 3);
        const float f = *reinterpret_cast<const float*>(sm + sa + 4 * (16 * kb + r0)) * qsc;
#pragma unroll
        for (int j = 0; j < 4; ++j) s[kb][r0 + j] = __builtin_fmaf(s[kb][r0 + j], f, nb0);
      }
    } else {
#pragma unroll
      for (int gq = 0; gq < 8 && kTokScales; ++gq) {
        const int kb = gq >> 2, r0 = 4 * (gq & 3);
        f32x4 sk;
        if constexpr (kBlock4) {
          const float s1 = *reinterpret_cast<const float*>(sm + sa + 4 * (16 * kb + r0));
          sk = f32x4{s1, s1, s1, s1};
        } else {
          sk = *reinterpret_cast<const f32x4*>(sm + sa + 4 * (16 * kb + r0));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) s[kb][r0 + j] *= sk[j];
      }
    }
    if (key0 + kBlockN > Skv) {   // the tile that holds S_kv: a real branch, not selects on every tile
      asm volatile("");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + 32 * hh + 16 * kb + r >= Skv) s[kb][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
    // row maximum of L over the tile
    const float lmax = kFold ? max_halves(mx) - (8.0f - mt) : max_halves(mx) * qsc;
    if constexpr (kSkip) {
      const int t = key0 / kBlockN;
      const bool keep = t == 0 || __any(qvalid && !(lmax - m < p.log2_lambda));
      if (bitmap_row != nullptr && lane == 0) bitmap_row[t] = keep ? 0 : 1;
      if (!keep) {   // wavefront-uniform: a real branch around the rest of the tile
        asm volatile("");
        ++skipped;
        return;
      }
      // Keeps the compiler from hoisting the BMM2 operand reads above the
      // vote (they would stay live beside S through the vote).
      asm volatile("" ::: "memory");
    }
    // Reference update: m' = max(m, tile max).  Lanes l and l + 32 hold the
    // same query and the same m.  alpha = 2^(m - m') is 0 on the first tile
    // (m = -inf; O and l are still zero) and 1 on rows that did not move.
    const float mnew = fmaxf(m, lmax);
    if (__any(mnew > m)) {
      const float alpha = exp2_fast(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      if constexpr (kFold) {   // y was taken against mt: shift it to the new reference
        const float d = mt - mnew;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] += d;
      }
      m = mnew;
    }
    // P = E4M3(2^y): byte 16 kb + r of this lane half is key 32 hh + 16 kb + r.
    // The row sum takes the fp32 values before they are rounded.
    const float nb = 8.0f - m;
    i32x8 pf;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = exp2_fast(kFold ? s[kb][r0 + j] : __builtin_fmaf(s[kb][r0 + j], qsc, nb));
      lsum += (x[0] + x[1]) + (x[2] + x[3]);
      // The low half is written over x[0]'s own register (x[0] is dead after
      // this), so no copy of an "old" value is needed.
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __builtin_bit_cast(int, x[0]), false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], word, true);
    }
    // BMM2 and row sums.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(sm + va[0] + db * 32 * kBlockN);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(sm + va[1] + db * 32 * kBlockN);
      const i32x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, o[db], 0, 0, 0, 127, 0, 127);
    }
  };

  // ---- Tiles: stage t % 4 holds tile t.  Step t: softmax and BMM2 of tile
  // t, then BMM1 of tile t+1 (its MFMAs run under the other wavefronts of the
  // SIMD); tiles t+2 and t+3 are in flight meanwhile.
  f32x16 sA[2];
  issue_loads(lds_addr(st0), 0);
  issue_loads(lds_addr(st1), 1);
  issue_loads(lds_addr(st2), 2);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerTile));   // tile 0 landed
  wg_barrier();
  bmm1(st0, sA);
  auto iteration = [&](auto s_c, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile));   // tile t+1 landed (t+2 may be in flight)
    wg_barrier();   // tiles t, t+1 visible to all; every wavefront is past tile t-1
    issue_loads(lds_addr(stage(IC<(S + 3) & 3>{})), t + 3);
    // Past the last tile the next stage holds zeros; that S is never used.
    softmax_bmm2(stage(IC<S>{}), sA, t * kBlockN);
    bmm1(stage(IC<(S + 1) & 3>{}), sA);
  };
  for (int t = 0;; t += 4) {
    iteration(IC<0>{}, t);
    if (t + 1 >= nkt) break;
    iteration(IC<1>{}, t + 1);
    if (t + 2 >= nkt) break;
    iteration(IC<2>{}, t + 2);
    if (t + 3 >= nkt) break;
    iteration(IC<3>{}, t + 3);
    if (t + 4 >= nkt) break;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (kSkip && p.counter != nullptr && lane == 0 && q0 < Sq && skipped)
    atomicAdd(p.counter, (unsigned long long)skipped);

  // ---- Epilogue: O = O^T * sv_d / l.
  const float* svp = p.v_scale + ((int64_t)b * p.Hkv + g) * kHeadDim;
  // l = both lane halves' sums (lanes l and l ^ 32 hold the same query).
  const float inv = 1.0f / (lsum + __shfl_xor(lsum, 32, 64));
  const int row = q0 + l32;
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
        for (int j = 0; j < 4; ++j) v[j] = o[db][4 * gq + j] * sv[j] * inv;
        if (p.o_fp32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + obase + d) = v;
        } else {
          const bf16x4 vb = __builtin_convertvector(v, bf16x4);
          *reinterpret_cast<bf16x4*>(static_cast<bf16_t*>(p.o) + obase + d) = vb;
        }
      }
  }
}

template <int kFmt, bool kBlock4>
void launch_fmt(const FmhaSageArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.skip)
    hipLaunchKernelGGL((fmha_sage_kernel<kFmt, kBlock4, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fmha_sage_kernel<kFmt, kBlock4, false>), grid, block, 0, stream, a);
}

}  // namespace

hipError_t launch_fmha_sage(const FmhaSageArgs& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kSageBlockM - 1) / kSageBlockM;
  const int64_t nwg = nqt * a.Hq * a.B;
  if (nwg <= 0) return hipSuccess;
  const dim3 grid((unsigned)nwg), block(kSageWaves * 64);
  const bool b4 = a.k_block % 4 == 0;
  switch (a.qk_fmt) {
    case kFmtI8:
      if (b4) launch_fmt<kFmtI8, true>(a, grid, block, stream);
      else launch_fmt<kFmtI8, false>(a, grid, block, stream);
      break;
    case kFmtF8:
      if (b4) launch_fmt<kFmtF8, true>(a, grid, block, stream);
      else launch_fmt<kFmtF8, false>(a, grid, block, stream);
      break;
    case kFmtMX8: launch_fmt<kFmtMX8, false>(a, grid, block, stream); break;
    case kFmtBF16: launch_fmt<kFmtBF16, false>(a, grid, block, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ditattn
