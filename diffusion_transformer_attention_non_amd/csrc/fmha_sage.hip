// SAGE attention on quantized codes for gfx950 ("TRTLLM Attention", section
// "SAGE quantization": both attention matmuls in low precision; "VisualGen
// Quantized Attention", section "SageAttention in the TRTLLM backend").
//
// Same decomposition as the BF16 kernel (workgroup = 4 wavefronts x 64 query
// rows, KV tiles of 64 keys, transposed products so that each query stays in
// one lane), with:
//   BMM1  S^T = Kc Qc^T on int8 (v_mfma_i32_32x32x32_i8, exact int32) or
//         OCP E4M3 (v_mfma_f32_32x32x64_f8f6f4) codes; the logit in log2
//         units is L_ij = acc_ij * sk_j * (sq_i * sm_scale * log2 e);
//   softmax per tile with a power-of-two reference: m' = max(m, ceil(tile max)),
//         e = 2^(L - m' + 8) = 2^8 p, p~ = E4M3(e), l = 2^(m - m') l + sum p~;
//   BMM2  O^T += Vc^T E4M3(e)^T on E4M3 codes (v_mfma_f32_32x32x64_f8f6f4),
//         V^T codes read as written by the quantizer (d-major);
//   epilogue O = acc * sv_d / l (bmm2 scale), l holding the 2^8 factor.
//
// Pipeline (per wavefront, tile t):
//   Y block: BMM1(t+1)  || exponentials of quads 5-15 of S(t)
//   X block: BMM2(t)    || dequantization and row max of S(t+1), quads 0-4 of S(t+1)
// A quad is four keys of one query: scale-and-shift, exp2, then E4M3 packing
// into one P register, on three consecutive MFMA slots.  The row sums come
// from MFMAs on the packed P (the values BMM2 multiplies).
// The X-block exponentials use the reference before tile t+1; when the tile
// raises some row's reference (the check after the block), those quads are
// redone, so every P value is relative to the reference as above.
//
// K codes, V^T codes and the tile's 64 K scales stream into a 4-stage LDS
// ring with buffer_load ... lds, three tiles ahead (out-of-range reads are
// zero).  LDS layouts (16-byte chunks, XOR-swizzled so that reads of 32 rows
// at one logical chunk hit distinct banks):
//   K:   64 rows x 128 B in MFMA-row order, physical chunk = logical ^ (row & 7);
//   V^T: 128 rows (channel) x 64 B (keys), physical chunk = logical ^ ((row >> 1) & 3).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kKTileB = kBlockN * kHeadDim;   // 8 KB of K codes
constexpr int kVTileB = kHeadDim * kBlockN;   // 8 KB of V^T codes
constexpr int kScaleOff = kKTileB + kVTileB;  // 64 fp32 K scales follow
constexpr int kStageB = kScaleOff + kBlockN * 4;
constexpr int kLoadsPerTile = 5;              // per wavefront: 2 K, 2 V, 1 scales
constexpr float kMaxRefGap = 64.0f;           // largest m - mo carried by the E8M0 P scale

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

template <bool kInt8>
__global__ __launch_bounds__(256, 1) void fmha_sage_kernel(FmhaSageArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kStageB];
  auto stage = [&](auto s) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return st0; else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2; else return st3;
  };

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
  const int nkt = (Skv + kBlockN - 1) / kBlockN;

  // ---- Q codes, B operand of BMM1.  E4M3: 2 k-steps of 64 channels, lane
  // half hh holds channels 64 ks + 32 hh + 0..31; int8: 4 k-steps of 32, lane
  // half holds 32 ks + 16 hh + 0..15.
  constexpr int kQSteps = kInt8 ? 4 : 2;
  i32x8 qf8[2][2];
  i32x4 qi8[2][4];
  float qsc[2];
  const float c = p.sm_scale * kLog2e;
  {
    const uint8_t* qbase = p.q_codes + ((int64_t)b * p.Hq + h) * s_pad * kHeadDim;
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = q0 + qb * 32 + l32;   // rows < s_pad hold codes (zero past S_q)
      const bool inb = row < s_pad;
      const uint8_t* qp = qbase + (int64_t)(inb ? row : 0) * kHeadDim;
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks) {
        if constexpr (kInt8) {
          qi8[qb][ks] = __builtin_bit_cast(i32x4, inb ? ldg16(qp + 32 * ks + 16 * hh) : z);
        } else {
          const uint4 lo = inb ? ldg16(qp + 64 * ks + 32 * hh) : z;
          const uint4 hi = inb ? ldg16(qp + 64 * ks + 32 * hh + 16) : z;
          qf8[qb][ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
      }
      const int qrow = row < Sq ? row : Sq - 1;
      qsc[qb] = p.q_scale[((int64_t)b * p.Hq + h) * p.n_qblk + qrow / p.q_block] * c;
    }
  }

  // ---- Loads.  Round R (0..7) of a tile's K covers LDS rows 8R..8R+7 and
  // of its V^T rows 16R..16R+15; wavefront w issues rounds 2w and 2w+1 of
  // each, plus the 64 scales (every wavefront writes the same 256 bytes).
  const uint8_t* kg = p.k_codes + ((int64_t)b * p.Hkv + g) * s_pad * kHeadDim;
  const uint8_t* vg = p.v_codes + ((int64_t)b * p.Hkv + g) * kHeadDim * s_pad;
  const float* skg = p.k_scale + ((int64_t)b * p.Hkv + g) * p.n_kblk;
  const i32x4 krsrc = make_rsrc(kg, (uint32_t)(s_pad * kHeadDim));
  const i32x4 vrsrc = make_rsrc(vg, (uint32_t)(s_pad * kHeadDim));
  const i32x4 srsrc = make_rsrc(skg, (uint32_t)(p.n_kblk * 4));
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int R = 2 * wave + i;
    const int krow = 8 * R + (lane >> 3);
    koff[i] = (uint32_t)(sage_key_of_row(krow) * kHeadDim + 16 * ((lane & 7) ^ (krow & 7)));
    const int vrow = 16 * R + (lane >> 2);
    voff[i] = (uint32_t)(vrow * s_pad + 16 * ((lane & 3) ^ ((vrow >> 1) & 3)));
  }
  const uint32_t soff = (uint32_t)(4 * (lane / p.k_block));
  const uint32_t sstep = (uint32_t)(4 * (kBlockN / p.k_block));   // scale bytes per tile
  const uint32_t wave_slot = (uint32_t)__builtin_amdgcn_readfirstlane(2048 * wave);
  // Load i (0..4) of tile t into stage sbase (LDS byte address).
  auto load_one = [&](uint32_t sbase, int t, int i) __attribute__((always_inline)) {
    if (i < 2)
      buffer_load_lds16(krsrc, sbase + wave_slot + 1024 * i, koff[i] + (uint32_t)t * kKTileB);
    else if (i < 4)
      buffer_load_lds16(vrsrc, sbase + kKTileB + wave_slot + 1024 * (i - 2), voff[i - 2] + (uint32_t)t * kBlockN);
    else
      buffer_load_lds4(srsrc, sbase + kScaleOff, soff + (uint32_t)t * sstep);
  };

  // ---- LDS read addresses (lane constants; the rest is immediate).
  //   K: E4M3 fragment (kb, ks) = row 32 kb + l32, logical chunks 4 ks + 2 hh + e;
  //      int8 fragment (kb, ks) = logical chunk 2 ks + hh.
  //   V^T: fragment db = row 32 db + l32, logical chunks 2 hh + e.
  int ka[4], va[2];
  {
    const int f = l32 & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lc = kInt8 ? 2 * i + hh : 4 * (i >> 1) + 2 * hh + (i & 1);
      ka[i] = l32 * kHeadDim + 16 * (lc ^ f);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) va[e] = kKTileB + l32 * kBlockN + 16 * ((2 * hh + e) ^ ((l32 >> 1) & 3));
  }

  f32x16 o[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.0f;
  // Softmax reference per query: m = ceil of the running maximum (log2
  // units, an integer), so p = 2^(L - m) <= 1 and P = E4M3(2^(L - m + 8)).
  // O and l stay relative to an older integer reference mo; BMM2 and the
  // row-sum MFMA multiply P by 2^(m - mo) through their E8M0 B-operand scale
  // (bsc = 127 + m - mo), so moving m never rescales O.  Only when m - mo
  // would leave the safe range is O rescaled, by an exact power of two.
  float m[2] = {kNegInf, kNegInf};
  float mo[2] = {kNegInf, kNegInf};
  int bsc[2] = {127, 127};
  float nb[2] = {__builtin_huge_valf(), __builtin_huge_valf()};   // 8 - m
  // Row sums l = sum of the E4M3 P values, accumulated by 32x32x64 MFMAs with
  // an all-ones A operand: every row of the result is the column (query)
  // sum.  The query block qb = 0 MFMA has ones in A rows 0-15 and qb = 1 in
  // rows 16-31, so one accumulator holds both: registers 0-7 of lane l are
  // query l % 32 of block 0, registers 8-15 of block 1.  The B scale of each
  // 32-key block comes from a lane holding the same query, as in BMM2.
  f32x16 lrow;
#pragma unroll
  for (int r = 0; r < 16; ++r) lrow[r] = 0.0f;
  const int ones0 = l32 < 16 ? 0x38383838 : 0, ones1 = l32 < 16 ? 0 : 0x38383838;   // E4M3 1.0 = 0x38
  const i32x8 sel_ones[2] = {{ones0, ones0, ones0, ones0, ones0, ones0, ones0, ones0},
                             {ones1, ones1, ones1, ones1, ones1, ones1, ones1, ones1}};

  f32x16 sb[2][2][2];   // dequantized S^T of two tiles in flight, [buffer][kb][qb]
  i32x16 si[2][2][2];   // int8: BMM1 accumulators before dequantization
  i32x8 pf[2][2];       // E4M3(2^8 p) of two tiles, [buffer][qb]: byte 16 kb + r of lane half hh = key 32 hh + 16 kb + r

  auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };

  // ---- BMM1 of tile (K from LDS stage ks) into sdst; valu(v) follows the MFMA of VALU slot v.
  auto bmm1_block = [&](const uint8_t* ksm, f32x16 (&sdst)[2][2], i32x16 (&idst)[2][2], auto&& valu)
      __attribute__((always_inline)) {
    if constexpr (kInt8) {
      // 16 MFMAs: (ks, kb, qb); VALU slot v after MFMA 2v+1.
      i32x4 kfr[3];
      auto kread = [&](int n) __attribute__((always_inline)) -> i32x4 {   // fragment n = 2 ks + kb
        return *reinterpret_cast<const i32x4*>(ksm + ka[n >> 1] + (n & 1) * 32 * kHeadDim);
      };
      kfr[0] = kread(0);
      kfr[1] = kread(1);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int n = t >> 1, qb = t & 1, ks = n >> 1, kb = n & 1;
        if (qb == 0 && n + 2 < 8) kfr[(n + 2) % 3] = kread(n + 2);
        i32x16 acc;
        if (ks == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0;
        } else {
          acc = idst[kb][qb];
        }
        idst[kb][qb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kfr[n % 3], qi8[qb][ks], acc, 0, 0, 0);
        if (qb == 1) valu(n);
        fence();
      }
    } else {
      // 8 MFMAs: (ks, kb, qb); VALU slot v after MFMA v.
      i32x8 kfr[3];
      auto kread = [&](int n) __attribute__((always_inline)) -> i32x8 {   // fragment n = 2 ks + kb
        const int ks = n >> 1, kb = n & 1;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(ksm + ka[2 * ks] + kb * 32 * kHeadDim);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(ksm + ka[2 * ks + 1] + kb * 32 * kHeadDim);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      kfr[0] = kread(0);
      kfr[1] = kread(1);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int n = t >> 1, qb = t & 1, ks = n >> 1, kb = n & 1;
        if (qb == 0 && n + 2 < 4) kfr[(n + 2) % 3] = kread(n + 2);
        f32x16 acc;
        if (ks == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        } else {
          acc = sdst[kb][qb];
        }
        sdst[kb][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kfr[n % 3], qf8[qb][ks], acc, 0, 0, 0, 0, 0, 0);
        valu(t);
        fence();
      }
    }
    valu(8);
    valu(9);
  };

  // ---- BMM2: O^T += V^T P^T (V^T from LDS stage vsm), 8 MFMAs (db, qb).
  auto bmm2_block = [&](const uint8_t* vsm, const i32x8 (&pin)[2], auto&& valu) __attribute__((always_inline)) {
    i32x8 vfr[3];
    auto vread = [&](int db) __attribute__((always_inline)) -> i32x8 {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(vsm + va[0] + db * 32 * kBlockN);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(vsm + va[1] + db * 32 * kBlockN);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    vfr[0] = vread(0);
    vfr[1] = vread(1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int db = t >> 1, qb = t & 1;
      if (qb == 0 && db + 2 < 4) vfr[(db + 2) % 3] = vread(db + 2);
      o[db][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vfr[db % 3], pin[qb], o[db][qb], 0, 0, 0, 127, 0,
                                                                 bsc[qb]);
      valu(t);
      fence();
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      lrow = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(sel_ones[qb], pin[qb], lrow, 0, 0, 0, 127, 0, bsc[qb]);
      fence();
    }
  };

  // ---- Softmax pieces.
  // Dequantization and row max of group gq (0..7: kb = gq / 4, registers
  // 4 (gq % 4) + j) of S buffer sv; scales from stage ssm.  In the tile that
  // holds S_kv (tail), keys at or past S_kv become -inf.
  float mp[2];
  // K scales of group gq (keys 32 hh + 4 gq + 0..3) of the tile in stage ssm,
  // read two groups ahead into a ring of three.
  f32x4 skr[3];
  auto read_scales = [&](const uint8_t* ssm, int gq) __attribute__((always_inline)) {
    skr[gq % 3] = *reinterpret_cast<const f32x4*>(ssm + kScaleOff + 4 * (32 * hh + 4 * gq));
  };
  auto dequant_group = [&](f32x16 (&sv)[2][2], const i32x16 (&iv)[2][2], int gq, int key0, bool tail)
      __attribute__((always_inline)) {
    const int kb = gq >> 2, r0 = 4 * (gq & 3);
    float t4[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = kInt8 ? (float)iv[kb][qb][r0 + j] : sv[kb][qb][r0 + j];
        t4[qb][j] = x * skr[gq % 3][j];
      }
    if (tail) {   // only the tile that holds S_kv: a real branch, not selects on every tile
      asm volatile("");
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key0 + 32 * hh + 16 * kb + r0 + j >= Skv) t4[0][j] = t4[1][j] = kNegInf;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[kb][qb][r0 + j] = t4[qb][j];
      mp[qb] = fmaxf(fmaxf(mp[qb], t4[qb][0]), t4[qb][1]);
      mp[qb] = fmaxf(fmaxf(mp[qb], t4[qb][2]), t4[qb][3]);
    }
  };
  // Quad k (0..15): qb = k / 8, P register w = k % 8 (kb = w / 4, S registers 4 (w % 4) + j).
  float ex[6][4];
  auto quad_stage = [&](int st, const f32x16 (&sv)[2][2], i32x8 (&pout)[2], int k, int slot)
      __attribute__((always_inline)) {
    const int qb = k >> 3, w = k & 7, kb = w >> 2, r0 = 4 * (w & 3);
    float(&x)[4] = ex[slot];
    if (st == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = __builtin_fmaf(sv[kb][qb][r0 + j], qsc[qb], nb[qb]);
      asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
    } else if (st == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = exp2_fast(x[j]);
      asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
    } else {
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __builtin_bit_cast(int, x[3]), false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], word, true);
      asm volatile("" : "+v"(word));
      pout[qb][w] = word;
    }
  };
  // X-block VALU: group v dequantized at slot v; quads 0, 8, 1, 9, 2 run
  // their three stages from slots 1..5.
  constexpr int kXQuads[5] = {0, 8, 1, 9, 2};
  auto x_valu = [&](f32x16 (&sv)[2][2], const i32x16 (&iv)[2][2], i32x8 (&pout)[2], const uint8_t* ssm, int key0,
                    bool tail, int v) __attribute__((always_inline)) {
    if (v == 0) {
      mp[0] = mp[1] = kNegInf;
    }
    if (v + 2 < 8) read_scales(ssm, v + 2);
    if (v < 8) dequant_group(sv, iv, v, key0, tail);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      if (v == i + 3) quad_stage(2, sv, pout, kXQuads[i], i);
      if (v == i + 2) quad_stage(1, sv, pout, kXQuads[i], i);
      if (v == i + 1) quad_stage(0, sv, pout, kXQuads[i], i);
    }
  };
  // Y-block VALU: the other 11 quads, scale-and-shift at slot kYStart[i].
  constexpr int kYQuads[11] = {10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15};
  constexpr int kYStart[11] = {0, 1, 1, 2, 3, 3, 4, 5, 5, 6, 7};
  auto y_valu = [&](const f32x16 (&sv)[2][2], i32x8 (&pout)[2], int v) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 11; ++i) {
      if (v == kYStart[i] + 2) quad_stage(2, sv, pout, kYQuads[i], i % 6);
      if (v == kYStart[i] + 1) quad_stage(1, sv, pout, kYQuads[i], i % 6);
      if (v == kYStart[i]) quad_stage(0, sv, pout, kYQuads[i], i % 6);
    }
  };
  // After an X block: update the running maximum; when it moved, rescale O
  // and l and redo the X-block quads with the new maximum.
  auto x_check = [&](const f32x16 (&sv)[2][2], i32x8 (&pout)[2]) __attribute__((always_inline)) {
    float mnew[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) mnew[qb] = fmaxf(m[qb], __builtin_ceilf(max_halves(mp[qb]) * qsc[qb]));
    if (__any(mnew[0] > m[0] || mnew[1] > m[1])) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (m[qb] == kNegInf) mo[qb] = mnew[qb];   // the first tile fixes the O reference
        m[qb] = mnew[qb];
        nb[qb] = 8.0f - mnew[qb];
      }
      if (__any(m[0] - mo[0] > kMaxRefGap || m[1] - mo[1] > kMaxRefGap)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float f = exp2_fast(mo[qb] - m[qb]);   // exact: the difference is an integer
          mo[qb] = m[qb];
#pragma unroll
          for (int r = 0; r < 8; ++r) lrow[8 * qb + r] *= f;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][qb][r] *= f;
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) bsc[qb] = 127 + (int)(m[qb] - mo[qb]);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        quad_stage(0, sv, pout, kXQuads[i], i);
        quad_stage(1, sv, pout, kXQuads[i], i);
        quad_stage(2, sv, pout, kXQuads[i], i);
      }
    }
  };

  // ---- Prologue: tiles 0..2 in flight; S(0) and its X-block work.
#pragma unroll
  for (int i = 0; i < kLoadsPerTile; ++i) load_one(lds_addr(st0), 0, i);
#pragma unroll
  for (int i = 0; i < kLoadsPerTile; ++i) load_one(lds_addr(st1), 1, i);
#pragma unroll
  for (int i = 0; i < kLoadsPerTile; ++i) load_one(lds_addr(st2), 2, i);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerTile));
  wg_barrier();
  read_scales(st0, 0);
  read_scales(st0, 1);
  bmm1_block(st0, sb[0], si[0], [](int) {});
#pragma unroll
  for (int v = 0; v < 8; ++v) x_valu(sb[0], si[0], pf[0], st0, 0, kBlockN > Skv, v);
  x_check(sb[0], pf[0]);

  // ---- Tile t (stage S = t % 4), S(t) and its X-block work done:
  //   Y: BMM1(t+1) || quads 5-15 of S(t), loads of tile t+3;
  //   X: BMM2(t)   || dequantization, max and quads 0-4 of S(t+1), then the check.
  // Past the last tile the K stage holds zeros and every key is masked, so
  // the extra BMM1 and X-block work change nothing.
  auto iteration = [&](auto s_c, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    constexpr int B0 = S & 1, B1 = (S + 1) & 1;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile));   // tile t+1 landed (t+2 may be in flight)
    wg_barrier();
    const uint32_t ldst = lds_addr(stage(IC<(S + 3) & 3>{}));
    bmm1_block(stage(IC<(S + 1) & 3>{}), sb[B1], si[B1], [&](int v) __attribute__((always_inline)) {
      if (v == 6) read_scales(stage(IC<(S + 1) & 3>{}), 0);
      if (v == 7) read_scales(stage(IC<(S + 1) & 3>{}), 1);
      y_valu(sb[B0], pf[B0], v);
      if (v < kLoadsPerTile) load_one(ldst, t + 3, v);
    });
    const int key1 = (t + 1) * kBlockN;
    const bool tail = key1 + kBlockN > Skv;
    bmm2_block(stage(IC<S>{}), pf[B0], [&](int v) __attribute__((always_inline)) {
      x_valu(sb[B1], si[B1], pf[B1], stage(IC<(S + 1) & 3>{}), key1, tail, v);
    });
    x_check(sb[B1], pf[B1]);
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

  // ---- Epilogue: O = O^T * sv_d / l.
  const float* svp = p.v_scale + ((int64_t)b * p.Hkv + g) * kHeadDim;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lrow[8 * qb];
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
