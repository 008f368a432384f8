// Skip-Softmax BF16 attention for gfx950.
//
// Fused multi-head attention O = softmax(sm_scale * Q K^T) V, full context,
// non-causal ("TRTLLM Attention", section "Dense mode"), with the
// Skip-Softmax tile test ("TRTLLM Attention", section "Skip-Softmax"; the
// threshold factor / seqlen of the knob table in "SAGE + Skip-Softmax - API
// Design & Test Plan", Part 1 section 4).
//
// Work decomposition
//   workgroup = 8 wavefronts = 256 query rows of one (batch, query head), two
//   wavefronts per SIMD; each wavefront owns 32 query rows and walks all KV
//   tiles of 64 keys.  One wavefront of a SIMD issues MFMAs while the other
//   runs its softmax VALU work.  Per tile and wavefront:
//     BMM1  S^T[key, query] = K Q^T   16 x v_mfma_f32_32x32x16_bf16
//           (A = K from LDS, B = Q kept in registers for the whole kernel);
//     softmax on S^T: each lane holds one query (lane % 32) and 32 keys, so
//           the row maximum is an in-lane max plus one v_permlane32_swap;
//     BMM2  O^T[d, query] += V^T P^T   16 x v_mfma_f32_32x32x16_bf16
//           (A = V^T read with ds_read_b64_tr_b16 from key-major V in LDS,
//           B = P^T straight from the softmax registers).
//   The first wavefront of each SIMD runs BMM1(t+1), softmax(t), BMM2(t) and
//   the second softmax(t), BMM2(t), BMM1(t+1), so the two alternate.
//
// K/V tiles stream into a 4-stage LDS ring with buffer_load ... lds (no
// register staging; out-of-range rows read as zero), three tiles ahead; one
// barrier per tile.  LDS layouts (256-byte rows, swizzled so that the lanes
// one LDS cycle serves hit 64 distinct four-byte banks):
//   K: row r = MFMA row (32*(r/32) + key_of_mfma_row(r%32) is the key),
//      physical 16-byte chunk = logical chunk ^ (r & 15);
//   V: row = key, physical 64-byte segment = logical segment ^ (key & 3).
//
// Online softmax with a lazy reference maximum: exponentials are taken
// relative to a per-row reference m_ref (log2 units) that is raised only when
// a tile's maximum exceeds it by more than 8, so P <= 2^8 and the O rescale
// runs only when some row's maximum grows that much.  Softmax is invariant to
// the reference, so the result is the same up to rounding.  Row sums add the
// fp32 exponentials.
//
// Skip-Softmax (kSkip): the vote tile is 32 rows (one wavefront) x 32 keys
// (half a KV tile).  After its BMM1, the wavefront skips the half (no
// exponentials, no BMM2) when every valid row i has exp(M_it - m_i) < lambda,
// M_it being the row's maximum over the half and m_i the running maximum over
// the halves kept so far; lambda = factor / S_kv.  The first half is kept.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // log2 headroom before the reference max moves
constexpr int kRowBytes = kHeadDim * 2;                 // one bf16 row of 128 channels
constexpr int kTileBytes = kBlockN * kRowBytes;         // 16 KB per K or V tile
constexpr int kLoadsPerTile = 4;                        // per wavefront: 2 K, 2 V

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int N>
using IC = std::integral_constant<int, N>;

// Accumulator register r of lane half h in a 32x32 S^T block holds MFMA row
// 8*(r/4) + 4*h + r%4.  Feeding MFMA row i with key
//   key(8a + 4h + b) = 16*(a/2) + 8*h + 4*(a%2) + b
// makes register r of lane half h hold key 16*(r/8) + 8*h + r%8: each lane
// half holds runs of 8 consecutive keys, exactly the B-operand slots of the
// BMM2 MFMA (8 consecutive k per lane half).
__device__ __forceinline__ int key_of_mfma_row(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

template <bool kSkip>
__global__ __launch_bounds__(kWavesPerWG * 64, 1) void fmha_skip_kernel(FmhaBf16Args p) {
  // Stage s: K tile at [0, 16 KB), V tile at [16 KB, 32 KB).
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[2 * kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[2 * kTileBytes];
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
  const int nkt = (Skv + kBlockN - 1) / kBlockN;
  const float c = p.sm_scale * kLog2e;

  // ---- Q fragments, B operand of BMM1: lane (query q0 + l32, half hh) holds
  // d = 16*ds + 8*hh + 0..7.
  bf16x8 qf[8];
  {
    const int row = q0 + l32;
    const bool ok = row < Sq;
    const bf16_t* qp = static_cast<const bf16_t*>(p.q) + b * p.qs[0] + (int64_t)(ok ? row : 0) * p.qs[1] +
                       h * p.qs[2] + 8 * hh;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const uint4 u = ok ? ldg16(qp + 16 * ds) : make_uint4(0, 0, 0, 0);
      qf[ds] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // ---- Loads.  Round R (0..15) of a tile covers LDS bytes [1024 R, 1024 R +
  // 1024) of the K (or V) tile = rows 4R..4R+3; wavefront w issues rounds 2w
  // and 2w+1 of each.  Lane l fills row 4R + l/16, physical chunk l%16.
  const uint32_t kstride = (uint32_t)(p.ks[1] * 2), vstride = (uint32_t)(p.vs[1] * 2);
  const char* kbase = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.k) + b * p.ks[0] + g * p.ks[2]);
  const char* vbase = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.v) + b * p.vs[0] + g * p.vs[2]);
  const i32x4 krsrc = make_rsrc(kbase, kstride * (uint32_t)Skv);
  const i32x4 vrsrc = make_rsrc(vbase, vstride * (uint32_t)Skv);
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * wave + i) + (lane >> 4);
    const int pc = lane & 15;
    const int kkey = 32 * (r >> 5) + key_of_mfma_row(r & 31);
    koff[i] = (uint32_t)kkey * kstride + 16u * (uint32_t)(pc ^ (r & 15));
    voff[i] = (uint32_t)r * vstride + 64u * (uint32_t)((pc >> 2) ^ (r & 3)) + 16u * (uint32_t)(pc & 3);
  }
  const uint32_t wave_slot = (uint32_t)__builtin_amdgcn_readfirstlane(2048 * wave);
  auto issue_loads = [&](uint32_t sbase, int t) __attribute__((always_inline)) {
    const uint32_t tk = (uint32_t)t * kBlockN * kstride, tv = (uint32_t)t * kBlockN * vstride;
#pragma unroll
    for (int i = 0; i < 2; ++i) buffer_load_lds16(krsrc, sbase + wave_slot + 1024 * i, koff[i] + tk);
#pragma unroll
    for (int i = 0; i < 2; ++i) buffer_load_lds16(vrsrc, sbase + kTileBytes + wave_slot + 1024 * i, voff[i] + tv);
  };

  // ---- LDS read addresses (lane constants; the rest is immediate).
  //   K fragment (kb, ds): row 32 kb + l32, logical chunk 2 ds + hh.
  //   V^T fragment (db, 4 keys from key k0 + 8 hh, k0 a multiple of 4), read
  //   with ds_read_b64_tr_b16: lane x of each 16-lane group addresses key
  //   k0 + 8 hh + (x%16)/4, channels 32 db + 16 ((x/16) % 2) + 4 (x%4) + 0..3;
  //   the transposing read hands lane 16 G + 4 a + j channel 32 db + 16 (G%2)
  //   + 4 a + j of the four keys.
  int ka[8], va[4];
  {
    const int f = l32 & 15;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) ka[ds] = l32 * kRowBytes + 16 * ((2 * ds + hh) ^ f);
    const int i = (lane & 15) >> 2, a = lane & 3, gg = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      va[db] = kTileBytes + (8 * hh + i) * kRowBytes + 64 * (db ^ i) + 32 * gg + 8 * a;
  }
  auto kfrag = [&](const uint8_t* sm, int kb, int ds) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(sm + ka[ds] + kb * 32 * kRowBytes);
  };
  // 8 keys 32 kb + 16 s2 + 8 hh + 0..7 of channel block db.
  auto vfrag = [&](const uint8_t* sm, int db, int kb, int s2) __attribute__((always_inline)) -> bf16x8 {
    const int off = (32 * kb + 16 * s2) * kRowBytes;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DITATTN_LDS s16x4*)(sm + va[db] + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DITATTN_LDS s16x4*)(sm + va[db] + off + 4 * kRowBytes));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4,
                                   5, 6, 7);
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float mref = kNegInf, mrun = kNegInf, lsum = 0.0f;
  const bool qvalid = q0 + l32 < Sq;
  unsigned skipped = 0;
  const int nqb = (Sq + kWaveRows - 1) / kWaveRows;
  const int nvote = (Skv + kSkipBlockN - 1) / kSkipBlockN;
  uint8_t* bitmap_row = nullptr;
  if (kSkip && p.bitmap != nullptr && q0 < Sq)
    bitmap_row = p.bitmap + ((int64_t)(b * p.Hq + h) * nqb + q0 / kWaveRows) * nvote;

  // ---- BMM1 of the tile in stage sm into s (block kb = keys 32 kb..32 kb+31).
  auto bmm1 = [&](const uint8_t* sm, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
    // Fragments are read two k-steps ahead; the scheduling fences keep the
    // reads ahead of the MFMAs that do not need them.
    bf16x8 kfr[3][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kfr[i][kb] = kfrag(sm, kb, i);
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      if (ds + 2 < 8) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kfr[(ds + 2) % 3][kb] = kfrag(sm, kb, ds + 2);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ds % 3][kb], qf[ds], s[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto rescale = [&](float mnew) __attribute__((always_inline)) {
    const float alpha = exp2_fast(mref - mnew);
    mref = mnew;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  };
  // Skip vote for half u (u > 0): kept unless every valid row is below lambda.
  auto decide = [&](float mx, int u) __attribute__((always_inline)) -> bool {
    bool keep = true;
    if (u > 0) keep = __any(qvalid && !(mx - mrun < p.log2_lambda));
    if (keep)
      mrun = fmaxf(mrun, mx);
    else
      ++skipped;
    if (bitmap_row != nullptr && lane == 0) bitmap_row[u] = keep ? 0 : 1;
    return keep;
  };
  // ---- Softmax of S(tile) (keys key0..key0+63, V in stage sm) and BMM2.
  auto softmax_bmm2 = [&](const uint8_t* sm, f32x16 (&s)[2], int key0) __attribute__((always_inline)) {
    if (key0 + kBlockN > Skv) {   // the tile that holds S_kv: a real branch, not selects on every tile
      asm volatile("");
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7) >= Skv) s[kb][r] = kNegInf;
    }
    float mh[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float m = s[kb][0];
#pragma unroll
      for (int r = 1; r < 16; r += 2) m = fmaxf(fmaxf(m, s[kb][r]), s[kb][r + 1 < 16 ? r + 1 : 15]);
      mh[kb] = max_halves(m) * c;
    }
    bool keep[2] = {true, true};
    if constexpr (kSkip) {
      const int u = 2 * (key0 / kBlockN);
      keep[0] = decide(mh[0], u);
      keep[1] = key0 + 32 < Skv ? decide(mh[1], u + 1) : false;
    }
    const float mx = kSkip ? fmaxf(keep[0] ? mh[0] : kNegInf, keep[1] ? mh[1] : kNegInf) : fmaxf(mh[0], mh[1]);
    if (__any(mx > mref + kRescaleSlack)) rescale(fmaxf(mref, mx));
    const float nb = -mref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kSkip && !keep[kb]) continue;
      bf16x8 pf[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        f32x8 e;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = exp2_fast(__builtin_fmaf(s[kb][8 * s2 + j], c, nb));
          lsum += e[j];
        }
        pf[s2] = __builtin_convertvector(e, bf16x8);
      }
      // V fragments read two MFMAs ahead (step n = 2 db + s2).
      bf16x8 vfr[3];
      vfr[0] = vfrag(sm, 0, kb, 0);
      vfr[1] = vfrag(sm, 0, kb, 1);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        if (n + 2 < 8) vfr[(n + 2) % 3] = vfrag(sm, (n + 2) >> 1, kb, (n + 2) & 1);
        o[n >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[n % 3], pf[n & 1], o[n >> 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- Tiles: stage t % 4 holds tile t; BMM1 of tile t+1 runs in step t.
  f32x16 sA[2], sB[2];
  issue_loads(lds_addr(st0), 0);
  issue_loads(lds_addr(st1), 1);
  issue_loads(lds_addr(st2), 2);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerTile));   // tile 0 landed
  wg_barrier();
  bmm1(st0, sA);
  auto iteration = [&](auto s_c, int t, f32x16 (&scur)[2], f32x16 (&snext)[2]) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile));   // tile t+1 landed (t+2 may be in flight)
    wg_barrier();   // tiles t, t+1 visible to all; every wavefront is past tile t-1
    issue_loads(lds_addr(stage(IC<(S + 3) & 3>{})), t + 3);
    // Past the last tile the next stage holds zeros; that S is never used.
    if (wave < kWavesPerWG / 2) {   // first wavefront of each SIMD: MFMA work first
      bmm1(stage(IC<(S + 1) & 3>{}), snext);
      softmax_bmm2(stage(IC<S>{}), scur, t * kBlockN);
    } else {                        // second: VALU work first, so the two alternate
      softmax_bmm2(stage(IC<S>{}), scur, t * kBlockN);
      bmm1(stage(IC<(S + 1) & 3>{}), snext);
    }
  };
  for (int t = 0;; t += 4) {
    iteration(IC<0>{}, t, sA, sB);
    if (t + 1 >= nkt) break;
    iteration(IC<1>{}, t + 1, sB, sA);
    if (t + 2 >= nkt) break;
    iteration(IC<2>{}, t + 2, sA, sB);
    if (t + 3 >= nkt) break;
    iteration(IC<3>{}, t + 3, sB, sA);
    if (t + 4 >= nkt) break;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  if (kSkip && p.counter != nullptr && lane == 0 && q0 < Sq && skipped)
    atomicAdd(p.counter, (unsigned long long)skipped);

  // ---- Epilogue: O = O^T / l, lane writes 4 consecutive d per register group.
  const float lrow = sum_halves(lsum);
  const float inv = 1.0f / lrow;
  const int row = q0 + l32;
  // LSE over the kept keys = (m_ref + log2 l) ln 2, P being 2^(L - m_ref).
  if (p.lse != nullptr && hh == 0 && row < Sq)
    p.lse[((int64_t)b * p.Hq + h) * Sq + row] = (mref + __log2f(lrow)) * kLn2;
  if (row < Sq) {
    const int64_t obase = b * p.os[0] + (int64_t)row * p.os[1] + h * p.os[2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * hh;
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = o[db][4 * gq + j] * inv;
        if (p.o_fp32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + obase + d) = v;
        } else {
          const bf16x4 vb = __builtin_convertvector(v, bf16x4);
          *reinterpret_cast<bf16x4*>(static_cast<bf16_t*>(p.o) + obase + d) = vb;
        }
      }
  }
}

}  // namespace

hipError_t launch_fmha_bf16_skip(const FmhaBf16Args& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBlockM - 1) / kBlockM;
  const int64_t nwg = nqt * a.Hq * a.B;
  if (nwg <= 0) return hipSuccess;
  hipLaunchKernelGGL(fmha_skip_kernel<true>, dim3((unsigned)nwg), dim3(kWavesPerWG * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ditattn
