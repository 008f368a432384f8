// Dense and Skip-Softmax BF16 attention for gfx950.
//
// Fused multi-head attention O = softmax(sm_scale * Q K^T) V, full context,
// non-causal ("TRTLLM Attention", section "Dense mode"; "Diffusion Attention
// Backends", backend table: BF16, native GQA, head_dim 128), and with kSkip
// the Skip-Softmax tile test ("TRTLLM Attention", section "Skip-Softmax";
// threshold factor / seqlen from the knob table of "SAGE + Skip-Softmax -
// API Design & Test Plan", Part 1 section 4).
//
// Work decomposition
//   workgroup = 4 wavefronts = 256 query rows of one (batch, query head);
//   each wavefront owns 64 query rows and walks all KV tiles of 64 keys.
//   Per 32-key half of a tile and wavefront:
//     BMM1  S^T[key, query] = K Q^T   16 x v_mfma_f32_32x32x16_bf16
//           (A = K from LDS, B = Q kept in registers for the whole kernel);
//     softmax on S^T: each lane holds one query column of each 32x32 block,
//           so the row maximum is an in-lane max plus one v_permlane32_swap;
//     BMM2  O^T[d, query] += V^T P^T   16 x v_mfma_f32_32x32x16_bf16
//           (A = V^T read with ds_read_b64_tr_b16 from row-major V in LDS,
//           B = P^T straight from the softmax registers).
//   Computing the transposed products keeps each query in one lane, so the
//   softmax state (max, sum, rescale factor) never leaves the lane.
//
// Pipeline
//   K/V tiles stream into a 4-stage LDS ring with buffer_load ... lds (no
//   register staging; out-of-range rows read as zero), three tiles ahead; the
//   loop is unrolled by the ring depth so every stage is a distinct array.
//   Each half's VALU work rides on two 16-MFMA blocks (described with the
//   blocks below); the order inside a block is written out (MFMA, its share
//   of VALU work, scheduling fence), with LDS fragments read ahead.
//
// Skip-Softmax (kSkip): the vote tile is the wavefront's 64 rows x one
// 32-key half.  Once a half's row maxima are known (the check after its Q
// block) the wavefront drops it when every valid row i has
// exp(M_it - m_i) < lambda, M_it the row's maximum over the half and m_i its
// exact running maximum over the kept halves; lambda = factor / S_kv.  The
// first half is kept.  A dropped half skips its BMM2 and row-sum MFMAs (the
// Q block that carries them runs its VALU work alone) and changes no
// softmax state; its speculative exponentials are simply unused.
//
// Online softmax with a lazy reference maximum: exponentials are taken
// relative to a per-row reference m_ref (log2 units) that is raised only when
// a tile's maximum exceeds it by more than 8, so P <= 2^8 and the O rescale
// runs only when some row's maximum grows that much.  Softmax is invariant to
// the reference, so the result is the same up to rounding.  Row sums are taken
// on the matrix cores from the bf16 P that BMM2 multiplies.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr int kDenseWaveRows = kSkipBlockM;   // query rows per wavefront (the skip vote's rows)
constexpr int kDenseWaves = kBlockM / kDenseWaveRows;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // log2 headroom before the reference max moves
constexpr int kRowBytes = kHeadDim * 2;                 // one bf16 row of 128 channels
constexpr int kTileBytes = kBlockN * kRowBytes;         // 16 KB per K or V tile
constexpr int kLoadsPerTile = 8;                        // buffer->LDS loads per wavefront per tile
constexpr int kPrefetch = 2;                            // LDS fragments are read this many MFMA steps ahead

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// sched_group_barrier instruction classes.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

template <int N>
using IC = std::integral_constant<int, N>;

// bf16 pair jp (0..3) of an 8-element vector.  Written as constant shuffles:
// extracting a lane of the bit-cast int vector instead was lowered to lane 0
// for every jp by the compiler used here.
__device__ __forceinline__ bf16x2 bf16_pair(const bf16x8 v, int jp) {
  switch (jp) {
    case 0: return __builtin_shufflevector(v, v, 0, 1);
    case 1: return __builtin_shufflevector(v, v, 2, 3);
    case 2: return __builtin_shufflevector(v, v, 4, 5);
    default: return __builtin_shufflevector(v, v, 6, 7);
  }
}

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

// LDS tile layouts (256-byte rows, swizzled so that the lanes one LDS cycle
// serves hit 64 distinct four-byte banks):
//   K: row r = MFMA row (32*(r/32) + key_of_mfma_row(r%32) is the key),
//      physical 16-byte chunk = logical chunk ^ (r & 15);
//   V: row = key, physical 64-byte segment = logical segment ^ (key & 3).

// kBitmap (with kSkip): the caller asked for the per-half skip bitmap; the
// common case has no store in the loop at all.
template <bool kSkip, bool kBitmap>
__global__ __launch_bounds__(kDenseWaves * 64, 1) void fmha_bf16_kernel(FmhaBf16Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sK2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sK3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV3[kTileBytes];
  auto kst = [&](auto s) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return sK0; else if constexpr (S == 1) return sK1;
    else if constexpr (S == 2) return sK2; else return sK3;
  };
  auto vst = [&](auto s) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return sV0; else if constexpr (S == 1) return sV1;
    else if constexpr (S == 2) return sV2; else return sV3;
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
  const int q0 = qt * kBlockM + wave * kDenseWaveRows;
  const int Sq = p.Sq, Skv = p.Skv;
  const int nkt = (Skv + kBlockN - 1) / kBlockN;

  // ---- Q fragments, B operand of BMM1: lane (query l32 of block qb, half hh)
  // holds d = 16*ds + 8*hh + 0..7.
  bf16x8 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 32 + l32;
    const bool ok = row < Sq;
    const bf16_t* qp = static_cast<const bf16_t*>(p.q) + b * p.qs[0] +
                       (int64_t)(ok ? row : 0) * p.qs[1] + h * p.qs[2] + 8 * hh;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 u = ok ? ldg16(qp + 16 * ds) : make_uint4(0, 0, 0, 0);
      qf[qb][ds] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // ---- Buffer resources over this (b, kv head)'s K and V rows; rows past
  // S_kv are out of range and load as zero.
  const uint32_t kstride = (uint32_t)(p.ks[1] * 2), vstride = (uint32_t)(p.vs[1] * 2);
  const char* kbase = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.k) + b * p.ks[0] + g * p.ks[2]);
  const char* vbase = reinterpret_cast<const char*>(static_cast<const bf16_t*>(p.v) + b * p.vs[0] + g * p.vs[2]);
  const i32x4 krsrc = make_rsrc(kbase, kstride * (uint32_t)Skv);
  const i32x4 vrsrc = make_rsrc(vbase, vstride * (uint32_t)Skv);

  // Load slots: round i (0..3) of the workgroup covers LDS bytes [4096 i, 4096 i + 4096);
  // lane fills 16-byte slot 256 i + 64 wave + lane = row 16 i + 4 wave + lane/16, chunk lane%16.
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + 4 * wave + (lane >> 4);
    const int pch = lane & 15;
    const int kkey = 32 * (r >> 5) + key_of_mfma_row(r & 31);
    koff[i] = (uint32_t)kkey * kstride + 16u * (uint32_t)(pch ^ (r & 15));
    voff[i] = (uint32_t)r * vstride + 64u * (uint32_t)((pch >> 2) ^ (r & 3)) + 16u * (uint32_t)(pch & 3);
  }
  const uint32_t wave_slot = (uint32_t)__builtin_amdgcn_readfirstlane(1024 * wave);
  auto issue_loads = [&](auto s, int t) __attribute__((always_inline)) {
    const uint32_t tk = (uint32_t)t * kBlockN * kstride, tv = (uint32_t)t * kBlockN * vstride;
#pragma unroll
    for (int i = 0; i < 4; ++i) buffer_load_lds16_at(krsrc, wave_slot, lds_addr(kst(s)) + 4096 * i, koff[i] + tk);
#pragma unroll
    for (int i = 0; i < 4; ++i) buffer_load_lds16_at(vrsrc, wave_slot, lds_addr(vst(s)) + 4096 * i, voff[i] + tv);
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
    for (int db = 0; db < 4; ++db) va[db] = (8 * hh + i) * kRowBytes + 64 * (db ^ i) + 32 * gg + 8 * a;
  }

  f32x16 o[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.0f;

  const float c = p.sm_scale * kLog2e;
  float mref[2];
  // Row sums of P on the matrix cores: v_mfma_f32_16x16x32_bf16 with B = the
  // BMM2 operand P^T (lane l: query 32 qb + l % 32, 8 keys from 8 (l / 32))
  // and a 0/1 selector A whose row 0 takes lane groups 0 and 2 (queries
  // 32 qb + 0..15) and row 1 groups 1 and 3 (queries 32 qb + 16..31).  Result
  // register r of lane n < 16 then holds the row sum of query 32 qb + 16 r + n
  // (r = 0, 1); every other entry stays zero.  The sums are of the bf16 P that
  // BMM2 multiplies.
  bf16x8 rsel;
  {
    const int m = lane & 15, grp = lane >> 4;
    const __bf16 one = (m < 2 && m == (grp & 1)) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) rsel[i] = one;
  }
  f32x4 rsum[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 4; ++r) rsum[qb][r] = 0.0f;

  // ---- Dense pipeline.  A half-tile (32 keys) goes through BMM1 (S), the row
  // maximum, 16 exponential pairs (P) and BMM2.  Two 16-MFMA blocks per half
  // carry its VALU work:
  //   Q block of half u: BMM2(u-1) || row max of S(u), exponential pairs 0-6 of S(u)
  //   P block of half u: BMM1(u+1) || exponential pairs 7-15 of S(u)
  // The exponentials of the Q block are taken with the reference maximum as
  // it stands (speculatively); the check after the block redoes them in the
  // rare case the reference has to move.  Every pair runs a three-stage
  // pipeline over consecutive MFMA slots (scale and shift, exp2, pack to
  // bf16), so no slot waits on its own results.
  auto fence = [&]() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
  auto kfrag = [&](const uint8_t* ks, int kb, int ds) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(ks + ka[ds] + kb * 32 * kRowBytes);
  };
  auto vfrag = [&](const uint8_t* vs, int half, int step) __attribute__((always_inline)) -> bf16x8 {
    const int s2 = step >> 2, db = step & 3;
    const int off = (32 * half + 16 * s2) * kRowBytes;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DITATTN_LDS s16x4*)(vs + va[db] + off));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((DITATTN_LDS s16x4*)(vs + va[db] + off + 4 * kRowBytes));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4,
                                   5, 6, 7);
  };
  // Fragment rings: the fragment of step s sits in slot s % (kPrefetch + 1).
  // A block reads its own fragments kPrefetch steps ahead, and in its last
  // kPrefetch steps the first ones of the block after it (next(i) reads
  // fragment i of that block), so no block starts by waiting on LDS.  The
  // block after a BMM1 block is a BMM2 block and vice versa, so next() never
  // writes a slot of the ring the current block still reads.
  bf16x8 kfr[kPrefetch + 1], vfr[kPrefetch + 1];
  auto kpre = [&](const uint8_t* ks, int kb) __attribute__((always_inline)) {
    return [&kfr, &kfrag, ks, kb](int i) __attribute__((always_inline)) { kfr[i] = kfrag(ks, kb, i); };
  };
  auto vpre = [&](const uint8_t* vs, int half) __attribute__((always_inline)) {
    return [&vfr, &vfrag, vs, half](int i) __attribute__((always_inline)) { vfr[i] = vfrag(vs, half, i); };
  };
  // 16 MFMA slots of BMM1 (half kb of K stage ks into sdst); valu(t) runs after slot t's MFMA.
  auto bmm1_block = [&](const uint8_t* ks, int kb, f32x16 (&sdst)[2], auto&& valu, auto&& next) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int ds = t >> 1, qb = t & 1;
      if (qb == 0 && ds + kPrefetch < 8) kfr[(ds + kPrefetch) % (kPrefetch + 1)] = kfrag(ks, kb, ds + kPrefetch);
      if (qb == 0 && ds + kPrefetch >= 8) next(ds + kPrefetch - 8);
      if (ds == 0) {
        f32x16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0f;
        sdst[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[0], qf[qb][0], z, 0, 0, 0);
      } else {
        sdst[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ds % (kPrefetch + 1)], qf[qb][ds], sdst[qb], 0, 0, 0);
      }
      valu(t);
      fence();
    }
  };
  // 16 MFMA slots of BMM2 (O^T += V^T P^T for half `half` of V stage vs).
  auto bmm2_block = [&](const uint8_t* vs, int half, const bf16x8 (&pin)[2][2], auto&& valu, auto&& next) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int step = t >> 1, qb = t & 1;
      const int s2 = step >> 2, db = step & 3;
      if (qb == 0 && step + kPrefetch < 8) vfr[(step + kPrefetch) % (kPrefetch + 1)] = vfrag(vs, half, step + kPrefetch);
      if (qb == 0 && step + kPrefetch >= 8) next(step + kPrefetch - 8);
      o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[step % (kPrefetch + 1)], pin[s2][qb], o[db][qb], 0, 0, 0);
      if ((t & 3) == 3) {
        const int rq = (t >> 2) & 1, rs = t >> 3;
        rsum[rq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel, pin[rs][rq], rsum[rq], 0, 0, 0);
      }
      valu(t);
      fence();
    }
  };
  // The VALU work of a Q block without its MFMAs (the half before was
  // skipped); it still reads the next block's first fragments.
  auto valu_block = [&](auto&& valu, auto&& next) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if ((t & 1) == 0 && (t >> 1) + kPrefetch >= 8) next((t >> 1) + kPrefetch - 8);
      valu(t);
      fence();
    }
  };
  // Exponential pipeline, pair k (0..15) of a half: qb = k / 8, 16-key step
  // s2 = (k / 4) % 2, register pair k % 4 of that step.
  float ex[3][2];       // pairs in flight, slot k % 3
  auto pair_stage = [&](int stage, const f32x16 (&sv)[2], bf16x8 (&pout)[2][2], int k) __attribute__((always_inline)) {
    const int qb = k >> 3, s2 = (k >> 2) & 1, jp = k & 3;
    float(&x)[2] = ex[k % 3];
    if (stage == 0) {
      x[0] = __builtin_fmaf(sv[qb][8 * s2 + 2 * jp], c, -mref[qb]);
      x[1] = __builtin_fmaf(sv[qb][8 * s2 + 2 * jp + 1], c, -mref[qb]);
      asm volatile("" : "+v"(x[0]), "+v"(x[1]));
    } else if (stage == 1) {
      x[0] = exp2_fast(x[0]);
      x[1] = exp2_fast(x[1]);
      asm volatile("" : "+v"(x[0]), "+v"(x[1]));
    } else {
      i32x4 w = __builtin_bit_cast(i32x4, pout[s2][qb]);
      const bf16x2 pr = {(__bf16)x[0], (__bf16)x[1]};
      int word = __builtin_bit_cast(int, pr);
      asm volatile("" : "+v"(word));
      w[jp] = word;
      pout[s2][qb] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // Row maximum of a half, one step per slot: i = 0..15 (qb = i / 8).
  float mpart[2];
  auto max_stage = [&](const f32x16 (&sv)[2], int i) __attribute__((always_inline)) {
    const int qb = i >> 3, r = i & 7;
    if (r == 0)
      mpart[qb] = max3_raw(sv[qb][0], sv[qb][1], sv[qb][2]);
    else if (r < 7)
      mpart[qb] = max3_raw(mpart[qb], sv[qb][2 * r + 1], sv[qb][2 * r + 2]);
    else
      mpart[qb] = max_raw(mpart[qb], sv[qb][15]);
  };
  // VALU work of a Q block: max step t, and pairs 0..6 at slots 2k (fma), 2k+1 (exp), 2k+2 (pack).
  auto q_valu = [&](const f32x16 (&sv)[2], bf16x8 (&pout)[2][2], int t) __attribute__((always_inline)) {
    max_stage(sv, t);
    if ((t & 1) == 0 && t >= 2) pair_stage(2, sv, pout, (t - 2) >> 1);
    if ((t & 1) == 1) pair_stage(1, sv, pout, (t - 1) >> 1);
    if ((t & 1) == 0 && t <= 12) pair_stage(0, sv, pout, t >> 1);
  };
  // VALU work of a P block: pairs 7..15 with their scale-and-shift at these slots.
  auto p_valu = [&](const f32x16 (&sv)[2], bf16x8 (&pout)[2][2], int t) __attribute__((always_inline)) {
    constexpr int f[9] = {0, 1, 3, 5, 7, 8, 10, 12, 13};
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      if (t == f[i] + 2) pair_stage(2, sv, pout, 7 + i);
      if (t == f[i] + 1) pair_stage(1, sv, pout, 7 + i);
      if (t == f[i]) pair_stage(0, sv, pout, 7 + i);
    }
  };
  // Row maximum in log2 units from the block's partial maxima.
  auto finish_max = [&](float (&mx)[2]) __attribute__((always_inline)) {
    mx[0] = max_halves(mpart[0]) * c;
    mx[1] = max_halves(mpart[1]) * c;
  };
  // Slow path after a Q block whose maximum moved the reference: rescale the
  // running state, then redo pairs 0..6 with the new reference.
  auto redo_q_pairs = [&](const f32x16 (&sv)[2], bf16x8 (&pout)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      pair_stage(0, sv, pout, k);
      pair_stage(1, sv, pout, k);
      pair_stage(2, sv, pout, k);
    }
  };
  // Tail mask of a half starting at key key0 (keys past S_kv take no part).
  auto mask_half = [&](f32x16 (&s)[2], int key0) __attribute__((always_inline)) {
    if (key0 + 32 > Skv) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 16 * (r >> 3) + 8 * hh + (r & 7);
        if (key >= Skv) {
          s[0][r] = kNegInf;
          s[1][r] = kNegInf;
        }
      }
    }
  };
  auto needs_rescale = [&](const float (&mx)[2]) __attribute__((always_inline)) -> bool {
    return __any(mx[0] > mref[0] + kRescaleSlack || mx[1] > mref[1] + kRescaleSlack);
  };
  auto rescale = [&](const float (&mx)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mnew = fmaxf(mref[qb], mx[qb]);
      const float alpha = exp2_fast(mref[qb] - mnew);
      mref[qb] = mnew;
      const float alpha_hi = __shfl(alpha, (lane & 15) + 16, 64);
      rsum[qb][0] *= alpha;
      rsum[qb][1] *= alpha_hi;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
    }
  };
  mref[0] = mref[1] = kNegInf;

  // ---- Prologue: tiles 0..2 in flight.
  issue_loads(IC<0>{}, 0);
  issue_loads(IC<1>{}, 1);
  issue_loads(IC<2>{}, 2);

  float mx0[2], mx1[2];
  f32x16 sb[2][2];       // dense: S^T of two halves in flight, [buffer][qb]
  bf16x8 pb[2][2][2];    // dense: P^T of two halves in flight, [buffer][16-key step][qb]
  // Skip-Softmax state: exact running maxima over kept halves, the
  // wavefront's skipped-half count and its bitmap row.
  // Lanes l and l + 32 hold the same rows, so one register carries both
  // query blocks: lane half 0 the rows of block 0, lane half 1 those of block 1.
  float mrun = kNegInf;
  unsigned skipped = 0;
  const int nvote = (Skv + kSkipBlockN - 1) / kSkipBlockN;
  const bool qv0 = q0 + l32 < Sq, qv1 = q0 + 32 + l32 < Sq;
  uint8_t* bitmap_row = nullptr;
  if (kBitmap && p.bitmap != nullptr && q0 < Sq)
    bitmap_row = p.bitmap + ((int64_t)(b * p.Hq + h) * ((Sq + kSkipBlockM - 1) / kSkipBlockM) + q0 / kSkipBlockM) * nvote;
  // After the Q block of half u: vote (kSkip), then move the reference if a
  // kept half's maximum passed the slack.  Returns whether half u is kept.
  auto q_check = [&](const f32x16 (&sv)[2], bf16x8 (&pout)[2][2], int u) __attribute__((always_inline)) -> bool {
    float mx[2];
    finish_max(mx);
    if constexpr (kSkip) {
      // Past the first half every valid row has a finite running maximum
      // and a finite half maximum, so >= is the negation of <.  The vote is
      // scalar arithmetic on wavefront-uniform values with one branch (on
      // keep): with one wavefront per SIMD every taken branch is lost time.
      // Halves past S_kv hold no keys: not kept, not counted.
      const float mxh = hh ? mx[1] : mx[0];
      const bool hot = (hh ? qv1 : qv0) & (mxh - mrun >= p.log2_lambda);
      const bool in_range = u < nvote;
      const bool keep = in_range & ((u == 0) | __any(hot));
      if constexpr (kBitmap) {
        if (bitmap_row != nullptr && in_range && lane == 0) bitmap_row[u] = keep ? 0 : 1;
      }
      skipped += (unsigned)(in_range & !keep);
      if (!keep) {
        asm volatile("");
        return false;
      }
      // Keeps the compiler from hoisting the next BMM2 block's operand reads
      // above the vote (they would stay live through it).
      asm volatile("" ::: "memory");
      mrun = max_raw(mrun, mxh);
    }
    if (__builtin_expect(needs_rescale(mx), 0)) {   // rare: laid out off the fall-through path
      rescale(mx);
      redo_q_pairs(sv, pout);
    }
    return true;
  };
  bool keep_b[2] = {true, true};   // kept flags of the halves in buffers 0 / 1
  if constexpr (true) {
    // S of half 0 (tile 0), then its Q-block VALU work with no BMM2 to pair with.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoadsPerTile));
    wg_barrier();
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) kpre(sK0, 0)(i);
    // The next block is BMM1 too, on the same K ring: its first fragments
    // are read once this block is done with the ring.
    bmm1_block(sK0, 0, sb[0], [](int) {}, [](int) {});
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) kpre(sK0, 1)(i);
    mask_half(sb[0], 0);
#pragma unroll
    for (int t = 0; t < 16; ++t) q_valu(sb[0], pb[0], t);
    keep_b[0] = q_check(sb[0], pb[0], 0);
  }

  // ---- One KV tile (halves u0 = 2j, u1 = 2j+1): stage S = j % 4 holds tile j.
  // Dense: S(u0) and the Q-block work on it come in from the previous step.
  //   P(u0): BMM1(u1)          || pairs 7-15 of S(u0)
  //   Q(u1): BMM2(u0)          || row max and pairs 0-6 of S(u1), then the check
  //   P(u1): BMM1(tile j+1, 0) || pairs 7-15 of S(u1)
  //   Q(u2): BMM2(u1)          || row max and pairs 0-6 of S(tile j+1, 0), then the check
  // Past the last tile the stages hold zeros and the keys are masked, so the
  // extra BMM1 and Q-block work change nothing.
  auto iteration = [&](auto s_c, int j) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    const uint8_t* ks = kst(IC<S>{});
    const uint8_t* vs = vst(IC<S>{});
    const int key0 = j * kBlockN;
    if constexpr (true) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerTile));   // tile j+1 landed (j+2 may be in flight)
      wg_barrier();
      // Tile j+3 goes into the stage tile j-1 used (every wavefront is past
      // it now): K loads ride in the first block, V loads in the second.
      const uint32_t tk = (uint32_t)(j + 3) * kBlockN * kstride, tv = (uint32_t)(j + 3) * kBlockN * vstride;
      const uint32_t kd = lds_addr(kst(IC<(S + 3) & 3>{}));   // plus wave_slot, added at each load
      const uint32_t vd = lds_addr(vst(IC<(S + 3) & 3>{}));
      bmm1_block(ks, 1, sb[1], [&](int t) __attribute__((always_inline)) {
        p_valu(sb[0], pb[0], t);
        if ((t & 3) == 2) buffer_load_lds16_at(krsrc, wave_slot, kd + 4096 * (t >> 2), koff[t >> 2] + tk);
      }, vpre(vs, 0));
      mask_half(sb[1], key0 + 32);
      auto qv_odd = [&](int t) __attribute__((always_inline)) {
        q_valu(sb[1], pb[1], t);
        if ((t & 3) == 2) buffer_load_lds16_at(vrsrc, wave_slot, vd + 4096 * (t >> 2), voff[t >> 2] + tv);
      };
      if (!kSkip || keep_b[0])
        bmm2_block(vs, 0, pb[0], qv_odd, kpre(kst(IC<(S + 1) & 3>{}), 0));
      else
        valu_block(qv_odd, kpre(kst(IC<(S + 1) & 3>{}), 0));
      keep_b[1] = q_check(sb[1], pb[1], 2 * j + 1);
      bmm1_block(kst(IC<(S + 1) & 3>{}), 0, sb[0], [&](int t) __attribute__((always_inline)) { p_valu(sb[1], pb[1], t); },
                 vpre(vs, 1));
      mask_half(sb[0], key0 + kBlockN);
      auto qv_even = [&](int t) __attribute__((always_inline)) { q_valu(sb[0], pb[0], t); };
      // The next step's first block is BMM1 of the same tile's second half
      // (already resident: the step's barrier does not change that stage).
      if (!kSkip || keep_b[1])
        bmm2_block(vs, 1, pb[1], qv_even, kpre(kst(IC<(S + 1) & 3>{}), 1));
      else
        valu_block(qv_even, kpre(kst(IC<(S + 1) & 3>{}), 1));
      keep_b[0] = q_check(sb[0], pb[0], 2 * j + 2);
    }
  };

  for (int j = 0;; j += 4) {
    iteration(IC<0>{}, j);
    if (j + 1 >= nkt) break;
    iteration(IC<1>{}, j + 1);
    if (j + 2 >= nkt) break;
    iteration(IC<2>{}, j + 2);
    if (j + 3 >= nkt) break;
    iteration(IC<3>{}, j + 3);
    if (j + 4 >= nkt) break;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (kSkip && p.counter != nullptr && lane == 0 && q0 < Sq && skipped)
    atomicAdd(p.counter, (unsigned long long)skipped);

  // ---- Epilogue: O = O^T / l, lane writes 4 consecutive d per register group.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float s_lo = __shfl(rsum[qb][0], l32 & 15, 64), s_hi = __shfl(rsum[qb][1], l32 & 15, 64);
    const float l = l32 < 16 ? s_lo : s_hi;
    const float inv = 1.0f / l;
    const int row = q0 + qb * 32 + l32;
    // LSE = ln(sum_j exp(s_ij)) = (m_ref + log2 l) ln 2, P being 2^(L - m_ref).
    if (p.lse != nullptr && hh == 0 && row < Sq)
      p.lse[((int64_t)b * p.Hq + h) * Sq + row] = (mref[qb] + __log2f(l)) * kLn2;
    if (row < Sq) {
      const int64_t obase = b * p.os[0] + (int64_t)row * p.os[1] + h * p.os[2];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * hh;
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = o[db][qb][4 * gq + j] * inv;
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

__global__ void zero_u64_kernel(unsigned long long* p) {
  if (threadIdx.x == 0) p[threadIdx.x] = 0ull;
}

__global__ void fill_u8_kernel(uint8_t* p, size_t n, uint8_t value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

}  // namespace

hipError_t launch_fmha_bf16(const FmhaBf16Args& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBlockM - 1) / kBlockM;
  const int64_t nwg = nqt * a.Hq * a.B;
  if (nwg <= 0) return hipSuccess;
  hipLaunchKernelGGL((fmha_bf16_kernel<false, false>), dim3((unsigned)nwg), dim3(kDenseWaves * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fmha_bf16_skip(const FmhaBf16Args& a, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBlockM - 1) / kBlockM;
  const int64_t nwg = nqt * a.Hq * a.B;
  if (nwg <= 0) return hipSuccess;
  if (a.bitmap != nullptr)
    hipLaunchKernelGGL((fmha_bf16_kernel<true, true>), dim3((unsigned)nwg), dim3(kDenseWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((fmha_bf16_kernel<true, false>), dim3((unsigned)nwg), dim3(kDenseWaves * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_zero_u64(unsigned long long* p, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fill_u8(uint8_t* p, size_t n, uint8_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

}  // namespace ditattn
