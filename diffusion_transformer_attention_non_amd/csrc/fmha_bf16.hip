// Dense and Skip-Softmax BF16 attention for gfx950.
//
// Fused multi-head attention O = softmax(sm_scale * Q K^T) V, full context,
// non-causal ("TRTLLM Attention", section "Dense mode"), with the optional
// Skip-Softmax tile test ("TRTLLM Attention", section "Skip-Softmax"; the
// threshold factor / seqlen of the knob table in "SAGE + Skip-Softmax - API
// Design & Test Plan", Part 1 section 4).
//
// Work decomposition
//   workgroup = 4 wavefronts = 256 query rows of one (batch, query head);
//   each wavefront owns 64 query rows and walks all KV tiles of 64 keys.
//   Per tile and wavefront:
//     BMM1  S^T[key, query] = K Q^T   32 x v_mfma_f32_32x32x16_bf16
//           (A = K from LDS, B = Q kept in registers for the whole kernel);
//     softmax on S^T: each lane holds one query column of each 32x32 block,
//           so the row maximum is an in-lane max plus one v_permlane32_swap;
//     BMM2  O^T[d, query] += V^T P^T   32 x v_mfma_f32_32x32x16_bf16
//           (A = V^T read with ds_read_b64_tr_b16 from row-major V in LDS,
//           B = P^T straight from the softmax registers).
//   Computing the transposed products keeps each query in one lane, so the
//   softmax state (max, sum, rescale factor) never leaves the lane.
//
// Online softmax with a lazy reference maximum: exponentials are taken
// relative to a per-row reference m_ref (log2 units) that is raised only when
// a tile's maximum exceeds it by more than 8, so P <= 2^8 and the O rescale
// runs only when some row's maximum grows that much.  Softmax is invariant to
// the reference, so the result is the same up to rounding.
//
// Skip-Softmax (kSkip): after BMM1 of tile t > 0, the wavefront skips the tile
// (no exponentials, no BMM2) when every valid row i of its 64 rows has
// exp(M_it - m_i) < lambda, M_it being the row's tile maximum and m_i the
// running maximum over the tiles kept so far; lambda = factor / S_kv.
#include "device_common.h"
#include "internal.h"

namespace ditattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;   // log2 headroom before the reference max moves

// LDS layout of one pipeline stage (bf16 elements):
//   K tile: 64 rows x 128 (+8 pad), rows stored in MFMA-row order (see
//           kv_row_of_key), 272-byte stride: the 8 lanes of a ds_read_b128
//           phase read 8 consecutive rows and land in 8 distinct 16-byte banks.
//   V tile: 64 keys x 128 (+16 pad) row-major, 288-byte stride: the 16 lanes
//           of a ds_read_b64_tr_b16 phase read 4 rows x 32 bytes that cover
//           the 128 bank bytes exactly once.
constexpr int kKRow = 136;
constexpr int kVRow = 144;
constexpr int kKTile = kBlockN * kKRow;
constexpr int kVTile = kBlockN * kVRow;
constexpr int kStage = kKTile + kVTile;

// Accumulator register r of lane half h in a 32x32 S^T block holds MFMA row
// 8*(r/4) + 4*h + r%4.  Reading K row "key(i)" for MFMA row i with
//   key(8a + 4h + b) = 16*(a/2) + 8*h + 4*(a%2) + b
// makes register r of lane half h hold key 16*(r/8) + 8*h + r%8, i.e. each
// lane half holds runs of 8 consecutive keys: exactly the B-operand slots of
// the BMM2 MFMA (8 consecutive k per lane half).  This maps a key to its row.
__device__ __forceinline__ int kv_row_of_key(int k) {
  const int a = 2 * (k >> 4) + ((k >> 2) & 1);
  return 8 * a + 4 * ((k >> 3) & 1) + (k & 3);
}

template <bool kSkip>
__global__ __launch_bounds__(256, 1) void fmha_bf16_kernel(FmhaBf16Args p) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * kStage];

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

  // Q fragments, B operand of BMM1: lane (query l32 of block qb, half hh)
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

  // Global -> LDS loader: thread covers rows 16*i + tid/16 (i = 0..3) of the
  // tile, 16-byte chunk tid % 16.
  const bf16_t* kg = static_cast<const bf16_t*>(p.k) + b * p.ks[0] + g * p.ks[2];
  const bf16_t* vg = static_cast<const bf16_t*>(p.v) + b * p.vs[0] + g * p.vs[2];
  const int lrow = tid >> 4, lchunk = tid & 15;
  int k_dst[4], v_dst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + lrow;
    k_dst[i] = (32 * (r >> 5) + kv_row_of_key(r & 31)) * kKRow + 8 * lchunk;
    v_dst[i] = kKTile + r * kVRow + 8 * lchunk;
  }
  uint4 kreg[4], vreg[4];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = t * kBlockN + 16 * i + lrow;
      const bool ok = key < Skv;
      const int64_t kk = ok ? key : 0;
      kreg[i] = ok ? ldg16(kg + kk * p.ks[1] + 8 * lchunk) : make_uint4(0, 0, 0, 0);
      vreg[i] = ok ? ldg16(vg + kk * p.vs[1] + 8 * lchunk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    bf16_t* base = smem + stage * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(base + k_dst[i]) = kreg[i];
      *reinterpret_cast<uint4*>(base + v_dst[i]) = vreg[i];
    }
  };

  // Lane-dependent parts of the LDS read addresses.
  const int ka_lane = l32 * kKRow + 8 * hh;
  const int r16 = lane & 15;
  const int va_lane = kKTile + (8 * hh + (r16 >> 2)) * kVRow + 16 * ((lane >> 4) & 1) + 4 * (r16 & 3);

  f32x16 o[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.0f;

  const float c = p.sm_scale * kLog2e;
  float mref[2] = {kNegInf, kNegInf};
  float mrun[2] = {kNegInf, kNegInf};
  float lsum[2] = {0.0f, 0.0f};
  const bool qvalid0 = q0 + l32 < Sq, qvalid1 = q0 + 32 + l32 < Sq;
  unsigned skipped = 0;
  const int nkt = (Skv + kBlockN - 1) / kBlockN;
  const int nqb = (Sq + kWaveRows - 1) / kWaveRows;
  uint8_t* bitmap_row = nullptr;
  if (kSkip && p.bitmap != nullptr && q0 < Sq)
    bitmap_row = p.bitmap + ((int64_t)(b * p.Hq + h) * nqb + q0 / kWaveRows) * nkt;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < nkt; ++t) {
    const bf16_t* st = smem + (t & 1) * kStage;
    if (t + 1 < nkt) gload(t + 1);

    // ---- BMM1: S^T = K Q^T over d = 128 (8 steps of 16).
    f32x16 s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + ka_lane + kb * 32 * kKRow + 16 * ds);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }

    // Keys past S_kv in the last tile take no part.
    if ((t + 1) * kBlockN > Skv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * kBlockN + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (key >= Skv) {
            s[kb][0][r] = kNegInf;
            s[kb][1][r] = kNegInf;
          }
        }
    }

    // ---- Tile maximum per query (log2 units).
    float mx[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[kb][qb][r]);
      mx[qb] = max_halves(m) * c;
    }

    bool keep = true;
    if (kSkip) {
      const bool need = (qvalid0 && !(mx[0] - mrun[0] < p.log2_lambda)) ||
                        (qvalid1 && !(mx[1] - mrun[1] < p.log2_lambda));
      keep = (t == 0) || __any(need);
      if (keep) {
        mrun[0] = fmaxf(mrun[0], mx[0]);
        mrun[1] = fmaxf(mrun[1], mx[1]);
      } else {
        ++skipped;
      }
      if (bitmap_row != nullptr && lane == 0) bitmap_row[t] = keep ? 0 : 1;
    }

    if (keep) {
      // ---- Lazy rescale of the running state.
      if (__any(mx[0] > mref[0] + kRescaleSlack || mx[1] > mref[1] + kRescaleSlack)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float mnew = fmaxf(mref[qb], mx[qb]);
          const float alpha = exp2_fast(mref[qb] - mnew);
          mref[qb] = mnew;
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
        }
      }

      // ---- P = exp2(s * c - m_ref), packed to bf16 as the BMM2 B operand.
      bf16x8 pf[2][2][2];  // [kb][16-key step][qb]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float nb = -mref[qb];
        float part = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            f32x8 e;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              e[j] = exp2_fast(__builtin_fmaf(s[kb][qb][8 * s2 + j], c, nb));
              part += e[j];
            }
            pf[kb][s2][qb] = __builtin_convertvector(e, bf16x8);
          }
        lsum[qb] += part;
      }

      // ---- BMM2: O^T += V^T P^T over the tile's 64 keys (4 steps of 16).
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int off = va_lane + (32 * kb + 16 * s2) * kVRow + 32 * db;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (DITATTN_LDS s16x4*)(st + off));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (DITATTN_LDS s16x4*)(st + off + 4 * kVRow));
            const bf16x4 lo_b = __builtin_bit_cast(bf16x4, lo);
            const bf16x4 hi_b = __builtin_bit_cast(bf16x4, hi);
            const bf16x8 a = __builtin_shufflevector(lo_b, hi_b, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][s2][qb], o[db][qb], 0, 0, 0);
          }
    }

    if (t + 1 < nkt) lstore((t + 1) & 1);
    __syncthreads();
  }

  if (kSkip && p.counter != nullptr && lane == 0 && q0 < Sq && skipped)
    atomicAdd(p.counter, (unsigned long long)skipped);

  // ---- Epilogue: O = O^T / l, lane writes 4 consecutive d per register group.
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

hipError_t launch_fmha_bf16(const FmhaBf16Args& a, bool skip, hipStream_t stream) {
  const int64_t nqt = (a.Sq + kBlockM - 1) / kBlockM;
  const int64_t nwg = nqt * a.Hq * a.B;
  if (nwg <= 0) return hipSuccess;
  if (skip)
    hipLaunchKernelGGL(fmha_bf16_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fmha_bf16_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, stream, a);
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
