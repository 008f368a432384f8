// C ABI of the library: argument validation, workspace layout and launches.
// Every check runs before anything is enqueued; on failure nothing is launched
// and the thread-local message says why.  No path falls back to another one.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/ditattn.h"
#include "internal.h"

using namespace ditattn;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return ATTN_OK;
}

constexpr int64_t kMaxIndex = (int64_t)1 << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The current device must be a gfx950 part; cached per device ordinal.
int check_device() {
  static std::mutex mu;
  static int known[64] = {0};  // 0 unknown, 1 good, -1 bad
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(ATTN_ERR_DEVICE, "no HIP device is available");
  if (dev >= 64) return fail(ATTN_ERR_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(ATTN_ERR_DEVICE, "cannot query device %d", dev);
    known[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  if (known[dev] < 0) return fail(ATTN_ERR_DEVICE, "device %d is not gfx950", dev);
  return ATTN_OK;
}

// Pointer must be device (or managed) memory of the current device.
int check_device_ptr(const void* p, const char* name) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_INVALID_ARG, "%s is not a HIP device pointer", name);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(ATTN_ERR_INVALID_ARG, "%s is not device memory", name);
  int dev = -1;
  (void)hipGetDevice(&dev);
  if (attr.device != dev) return fail(ATTN_ERR_DEVICE, "%s lives on device %d, current device is %d", name, attr.device, dev);
  return ATTN_OK;
}

int check_shape(const attn_shape* s) {
  if (s == nullptr) return fail(ATTN_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 0 || s->S_q < 0 || s->S_kv < 0 || s->Hq < 0 || s->Hkv < 0)
    return fail(ATTN_ERR_INVALID_ARG, "negative size in shape");
  if (s->D != kHeadDim) return fail(ATTN_ERR_UNSUPPORTED_HEAD_DIM, "head_dim %lld is not 128", (long long)s->D);
  if (s->Hkv == 0 || s->Hq % s->Hkv != 0)
    return fail(ATTN_ERR_BAD_GQA, "Hq=%lld is not a multiple of Hkv=%lld", (long long)s->Hq, (long long)s->Hkv);
  if (s->S_q >= kMaxIndex || s->S_kv >= kMaxIndex || s->B * s->Hq >= kMaxIndex)
    return fail(ATTN_ERR_INVALID_ARG, "problem too large for 32-bit tile indices");
  const int64_t nwg = ((s->S_q + kBlockM - 1) / kBlockM) * s->Hq * s->B;
  if (nwg >= kMaxIndex) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  const int64_t* strides[4] = {s->q_stride, s->k_stride, s->v_stride, s->o_stride};
  const char* names[4] = {"q", "k", "v", "o"};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i) {
      const int64_t st = strides[t][i];
      if (st < 0 || (st & 7) != 0)
        return fail(ATTN_ERR_BAD_LAYOUT, "%s stride[%d]=%lld must be a non-negative multiple of 8 elements",
                    names[t], i, (long long)st);
    }
  // K and V rows must not overlap: the kernels size their buffer views from
  // the row stride (a stride of 0, e.g. a broadcast view, would read zeros).
  if (s->S_kv > 0 && (s->k_stride[1] < kHeadDim || s->v_stride[1] < kHeadDim))
    return fail(ATTN_ERR_BAD_LAYOUT, "k and v stride[1] must be at least 128 elements (rows may not overlap)");
  // O rows must not overlap: sorted by stride, every dimension of size > 1
  // starts past the end of the ones inside it (a row is 128 elements).
  {
    int64_t st[3] = {s->o_stride[0], s->o_stride[1], s->o_stride[2]};
    int64_t sz[3] = {s->B, s->S_q, s->Hq};
    for (int i = 0; i < 3; ++i)
      for (int j = i + 1; j < 3; ++j)
        if (st[j] < st[i]) {
          std::swap(st[i], st[j]);
          std::swap(sz[i], sz[j]);
        }
    int64_t extent = kHeadDim;
    for (int i = 0; i < 3; ++i) {
      if (sz[i] <= 1) continue;
      if (st[i] < extent) return fail(ATTN_ERR_BAD_LAYOUT, "o strides make output rows overlap");
      extent = st[i] * sz[i];
    }
  }
  return ATTN_OK;
}

bool empty(const attn_shape* s) { return s->B == 0 || s->S_q == 0 || s->Hq == 0; }

// The BF16 kernels address one (batch, kv head)'s K and V rows through 32-bit
// buffer offsets, including up to four tiles past the end.
int check_kv_span(const attn_shape* s) {
  const int64_t rows = s->S_kv + 4 * kBlockN;
  if (rows * s->k_stride[1] * 2 >= ((int64_t)1 << 32) || rows * s->v_stride[1] * 2 >= ((int64_t)1 << 32))
    return fail(ATTN_ERR_INVALID_ARG, "K/V span of one head exceeds 4 GiB");
  return ATTN_OK;
}

int check_common(const void* q, const void* k, const void* v, const void* o, attn_dtype o_dtype,
                 const attn_shape* shape, float sm_scale) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (o_dtype != ATTN_DTYPE_BF16 && o_dtype != ATTN_DTYPE_FP32)
    return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be BF16 or FP32");
  if (!(std::isfinite(sm_scale) && sm_scale > 0.0f))
    return fail(ATTN_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (empty(shape)) return ATTN_OK;
  if (shape->S_kv == 0) return fail(ATTN_ERR_INVALID_ARG, "S_kv = 0: softmax over no keys");
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_BAD_LAYOUT, "q, k, v and o must be 16-byte aligned");
  return ATTN_OK;
}

int check_ptrs(const void* q, const void* k, const void* v, const void* o) {
  int rc;
  if ((rc = check_device())) return rc;
  if ((rc = check_device_ptr(q, "q"))) return rc;
  if ((rc = check_device_ptr(k, "k"))) return rc;
  if ((rc = check_device_ptr(v, "v"))) return rc;
  if (o && (rc = check_device_ptr(o, "o"))) return rc;
  return ATTN_OK;
}

// The optional LSE output: 4-byte aligned (checked on the host first), device memory.
int check_lse_align(const float* lse) {
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(ATTN_ERR_BAD_LAYOUT, "lse must be 4-byte aligned");
  return ATTN_OK;
}
int check_lse(const float* lse) { return lse ? check_device_ptr(lse, "lse") : ATTN_OK; }

FmhaBf16Args bf16_args(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype,
                       const attn_shape* s, float sm_scale) {
  FmhaBf16Args a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = s->q_stride[i];
    a.ks[i] = s->k_stride[i];
    a.vs[i] = s->v_stride[i];
    a.os[i] = s->o_stride[i];
  }
  a.B = (int)s->B;
  a.Sq = (int)s->S_q;
  a.Skv = (int)s->S_kv;
  a.Hq = (int)s->Hq;
  a.Hkv = (int)s->Hkv;
  a.sm_scale = sm_scale;
  a.o_fp32 = o_dtype == ATTN_DTYPE_FP32;
  return a;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// The accepted recipes (qk_dtype, v_dtype, (q_block, k_block, v_block)):
//   SageAttention  (INT8 | FP8_E4M3, FP8_E4M3, (1|4|16, 1|4|16, 1))
//   QK16PV8        (BF16, FP8_E4M3, (0, 0, 0))
//   MXFP8 Q/K      (MXFP8, FP8_E4M3, (0, 0, 0|1))
int check_recipe(const attn_recipe* r) {
  if (r == nullptr) return fail(ATTN_ERR_INVALID_ARG, "recipe is NULL");
  if (r->v_dtype != ATTN_DTYPE_FP8_E4M3) return fail(ATTN_ERR_UNSUPPORTED_RECIPE, "v_dtype must be FP8_E4M3");
  if (r->qk_dtype == ATTN_DTYPE_INT8 || r->qk_dtype == ATTN_DTYPE_FP8_E4M3) {
    auto blk_ok = [](int b) { return b == 1 || b == 4 || b == 16; };
    if (!blk_ok(r->q_block) || !blk_ok(r->k_block))
      return fail(ATTN_ERR_UNSUPPORTED_RECIPE, "q_block and k_block must be 1, 4 or 16 (got %d, %d)", r->q_block,
                  r->k_block);
    if (r->v_block != 1) return fail(ATTN_ERR_UNSUPPORTED_RECIPE, "v_block must be 1 (one V scale per channel)");
    return ATTN_OK;
  }
  if (r->qk_dtype == ATTN_DTYPE_BF16) {
    if (r->q_block != 0 || r->k_block != 0 || r->v_block != 0)
      return fail(ATTN_ERR_UNSUPPORTED_RECIPE, "the BF16 Q/K recipe (QK16PV8) takes blocks (0, 0, 0)");
    return ATTN_OK;
  }
  if (r->qk_dtype == ATTN_DTYPE_MXFP8) {
    if (r->q_block != 0 || r->k_block != 0 || (r->v_block != 0 && r->v_block != 1))
      return fail(ATTN_ERR_UNSUPPORTED_RECIPE, "the MXFP8 Q/K recipe takes blocks (0, 0, 0) or (0, 0, 1)");
    return ATTN_OK;
  }
  return fail(ATTN_ERR_UNSUPPORTED_RECIPE, "qk_dtype must be INT8, FP8_E4M3, BF16 or MXFP8");
}

int qk_fmt(const attn_recipe* r) {
  switch (r->qk_dtype) {
    case ATTN_DTYPE_INT8: return kQkInt8;
    case ATTN_DTYPE_FP8_E4M3: return kQkFp8;
    case ATTN_DTYPE_MXFP8: return kQkMxfp8;
    default: return kQkBf16;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

void sage_layout(const attn_shape* s, const attn_recipe* r, attn_sage_layout* L) {
  const int64_t S = s->S_q > s->S_kv ? s->S_q : s->S_kv;
  L->s_pad = (S + kBlockN - 1) / kBlockN * kBlockN;
  const int fmt = qk_fmt(r);
  if (fmt == kQkInt8 || fmt == kQkFp8) {
    L->n_qblk = (s->S_q + r->q_block - 1) / r->q_block;
    L->n_kblk = (s->S_kv + r->k_block - 1) / r->k_block;
  } else if (fmt == kQkMxfp8) {   // one 4-byte word of E8M0 scales per token row
    L->n_qblk = L->s_pad;
    L->n_kblk = L->s_pad;
  } else {                        // BF16 Q/K: no codes, no scales
    L->n_qblk = 0;
    L->n_kblk = 0;
  }
  const int64_t code_rows = fmt == kQkBf16 ? 0 : L->s_pad;
  const int64_t nchunks = (s->S_kv + kMeanChunk - 1) / kMeanChunk;
  size_t off = 0;
  L->q_codes_off = off;
  off = align256(off + (size_t)(s->B * s->Hq * code_rows * kHeadDim));
  L->k_codes_off = off;
  off = align256(off + (size_t)(s->B * s->Hkv * code_rows * kHeadDim));
  L->v_codes_off = off;
  off = align256(off + (size_t)(s->B * s->Hkv * L->s_pad * kHeadDim));
  L->q_scale_off = off;
  off = align256(off + sizeof(float) * (size_t)(s->B * s->Hq * L->n_qblk));
  L->k_scale_off = off;
  off = align256(off + sizeof(float) * (size_t)(s->B * s->Hkv * L->n_kblk));
  L->v_scale_off = off;
  off = align256(off + sizeof(float) * (size_t)(s->B * s->Hkv * kHeadDim));
  L->k_mean_off = off;
  off = align256(off + sizeof(float) * (size_t)(s->B * s->Hkv * kHeadDim));
  L->scratch_off = off;
  off = align256(off + sizeof(float) * (size_t)(s->B * s->Hkv * nchunks * kHeadDim));
  off = align256(off + sizeof(unsigned) * (size_t)(s->B * s->Hkv * kHeadDim));
  L->total_bytes = off;
}

// ws must hold the layout's total_bytes, or only its first scratch_off bytes
// when the statistics live elsewhere (stats_in_ws false).
int check_sage(const void* q, const void* k, const void* v, const attn_shape* shape, const attn_recipe* recipe,
               void* ws, size_t ws_bytes, attn_sage_layout* L, bool stats_in_ws = true) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_recipe(recipe))) return rc;
  sage_layout(shape, recipe, L);
  if (empty(shape) && shape->S_kv == 0) return ATTN_OK;
  // The low-precision kernel addresses one head's codes (and, for BF16 Q/K,
  // its K rows) through 32-bit buffer offsets, including tiles past the end.
  if ((L->s_pad + 4 * kBlockN) * kHeadDim >= ((int64_t)1 << 32))
    return fail(ATTN_ERR_INVALID_ARG, "codes of one head exceed 4 GiB (S too large)");
  if (qk_fmt(recipe) == kQkBf16 && (shape->S_kv + 4 * kBlockN) * shape->k_stride[1] * 2 >= ((int64_t)1 << 32))
    return fail(ATTN_ERR_INVALID_ARG, "K span of one head exceeds 4 GiB");
  if (!q || !k || !v) return fail(ATTN_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(ATTN_ERR_BAD_LAYOUT, "q, k, v must be 16-byte aligned");
  if (ws == nullptr) return fail(ATTN_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(ATTN_ERR_BAD_LAYOUT, "workspace must be 256-byte aligned");
  const size_t need = stats_in_ws ? L->total_bytes : L->scratch_off;
  if (ws_bytes < need)
    return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace holds %zu bytes, %zu needed", ws_bytes, need);
  return ATTN_OK;
}

// Bytes of the quantizer's statistics (K chunk sums, then V channel maxima).
size_t stats_bytes(const attn_shape* s) {
  const int64_t nchunks = (s->S_kv + kMeanChunk - 1) / kMeanChunk;
  return align256(sizeof(float) * (size_t)(s->B * s->Hkv * nchunks * kHeadDim)) +
         align256(sizeof(unsigned) * (size_t)(s->B * s->Hkv * kHeadDim));
}

// The statistics scratch of sage_quantize_noalloc: one array per device,
// held until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, resolved once per device with that device current.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
__device__ __align__(256) static unsigned char scratch[kStaticScratchBytes];

int static_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(ATTN_ERR_DEVICE, "no HIP device is available");
  if (dev >= 64) return fail(ATTN_ERR_DEVICE, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(ATTN_ERR_DEVICE, "cannot resolve the static scratch array on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return ATTN_OK;
}

// Quantizer arguments for the outputs in ws; the statistics go to `stats`
// (a region of stats_bytes) or, when it is NULL, to ws at the layout's
// scratch offset.
SageQuantArgs quant_args(const void* q, const void* k, const void* v, const attn_shape* s, const attn_recipe* r,
                         void* ws, const attn_sage_layout& L, void* stats = nullptr) {
  SageQuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = s->q_stride[i];
    a.ks[i] = s->k_stride[i];
    a.vs[i] = s->v_stride[i];
  }
  a.B = (int)s->B;
  a.Sq = (int)s->S_q;
  a.Skv = (int)s->S_kv;
  a.Hq = (int)s->Hq;
  a.Hkv = (int)s->Hkv;
  a.qk_fmt = qk_fmt(r);
  a.smooth = a.qk_fmt == kQkInt8 || a.qk_fmt == kQkFp8;
  a.v_tensor = r->v_block == 0;
  a.q_block = r->q_block;
  a.k_block = r->k_block;
  a.s_pad = L.s_pad;
  a.n_qblk = L.n_qblk;
  a.n_kblk = L.n_kblk;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.q_codes = w + L.q_codes_off;
  a.k_codes = w + L.k_codes_off;
  a.v_codes = w + L.v_codes_off;
  a.q_scale = reinterpret_cast<float*>(w + L.q_scale_off);
  a.k_scale = reinterpret_cast<float*>(w + L.k_scale_off);
  a.v_scale = reinterpret_cast<float*>(w + L.v_scale_off);
  a.k_mean = reinterpret_cast<float*>(w + L.k_mean_off);
  uint8_t* st = stats != nullptr ? static_cast<uint8_t*>(stats) : w + L.scratch_off;
  const int64_t nchunks = (s->S_kv + kMeanChunk - 1) / kMeanChunk;
  a.k_partial = reinterpret_cast<float*>(st);
  a.v_absmax = reinterpret_cast<unsigned*>(st + align256(sizeof(float) * (size_t)(s->B * s->Hkv * nchunks * kHeadDim)));
  a.q_mx = w + L.q_scale_off;
  a.k_mx = w + L.k_scale_off;
  return a;
}

// SAGE attention, with the Skip-Softmax tile test when threshold_factor > 0:
// quantize into ws, then one attention launch.
int run_sage(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype, const attn_shape* shape,
             const attn_recipe* recipe, float sm_scale, float threshold_factor, uint8_t* skip_bitmap,
             uint64_t* skipped_tiles, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_common(q, k, v, o, o_dtype, shape, sm_scale);
  if (rc) return rc;
  attn_sage_layout L;
  if ((rc = check_recipe(recipe))) return rc;
  if (empty(shape)) return ok();
  if ((rc = check_sage(q, k, v, shape, recipe, ws, ws_bytes, &L))) return rc;
  if ((rc = check_ptrs(q, k, v, o))) return rc;
  if ((rc = check_device_ptr(ws, "workspace"))) return rc;
  if (skip_bitmap && (rc = check_device_ptr(skip_bitmap, "skip_bitmap"))) return rc;
  if (skipped_tiles) {
    if ((reinterpret_cast<uintptr_t>(skipped_tiles) & 7u) != 0)
      return fail(ATTN_ERR_BAD_LAYOUT, "skipped_tiles must be 8-byte aligned");
    if ((rc = check_device_ptr(skipped_tiles, "skipped_tiles"))) return rc;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SageQuantArgs qa = quant_args(q, k, v, shape, recipe, ws, L);
  if ((rc = launched(launch_sage_quantize(qa, st), "SAGE quantization"))) return rc;
  FmhaSageArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_codes = qa.q_codes;
  a.k_codes = qa.k_codes;
  a.v_codes = qa.v_codes;
  a.q_scale = qa.q_scale;
  a.k_scale = qa.k_scale;
  a.v_scale = qa.v_scale;
  a.o = o;
  for (int i = 0; i < 3; ++i) a.os[i] = shape->o_stride[i];
  a.B = qa.B;
  a.Sq = qa.Sq;
  a.Skv = qa.Skv;
  a.Hq = qa.Hq;
  a.Hkv = qa.Hkv;
  a.s_pad = L.s_pad;
  a.n_qblk = L.n_qblk;
  a.n_kblk = L.n_kblk;
  a.q_block = recipe->q_block;
  a.k_block = recipe->k_block;
  a.qk_fmt = qa.qk_fmt;
  a.q_mx = qa.q_mx;
  a.k_mx = qa.k_mx;
  a.q = q;
  a.k = k;
  for (int i = 0; i < 3; ++i) {
    a.qs[i] = shape->q_stride[i];
    a.ks[i] = shape->k_stride[i];
  }
  a.sm_scale = sm_scale;
  a.o_fp32 = o_dtype == ATTN_DTYPE_FP32;
  unsigned long long* counter = reinterpret_cast<unsigned long long*>(skipped_tiles);
  if (counter && (rc = launched(launch_zero_u64(counter, st), "counter reset"))) return rc;
  if (threshold_factor > 0.0f) {
    a.skip = 1;
    a.log2_lambda = (float)std::log2((double)threshold_factor / (double)shape->S_kv);
    a.bitmap = skip_bitmap;
    a.counter = counter;
  } else if (skip_bitmap) {
    // lambda = 0: nothing can be skipped; the plain SAGE kernel runs.
    const int64_t nqb = (shape->S_q + kWaveRows - 1) / kWaveRows;
    const int64_t nkt = (shape->S_kv + kBlockN - 1) / kBlockN;
    const size_t n = (size_t)(shape->B * shape->Hq * nqb * nkt);
    if ((rc = launched(launch_fill_u8(skip_bitmap, n, 0, st), "bitmap clear"))) return rc;
  }
  return launched(launch_fmha_sage(a, st), a.skip ? "SAGE skip-softmax attention" : "SAGE attention");
}

}  // namespace

extern "C" {

int attn_version(void) { return 100; }

const char* attn_last_error(void) { return g_err; }

int attn_tile_config(int* block_m, int* block_n, int* kv_tile, int* sage_block_m) {
  if (!block_m || !block_n || !kv_tile || !sage_block_m) return fail(ATTN_ERR_INVALID_ARG, "NULL output pointer");
  *block_m = kSkipBlockM;
  *block_n = kSkipBlockN;
  *kv_tile = kBlockN;
  *sage_block_m = kWaveRows;
  return ok();
}

int attn_skip_gate(float t, float disabled_until_timestep, int* enabled) {
  if (!enabled) return fail(ATTN_ERR_INVALID_ARG, "NULL output pointer");
  if (!(std::isfinite(t) && t >= 0.0f && t <= 1.0f))
    return fail(ATTN_ERR_INVALID_ARG, "timestep must be finite and in [0, 1]");
  if (!(std::isfinite(disabled_until_timestep) && disabled_until_timestep >= 0.0f && disabled_until_timestep <= 1.0f))
    return fail(ATTN_ERR_INVALID_ARG, "disabled_until_timestep must be finite and in [0, 1]");
  *enabled = t <= disabled_until_timestep ? 1 : 0;
  return ok();
}

int attn_dense_bf16(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype,
                    const attn_shape* shape, float sm_scale, float* lse, void* stream) {
  int rc = check_common(q, k, v, o, o_dtype, shape, sm_scale);
  if (rc) return rc;
  if (empty(shape)) return ok();
  if ((rc = check_kv_span(shape))) return rc;
  if ((rc = check_lse_align(lse))) return rc;
  if ((rc = check_ptrs(q, k, v, o))) return rc;
  if ((rc = check_lse(lse))) return rc;
  FmhaBf16Args a = bf16_args(q, k, v, o, o_dtype, shape, sm_scale);
  a.lse = lse;
  return launched(launch_fmha_bf16(a, static_cast<hipStream_t>(stream)), "dense attention");
}

int attn_skip_softmax(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype,
                      const attn_shape* shape, float sm_scale, float threshold_factor, uint8_t* skip_bitmap,
                      uint64_t* skipped_tiles, float* lse, void* stream) {
  int rc = check_common(q, k, v, o, o_dtype, shape, sm_scale);
  if (rc) return rc;
  if (!(std::isfinite(threshold_factor) && threshold_factor >= 0.0f))
    return fail(ATTN_ERR_BAD_THRESHOLD, "threshold factor must be finite and >= 0");
  if (empty(shape)) return ok();
  if ((rc = check_kv_span(shape))) return rc;
  if ((rc = check_lse_align(lse))) return rc;
  if ((rc = check_ptrs(q, k, v, o))) return rc;
  if (skip_bitmap && (rc = check_device_ptr(skip_bitmap, "skip_bitmap"))) return rc;
  if (skipped_tiles) {
    if ((reinterpret_cast<uintptr_t>(skipped_tiles) & 7u) != 0)
      return fail(ATTN_ERR_BAD_LAYOUT, "skipped_tiles must be 8-byte aligned");
    if ((rc = check_device_ptr(skipped_tiles, "skipped_tiles"))) return rc;
  }
  if ((rc = check_lse(lse))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  FmhaBf16Args a = bf16_args(q, k, v, o, o_dtype, shape, sm_scale);
  a.lse = lse;
  unsigned long long* counter = reinterpret_cast<unsigned long long*>(skipped_tiles);
  if (counter && (rc = launched(launch_zero_u64(counter, st), "counter reset"))) return rc;
  if (threshold_factor == 0.0f) {
    // lambda = 0: nothing can be skipped; run the dense kernel itself.
    if (skip_bitmap) {
      const int64_t nqb = (shape->S_q + kSkipBlockM - 1) / kSkipBlockM;
      const int64_t nkt = (shape->S_kv + kSkipBlockN - 1) / kSkipBlockN;
      const size_t n = (size_t)(shape->B * shape->Hq * nqb * nkt);
      if ((rc = launched(launch_fill_u8(skip_bitmap, n, 0, st), "bitmap clear"))) return rc;
    }
    return launched(launch_fmha_bf16(a, st), "dense attention");
  }
  a.log2_lambda = (float)std::log2((double)threshold_factor / (double)shape->S_kv);
  a.bitmap = skip_bitmap;
  a.counter = counter;
  return launched(launch_fmha_bf16_skip(a, st), "skip-softmax attention");
}

int attn_sage_layout_query(const attn_shape* shape, const attn_recipe* recipe, attn_sage_layout* out) {
  if (!out) return fail(ATTN_ERR_INVALID_ARG, "NULL output pointer");
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_recipe(recipe))) return rc;
  sage_layout(shape, recipe, out);
  return ok();
}

int sage_quantize(const void* q, const void* k, const void* v, const attn_shape* shape, const attn_recipe* recipe,
                  void* ws, size_t ws_bytes, void* stream) {
  attn_sage_layout L;
  int rc = check_sage(q, k, v, shape, recipe, ws, ws_bytes, &L);
  if (rc) return rc;
  if (shape->B == 0 || (shape->S_q == 0 && shape->S_kv == 0) || shape->Hq == 0) return ok();
  if ((rc = check_ptrs(q, k, v, nullptr))) return rc;
  if ((rc = check_device_ptr(ws, "workspace"))) return rc;
  const SageQuantArgs a = quant_args(q, k, v, shape, recipe, ws, L);
  return launched(launch_sage_quantize(a, static_cast<hipStream_t>(stream)), "SAGE quantization");
}

int sage_quantize_noalloc(const void* q, const void* k, const void* v, const attn_shape* shape,
                          const attn_recipe* recipe, void* out, size_t out_bytes, void* stream) {
  attn_sage_layout L;
  int rc = check_sage(q, k, v, shape, recipe, out, out_bytes, &L, false);
  if (rc) return rc;
  if (shape->B == 0 || (shape->S_q == 0 && shape->S_kv == 0) || shape->Hq == 0) return ok();
  const size_t need = stats_bytes(shape);
  if (need > kStaticScratchBytes)
    return fail(ATTN_ERR_WORKSPACE_TOO_SMALL,
                "the statistics of this problem take %zu bytes, more than the %zu-byte static scratch "
                "(B * Hkv * ceil(S_kv / 256) must stay below about %zu)",
                need, kStaticScratchBytes, kStaticScratchBytes / (kHeadDim * sizeof(float)) - 1);
  if ((rc = check_ptrs(q, k, v, nullptr))) return rc;
  if ((rc = check_device_ptr(out, "out"))) return rc;
  void* stats = nullptr;
  if ((rc = static_scratch(&stats))) return rc;
  const SageQuantArgs a = quant_args(q, k, v, shape, recipe, out, L, stats);
  return launched(launch_sage_quantize(a, static_cast<hipStream_t>(stream)), "SAGE quantization");
}

int attn_sage(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype, const attn_shape* shape,
              const attn_recipe* recipe, float sm_scale, void* ws, size_t ws_bytes, void* stream) {
  return run_sage(q, k, v, o, o_dtype, shape, recipe, sm_scale, 0.0f, nullptr, nullptr, ws, ws_bytes, stream);
}

int attn_sage_skip_softmax(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype,
                           const attn_shape* shape, const attn_recipe* recipe, float sm_scale,
                           float threshold_factor, uint8_t* skip_bitmap, uint64_t* skipped_tiles, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!(std::isfinite(threshold_factor) && threshold_factor >= 0.0f))
    return fail(ATTN_ERR_BAD_THRESHOLD, "threshold factor must be finite and >= 0");
  return run_sage(q, k, v, o, o_dtype, shape, recipe, sm_scale, threshold_factor, skip_bitmap, skipped_tiles, ws,
                  ws_bytes, stream);
}

}  // extern "C"
