/*
 * ditattn: full-context, non-causal fused multi-head attention for diffusion
 * transformers on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operations follow these pages (titles as published):
 *   [TA]  "TRTLLM Attention" (vllm-omni user guide): "Requirements",
 *         "Dense mode", "Skip-Softmax", "SAGE quantization".
 *   [DAB] "Diffusion Attention Backends" (vllm-omni user guide): backend
 *         table ("BF16, GQA native, head_dim=128"), "TRTLLM_ATTN Backend and
 *         Skip-Softmax", "TRTLLM_ATTN SAGE Quantization".
 *   [SSD] "SAGE + Skip-Softmax - API Design & Test Plan": Part 1 section 4,
 *         the knob to kernel-argument table (sage_block_sizes=(q,k,v),
 *         bmm1_scale/bmm2_scale, threshold = factor / seqlen, the timestep
 *         gate being host-side with no kernel argument).
 *   [VQA] "VisualGen Quantized Attention (Beta)": "Recipes" (the recipe tuple
 *         (qk_dtype, v_dtype, (q_block_size, k_block_size, v_block_size))) and
 *         "SageAttention in the TRTLLM backend" (one scale per token block per
 *         head for Q/K; one scale per head per channel for V).
 *
 * Conventions shared by every entry point
 *   - Every call returns an int status: ATTN_OK (0) or a negative attn_status.
 *     All arguments are validated before anything is launched; an invalid
 *     call launches nothing and never falls back to another path.
 *     attn_last_error() gives a message for the calling thread's last failure.
 *   - Ownership: the caller allocates and owns every buffer.  The library
 *     never allocates, frees or synchronizes device memory; all work is
 *     enqueued asynchronously on the caller's stream (`stream`, a
 *     hipStream_t; NULL = the default stream).  Pointers marked "device" must
 *     be device memory of the current device, 16-byte aligned.
 *   - Layout: Q is [B, S_q, Hq, D], K and V are [B, S_kv, Hkv, D], O is
 *     [B, S_q, Hq, D], each with arbitrary element strides for (b, s, h) given
 *     in attn_shape and a contiguous d axis.  Strides must be multiples of 8
 *     elements (16 bytes); K and V rows may not overlap (stride[1] >= 128
 *     elements) and neither may the rows of O (BAD_LAYOUT otherwise; Q may
 *     be any read-only view).  D must be 128 ([TA] "Requirements").  Query head
 *     h reads KV head h / (Hq / Hkv) ("GQA native", [DAB] backend table).
 *   - Attention is full-context and non-causal; there is no mask argument
 *     ([TA] "Requirements": a packed or mask-free path).
 *   - Size limits (INVALID_ARG beyond them, checked before any device call):
 *     S_q, S_kv and B * Hq below 2^31 and fewer than 2^31 workgroups; the
 *     kernels address one (batch, kv head)'s rows through 32-bit byte
 *     offsets, so (S_kv + 256) * k_stride[1] * 2 and the same for v_stride
 *     must stay below 4 GiB on the BF16 paths (with packed QKV of 40 heads,
 *     S_kv up to about 139,000), and for the quantized paths the padded
 *     sequence (S rounded up to 64, plus 256) times 128 bytes as well
 *     (S up to about 33.5 million).
 *   - Calls that run on the same stream are ordered; concurrent calls on
 *     different streams that share an output buffer or workspace race.
 */
#ifndef DITATTN_H
#define DITATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,          /* null pointer, negative size, bad enum */
  ATTN_ERR_UNSUPPORTED_HEAD_DIM = -2, /* D != 128 */
  ATTN_ERR_BAD_GQA = -3,              /* Hq % Hkv != 0 */
  ATTN_ERR_UNSUPPORTED_RECIPE = -4,   /* recipe outside the accepted set */
  ATTN_ERR_BAD_LAYOUT = -5,           /* stride or alignment not supported */
  ATTN_ERR_BAD_THRESHOLD = -6,        /* factor not finite or negative */
  ATTN_ERR_WORKSPACE_TOO_SMALL = -7,
  ATTN_ERR_DEVICE = -8,               /* no device, wrong device, launch failure */
  ATTN_ERR_NOT_IMPLEMENTED = -9
} attn_status;

typedef enum {
  ATTN_DTYPE_BF16 = 0,
  ATTN_DTYPE_FP32 = 1,
  ATTN_DTYPE_INT8 = 2,
  ATTN_DTYPE_FP8_E4M3 = 3,            /* OCP OFP8 E4M3 */
  ATTN_DTYPE_MXFP8 = 4                /* OCP MX: E4M3 elements, E8M0 scale per 32 */
} attn_dtype;

/* Problem shape and strides (in elements).  stride[0..2] = b, s, h. */
typedef struct {
  int64_t B, S_q, S_kv, Hq, Hkv, D;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
} attn_shape;

/* Low-precision attention recipe ([VQA] "Recipes": the tuple (qk_dtype,
 * v_dtype, (q_block, k_block, v_block))).  Accepted:
 *   SageAttention  qk_dtype INT8 or FP8_E4M3, q_block and k_block in
 *                  {1, 4, 16} tokens ([TA], [DAB] key tables), v_block = 1
 *                  (one V scale per head per channel, [VQA]);
 *   QK16PV8        qk_dtype BF16, blocks (0, 0, 0): Q/K stay BF16, V in
 *                  E4M3 with one tensor-wide scale ([VQA] "QK16PV8 Attention
 *                  Kernels in the CUTEDSL Backend");
 *   MXFP8 Q/K      qk_dtype MXFP8, blocks (0, 0, 0) or (0, 0, 1): Q/K in OCP
 *                  MXFP8 along the head dimension, V in E4M3 with a
 *                  tensor-wide (0) or per-channel (1) scale ([VQA] "MXFP8
 *                  and NVFP4 in the CUTEDSL and FlashInfer backends").
 * v_dtype is FP8_E4M3 for all. */
typedef struct {
  attn_dtype qk_dtype;
  attn_dtype v_dtype;
  int32_t q_block;
  int32_t k_block;
  int32_t v_block;
} attn_recipe;

/* Where sage_quantize puts each quantized tensor inside the workspace (byte
 * offsets from ws) and how the tensors are laid out:
 *   q_codes  [B, Hq,  s_pad, 128]  int8 or E4M3 bytes (token rows >= S_q are 0)
 *   k_codes  [B, Hkv, s_pad, 128]  codes of K - mean (rows >= S_kv are 0)
 *   v_codes  [B, Hkv, 128, s_pad]  E4M3 bytes, transposed (d-major)
 *   q_scale  [B, Hq,  n_qblk]      fp32, n_qblk = ceil(S_q / q_block)
 *   k_scale  [B, Hkv, n_kblk]      fp32, n_kblk = ceil(S_kv / k_block)
 *   v_scale  [B, Hkv, 128]         fp32 (all equal for a tensor-wide scale)
 *   k_mean   [B, Hkv, 128]         fp32 (the K-smoothing mean; 0 when the
 *                                  recipe does not smooth)
 * s_pad is max(S_q, S_kv) rounded up to a multiple of 64.  MXFP8: q_codes
 * and k_codes hold E4M3 codes of Q and K (no smoothing), and the q_scale /
 * k_scale regions hold [B, H, s_pad, 4] E8M0 bytes (byte c scales channels
 * 32 c..32 c + 31 by 2^(byte - 127); n_qblk = n_kblk = s_pad).  BF16
 * (QK16PV8): the code and scale regions of Q and K are empty (n_qblk =
 * n_kblk = 0). */
typedef struct {
  size_t total_bytes;
  size_t q_codes_off, k_codes_off, v_codes_off;
  size_t q_scale_off, k_scale_off, v_scale_off, k_mean_off, scratch_off;
  int64_t s_pad, n_qblk, n_kblk;
} attn_sage_layout;

/* Dense BF16 attention ([TA] "Dense mode"; [DAB] backend table).
 *   O = softmax(sm_scale * Q K^T) V, per batch entry and query head.
 *   q, k, v: device bf16 per the layout above; o: device, o_dtype BF16 or
 *   FP32 (round to nearest even).  sm_scale: finite and > 0 (typically
 *   1/sqrt(128); INVALID_ARG otherwise).  Errors: INVALID_ARG,
 *   UNSUPPORTED_HEAD_DIM, BAD_GQA,
 *   BAD_LAYOUT, DEVICE.  Empty problems (B, S_q, Hq = 0) return OK with no
 *   launch; S_kv = 0 with S_q > 0 is INVALID_ARG (softmax over no keys).
 *   S_q and S_kv are independent (cross-attention: Q from one sequence, K/V
 *   from another).
 *   lse (nullable, device, 4-byte aligned): [B, Hq, S_q] fp32, contiguous,
 *   receives LSE_i = ln sum_j exp(sm_scale <q_i, k_j>) per row: the weight
 *   that merges attention results over disjoint key sets, as context
 *   parallelism needs ([VQA] "Interaction With Other Features": the dense
 *   backend that exports LSE composes with ring / Attention2D parallelism).
 *   BAD_LAYOUT if misaligned. */
int attn_dense_bf16(const void* q, const void* k, const void* v, void* o,
                    attn_dtype o_dtype, const attn_shape* shape, float sm_scale,
                    float* lse, void* stream);

/* Workspace layout for sage_quantize / attn_sage ([VQA] "SageAttention in
 * the TRTLLM backend").  Host-only; fills *out.  Errors as sage_quantize. */
int attn_sage_layout_query(const attn_shape* shape, const attn_recipe* recipe,
                           attn_sage_layout* out);

/* SAGE quantization of Q, K and V into the workspace ([TA] "SAGE
 * quantization": Q/K per block, V per channel, K-smoothing internal).
 *   mu[b,g,d] = mean of K over all S_kv tokens (binary32; tokens summed in
 *     chunks of 256 in ascending order, chunk sums added in ascending order,
 *     then divided by S_kv);
 *   K_hat = K - mu; Q and K_hat quantized per block of q_block / k_block
 *     tokens x 128 channels of one head: a = max|x|, scale = a / QMAX (1 if
 *     a == 0), code = round_nearest_even(x / scale) saturated to +-QMAX, QMAX
 *     = 127 (int8) or 448 (E4M3);
 *   V quantized to E4M3 per (b, kv head, channel) with scale max|v| / 448.
 * Every division is a correctly rounded binary32 division.  ws must hold
 * layout.total_bytes (device, 256-byte aligned); the output tensors sit at
 * the layout's offsets.  Errors: INVALID_ARG, UNSUPPORTED_HEAD_DIM, BAD_GQA,
 * UNSUPPORTED_RECIPE, BAD_LAYOUT, WORKSPACE_TOO_SMALL, DEVICE. */
int sage_quantize(const void* q, const void* k, const void* v, const attn_shape* shape,
                  const attn_recipe* recipe, void* ws, size_t ws_bytes, void* stream);

/* sage_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same quantization, bit for bit, but the statistics scratch (K chunk
 * sums and V channel maxima, the layout's region from scratch_off on) lives
 * in a static device array of the library, 16 MiB per device, held until the
 * process ends.  out receives the other regions at the layout's offsets and
 * must hold layout.scratch_off bytes (device, 256-byte aligned); the call
 * allocates nothing.  Problems whose statistics exceed the array,
 * 512 * B * Hkv * (ceil(S_kv / 256) + 1) bytes or so (B * Hkv *
 * ceil(S_kv / 256) up to about 32,000: 40 KV heads up to S_kv of about
 * 200,000), return WORKSPACE_TOO_SMALL before any device call.  Every call on
 * one device shares that device's array (each call clears what must start at
 * zero): calls that overlap in time on one device race, so issue them on one
 * stream.  Errors as sage_quantize. */
int sage_quantize_noalloc(const void* q, const void* k, const void* v, const attn_shape* shape,
                          const attn_recipe* recipe, void* out, size_t out_bytes, void* stream);

/* SAGE attention ([TA] "SAGE quantization": both matmuls in low precision;
 * [SSD] knob table: sage_block_sizes, bmm1_scale / bmm2_scale).
 *   Runs sage_quantize into ws, then attention on the codes:
 *   L_ij = log2(e) * sm_scale * sq_i * sk_j * <qc_i, kc_j> (bmm1 scale);
 *   online softmax over KV tiles of 64 keys in ascending order against the
 *   exact running maximum m_i of L; P enters BMM2 as p~ = E4M3(2^8 p) with
 *   p = 2^(L - m); the row sum l adds the unrounded p; O = acc * sv_d /
 *   (2^8 l) (bmm2 scale).  o_dtype BF16 or FP32.  Errors as sage_quantize. */
int attn_sage(const void* q, const void* k, const void* v, void* o, attn_dtype o_dtype,
              const attn_shape* shape, const attn_recipe* recipe, float sm_scale,
              void* ws, size_t ws_bytes, void* stream);

/* SAGE attention with Skip-Softmax, both in one kernel ([DAB] and [TA]:
 * Skip-Softmax runs on the TRTLLM backend that SAGE uses; [VQA]
 * "Interaction With Other Features": the two are exercised together; [SSD]
 * knob table: threshold = factor / seqlen).
 *   As attn_sage, plus the tile test of attn_skip_softmax applied to the
 *   dequantized logits L of attn_sage (log2 units): queries in blocks of
 *   sage_block_m rows, keys in the KV tiles of kv_tile keys
 *   (attn_tile_config: 32 rows x 64 keys); tile t > 0 is skipped when every
 *   valid row i of the
 *   block has 2^(M_it - m_i) < lambda = threshold_factor / S_kv, M_it the
 *   row's largest L in the tile and m_i its running maximum of L over the
 *   kept tiles.  A skipped tile changes nothing (not m_i, not the reference
 *   M, not the row sum).  threshold_factor = 0 runs exactly attn_sage
 *   (bit-identical).  skip_bitmap (nullable, device): [B, Hq,
 *   ceil(S_q/sage_block_m), ceil(S_kv/kv_tile)] uint8, 1 = skipped; skipped_tiles
 *   (nullable, device, 8-byte aligned): number of skipped (query block, KV
 *   tile) pairs.  ws as attn_sage.  Errors: as attn_sage, plus BAD_THRESHOLD
 *   (factor not finite or < 0). */
int attn_sage_skip_softmax(const void* q, const void* k, const void* v, void* o,
                           attn_dtype o_dtype, const attn_shape* shape,
                           const attn_recipe* recipe, float sm_scale,
                           float threshold_factor, uint8_t* skip_bitmap,
                           uint64_t* skipped_tiles, void* ws, size_t ws_bytes,
                           void* stream);

/* Skip-Softmax attention on BF16 ([TA] "Skip-Softmax"; [SSD] knob table:
 * skip_softmax_threshold_scale_factor, threshold = factor / seqlen).
 *   lambda = threshold_factor / S_kv.  Queries are tiled in blocks of
 *   block_m rows and keys in tiles of block_n keys (attn_tile_config: 64
 *   rows x 32 keys).  For
 *   each query block, KV tiles are visited in ascending order; tile t > 0 is
 *   skipped when, for every valid row i of the block,
 *   exp(M_it - m_i) < lambda, where M_it is the row's largest logit in the
 *   tile and m_i its running maximum over the tiles kept so far.  A skipped
 *   tile contributes nothing (no exponentials, no P V).  threshold_factor = 0
 *   runs exactly the dense kernel (bit-identical to attn_dense_bf16).
 *   skip_bitmap (nullable, device): [B, Hq, ceil(S_q/block_m),
 *   ceil(S_kv/block_n)] uint8, 1 = skipped.  skipped_tiles (nullable,
 *   device): receives the number of skipped (query block, KV tile) pairs.
 *   lse (nullable): as attn_dense_bf16, over the kept keys of each row.
 *   Errors: as attn_dense_bf16, plus BAD_THRESHOLD (factor not finite or
 *   < 0). */
int attn_skip_softmax(const void* q, const void* k, const void* v, void* o,
                      attn_dtype o_dtype, const attn_shape* shape, float sm_scale,
                      float threshold_factor, uint8_t* skip_bitmap,
                      uint64_t* skipped_tiles, float* lse, void* stream);

/* Host-side timestep gate ([TA] "Skip-Softmax", key disabled_until_timestep;
 * [SSD]: host-side gate, no kernel argument).  *enabled = (t <= D), with t
 * the normalized denoising timestep (1 = noisiest, 0 = clean).  Errors:
 * INVALID_ARG when t or D is not finite or outside [0, 1]. */
int attn_skip_gate(float t, float disabled_until_timestep, int* enabled);

/* Tile sizes of the attention kernels: block_m query rows and block_n keys
 * per Skip-Softmax vote of attn_skip_softmax (the skip bitmap's tile),
 * kv_tile keys per KV tile of the online softmax (the tile order SAGE's P
 * rounding follows), and sage_block_m query rows per vote of
 * attn_sage_skip_softmax (which votes on sage_block_m rows x kv_tile keys).
 * Host-only. */
int attn_tile_config(int* block_m, int* block_n, int* kv_tile, int* sage_block_m);

/* Message for the calling thread's last failed call ("" if none). */
const char* attn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DITATTN_H */
