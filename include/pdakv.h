/*
 * pdakv.h — paged INT8-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpdakv.so. Plain pointers and sizes only; no framework types.
 *
 * What the library computes
 * -------------------------
 * 1. kv_quant_int8_sym_write — per-token symmetric INT8 quantization of K and
 *    V into a paged cache (MoE-Infinity PR #183 "feat: opt-in INT8 KV-cache
 *    quantization", section "What landed", format-contract bullet, and section
 *    "Precision & memory"; mlxcel PR #717 "fix(cuda/kv): correct Int8 KV
 *    per-token scale ...", section "The Int8 bug and fix"). For every written
 *    token, KV head, and each of K and V separately:
 *        a     = max_d |x_d|
 *        scale = 1.0                                  if a == 0
 *              = smallest FP16 >= fl32(a / 127)        otherwise
 *        code  = clamp(round_half_even(fl32(x_d / scale)), -127, 127)
 *    so codes never take -128, exact zeros stay zero and every element obeys
 *    |x - code * scale| <= scale / 2 (+1e-6).
 * 2. paged_attn_decode_int8 — one decode query per sequence attending over
 *    that sequence's INT8 pages, reading the codes and FP16 scales directly,
 *    dequantizing in registers and accumulating with an FP32 online softmax;
 *    MHA and GQA (MoE-Infinity PR #183, "What landed", native-kernel bullet;
 *    "Scope & fallback").
 * 3. paged_attn_decode_fp16 — the same decode over 16-bit (fp16 or bf16) K/V
 *    pages with the same block-table layout, as a control.
 * 4. Static-scale variant — kv_quant_int8_static_write and
 *    paged_attn_decode_int8_static: one calibrated FP32 scalar for all of K
 *    and one for all of V of a layer, held by the caller, and codes-only
 *    pages (InfiniLM PR #553, "Summary" and "Notes for Reviewers";
 *    TensorRT-LLM PR #18953, "Summary"). code = clamp(round_half_even(
 *    fl32(x / scale)), -127, 127); values beyond 127.5 * scale saturate.
 *    The pages do not write the element rule out; this is the per-token
 *    rule with the given scale. A shared K/V scale is the case
 *    k_scale == v_scale (for instance the larger of two calibrated scales).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Ownership: the caller allocates and owns every buffer (device memory for
 *   all data pointers) and the stream. The library allocates nothing, keeps no
 *   global state and never synchronizes; every call is asynchronous on
 *   `stream` (a hipStream_t passed as void*; NULL = the default stream).
 * - Errors: every int-returning call returns PDAKV_OK (0) or a negative
 *   PDAKV_ERR_* code; nothing is launched when a call fails. Host-side checks
 *   look only at scalar arguments and pointer values, never at device memory.
 *   There is no silent fallback: an unsupported shape or dtype is an error.
 * - Data-dependent problems (a slot, block id or context length out of range,
 *   a scale beyond FP16) are found in the kernels: the offending token, page
 *   or row is skipped and, when `err_flag` (device int32, may be NULL) is
 *   given, the matching PDAKV_EFLAG_* bit is OR-ed into it. The caller clears
 *   it.
 * - Supported: head_dim 64 or 128; block_size 16; num_q_heads a multiple of
 *   num_kv_heads with at most 16 query heads per KV head; q/K/V dtype fp16 or
 *   bf16; FP16 scales always.
 * - Strides are in elements and must be >= 0; the innermost (head_dim)
 *   stride of q and out is 1.
 *
 * Page layout (the contract between writer, reader and any other user)
 * --------------------------------------------------------------------
 * One pool per layer: uint8 pool[num_blocks][page_bytes], 16-byte aligned.
 * A token at position t of a sequence lives in page block_table[t / 16] at
 * slot t % 16; writers address it as slot_id = page * 16 + t % 16.
 *
 * INT8 page (kv_format PDAKV_KV_INT8_SYM): every KV head's codes, then every
 * KV head's scales. For each KV head h in order, a code block of 2*16*D bytes
 * at h*32*D:
 *     +0          K codes  int8 [16][D]        token-major
 *     +16*D       V codes  int8 [4][D][4]      byte (p/4)*4*D + 4*d + p%4
 * then, at Hkv*32*D + 64*h, the head's scales as four 16-byte records, one
 * per group of four tokens (record p/4 at 16*(p/4)):
 *     +2*(p%4)     K scale fp16 of token p
 *     +8+2*(p%4)   V scale fp16 of token p
 *   page_bytes = Hkv * (32*D + 64): 33,280 for (16, 8, 128), 4,224 for
 *   (16, 2, 64). The V codes are grouped four tokens at a time so that one
 *   32-bit word holds one dimension of four consecutive tokens, which is the
 *   operand shape of the matrix instructions the reader uses; the scales sit
 *   after all code blocks so that each code block starts at a multiple of
 *   32*D bytes into the page, and one 16-byte read gives a token group's K
 *   and V scales.
 * Static-scale INT8 page (kv_format PDAKV_KV_INT8_STATIC), for each KV head h,
 * a head block of 2*16*D bytes:
 *     +0          K codes  int8 [16][D]        token-major
 *     +16*D       V codes  int8 [4][D][4]      as in the per-token page
 *   page_bytes = Hkv * 32 * D: 32,768 for (16, 8, 128), half the 16-bit page.
 * 16-bit page (kv_format PDAKV_KV_16BIT), for each KV head h, 4*16*D bytes:
 *     +0          K  [16][D]                    token-major
 *     +32*D       V  [4][D][4]                  element (p/4)*4*D + 4*d + p%4
 *   page_bytes = Hkv * 64 * D: 65,536 for (16, 8, 128).
 */
#ifndef PDAKV_H
#define PDAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------- */
#define PDAKV_OK               0
#define PDAKV_ERR_INVALID_ARG (-1) /* null pointer, negative size/stride, misalignment */
#define PDAKV_ERR_UNSUPPORTED (-2) /* shape outside the supported set */
#define PDAKV_ERR_DTYPE       (-3) /* dtype code not accepted by this call */
#define PDAKV_ERR_WORKSPACE   (-4) /* workspace missing or too small */
#define PDAKV_ERR_HIP         (-5) /* a HIP runtime call or kernel launch failed */
#define PDAKV_ERR_NO_DEVICE   (-6) /* no usable HIP device */

/* ---- dtype codes ------------------------------------------------------ */
#define PDAKV_DTYPE_F32  0
#define PDAKV_DTYPE_F16  1
#define PDAKV_DTYPE_BF16 2

/* ---- KV page formats -------------------------------------------------- */
#define PDAKV_KV_INT8_SYM    1
#define PDAKV_KV_16BIT       2
#define PDAKV_KV_INT8_STATIC 3

/* ---- bits OR-ed into the optional device error flag ------------------- */
#define PDAKV_EFLAG_SLOT_RANGE    1 /* slot_id >= num_blocks * block_size   */
#define PDAKV_EFLAG_BLOCK_RANGE   2 /* block table entry outside the pool   */
#define PDAKV_EFLAG_CONTEXT_RANGE 4 /* context_lens[b] < 0 or > max_context */
#define PDAKV_EFLAG_SCALE_RANGE   8 /* absmax / 127 beyond the FP16 range   */

/* ---- capability bits -------------------------------------------------- */
#define PDAKV_CAP_GFX950      1u  /* current device is gfx950             */
#define PDAKV_CAP_HEAD_DIM_64 2u
#define PDAKV_CAP_HEAD_DIM_128 4u
#define PDAKV_CAP_BLOCK_16    8u
#define PDAKV_CAP_F16         16u
#define PDAKV_CAP_BF16        32u

/* Library version, major*10000 + minor*100 + patch. */
int pdakv_version(void);

/* Human-readable text for a status code (static storage; never NULL). */
const char* pdakv_status_string(int status);

/* Bytes of one page of the given format (MoE-Infinity PR #183, "Precision &
 * memory": 33,280 INT8 vs 65,536 FP16 bytes for block 16, 8 KV heads,
 * head_dim 128). Returns 0 for an unsupported combination. Pure host
 * arithmetic; needs no device. */
size_t pdakv_page_bytes(int kv_format, int block_size, int num_kv_heads, int head_dim);

/* Capability probe of the current HIP device (the native-binding check of
 * MoE-Infinity PR #183, "What landed", runtime-integration bullet). Writes the
 * PDAKV_CAP_* bits to *flags_out. Returns PDAKV_ERR_NO_DEVICE without a
 * device, PDAKV_ERR_INVALID_ARG for a NULL flags_out. */
int pdakv_capabilities(uint32_t* flags_out);

/* Launch plan of the one-token decode calls for these sizes. The work of a
 * call is the list of (sequence, KV head, page) items; the kernel splits the
 * items of the actual context lengths evenly over *num_waves 64-lane waves
 * (at least 2 items each, a unit that spans several waves is merged
 * afterwards): one resident round of waves, one per SIMD where a KV head's
 * block of a page holds 4 KB or more (INT8 pages at head_dim 128, 16-bit
 * pages) and that round holds every item at <= 128 each, else two (more
 * rounds only beyond 128 items per wave). *max_pages_per_wave is the share
 * when every sequence is at max_context_len (<= 128). kv_format is one of
 * the PDAKV_KV_* formats.
 * Either output pointer may be NULL. Returns PDAKV_ERR_INVALID_ARG for a bad
 * format or negative sizes and PDAKV_ERR_UNSUPPORTED for a head_dim other
 * than 64 or 128 or above 2^30 items. Host arithmetic only. */
int pdakv_decode_plan(int kv_format, int num_seqs, int num_kv_heads, int head_dim,
                      int max_context_len, int* num_waves, int* max_pages_per_wave);

/* Device workspace the decode calls need for these sizes (0 when
 * max_context_len or num_seqs is 0). The same value serves every decode
 * entry point. Layout: float partials
 * [num_waves + num_seqs * num_kv_heads][num_q_heads / num_kv_heads][head_dim + 2]
 * (num_waves: the plan at two waves per SIMD, which no decode plan exceeds;
 * the region padded to a multiple of 16 bytes), then int32
 * [num_seqs * num_kv_heads][2] merge records. */
size_t pdakv_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int max_context_len);

/* Device workspace of the decode calls for any KV-head count: the largest
 * pdakv_decode_workspace_bytes() over every num_kv_heads that divides
 * num_q_heads with at most 16 query heads per KV head (0 when num_seqs,
 * max_context_len or num_q_heads is 0, or no such count exists). For callers
 * that size one workspace before the KV-head count is known; a workspace of
 * this size serves every one-token decode entry point with these sizes. Host
 * arithmetic only. */
size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                         int max_context_len);

/* Quantize-on-write (MoE-Infinity PR #183, "What landed": write_chunk into
 * the paged store; the quantizer of the format-contract bullet).
 *   k_src, v_src   device, [num_tokens][num_kv_heads][head_dim] of src_dtype
 *                  (PDAKV_DTYPE_F16 or _BF16) addressed through the given
 *                  element strides, so views of a fused QKV buffer can be
 *                  passed without a copy (K/V are read in model precision
 *                  before quantization, as InfiniLM PR #553 "Summary" asks).
 *   slot_mapping   device int32 [num_tokens]; slot_id = page * block_size +
 *                  offset; a negative entry marks a padding token, which is
 *                  skipped; an entry >= num_blocks * block_size is skipped
 *                  and flagged PDAKV_EFLAG_SLOT_RANGE.
 *   kv_pool        device, num_blocks pages of the INT8 format.
 * Two tokens of one call must not name the same slot. A (token, KV head)
 * whose K or V scale would exceed 65504, or whose K or V row holds a NaN or
 * an infinity, is left unwritten and flagged PDAKV_EFLAG_SCALE_RANGE. */
int kv_quant_int8_sym_write(const void* k_src, const void* v_src, int src_dtype,
                            int64_t num_tokens, int num_kv_heads, int head_dim,
                            int64_t k_stride_tok, int64_t k_stride_head, int64_t k_stride_dim,
                            int64_t v_stride_tok, int64_t v_stride_head, int64_t v_stride_dim,
                            const int32_t* slot_mapping, void* kv_pool, int64_t num_blocks,
                            int block_size, int32_t* err_flag, void* stream);

/* Plain 16-bit write into a PDAKV_KV_16BIT pool: fills the cache of the
 * FP16-KV control, whose pages hold the model-precision values, 65,536 bytes
 * per (block 16, 8 KV heads, head_dim 128) page (MoE-Infinity PR #183,
 * "Precision & memory"; the pre-existing FP16 paged cache of "What landed").
 * Same arguments and conventions as kv_quant_int8_sym_write; values are
 * copied unchanged (no scale, so nothing is flagged for range), in the
 * 16-bit page layout above. */
int kv_write_16bit(const void* k_src, const void* v_src, int src_dtype,
                   int64_t num_tokens, int num_kv_heads, int head_dim,
                   int64_t k_stride_tok, int64_t k_stride_head, int64_t k_stride_dim,
                   int64_t v_stride_tok, int64_t v_stride_head, int64_t v_stride_dim,
                   const int32_t* slot_mapping, void* kv_pool, int64_t num_blocks,
                   int block_size, int32_t* err_flag, void* stream);

/* Paged decode over INT8 pages (MoE-Infinity PR #183, "What landed",
 * native-kernel bullet: INT8 + FP16-scale paged decode with FP32
 * accumulation, MHA/GQA).
 *   out            device [num_seqs][num_q_heads][head_dim] of out_dtype
 *                  (F32, F16 or BF16), strides out_stride_seq/_head.
 *   q              device [num_seqs][num_q_heads][head_dim], q_dtype F16/BF16.
 *   kv_pool        INT8 pool of num_blocks pages (layout above); at least one
 *                  page when max_context_len > 0.
 *   block_tables   device int32 [num_seqs][block_table_stride]; row b lists the
 *                  pages of sequence b; only the first ceil(context_lens[b]/16)
 *                  entries are read.
 *   context_lens   device int32 [num_seqs]; 0 gives a zero output row; values
 *                  above max_context_len are clamped and flagged. Pages
 *                  whose block id is out of range are flagged and skipped; a
 *                  (sequence, KV head) left with no token gives zero rows.
 *   max_context_len host upper bound of context_lens (sizes the launch).
 *   sm_scale       logit scale (usually 1/sqrt(head_dim)).
 *   workspace      device scratch of at least pdakv_decode_workspace_bytes(),
 *                  16-byte aligned; may be NULL when that is 0. Its contents
 *                  need no initialization and are garbage afterwards. Calls
 *                  that share one workspace must not overlap in time.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads). The output
 * must not alias any input. */
int paged_attn_decode_int8(void* out, int out_dtype, int64_t out_stride_seq,
                           int64_t out_stride_head, const void* q, int q_dtype,
                           int64_t q_stride_seq, int64_t q_stride_head, const void* kv_pool,
                           int64_t num_blocks, int block_size, const int32_t* block_tables,
                           int64_t block_table_stride, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_context_len, float sm_scale, void* workspace,
                           size_t workspace_bytes, int32_t* err_flag, void* stream);

/* Bytes of the device scratch that paged_attn_decode_int8_noalloc uses in
 * place of a workspace (32 MiB per GPU). */
#define PDAKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/* paged_attn_decode_int8 without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments, result and error
 * convention as paged_attn_decode_int8 minus workspace / workspace_bytes.
 * The library's own scratch stands in for the workspace: a file-scope device
 * array of PDAKV_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends;
 * its device address is looked up on a device's first call (make that call
 * outside graph capture). The call allocates nothing.
 *   - A call whose pdakv_decode_workspace_bytes() exceeds
 *     PDAKV_NOALLOC_SCRATCH_BYTES returns PDAKV_ERR_WORKSPACE and launches
 *     nothing (use paged_attn_decode_int8 with a workspace instead).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (nothing in it needs to start at zero). Calls that
 *     overlap in time on one GPU -- on different streams, or from different
 *     threads without ordering -- race on it and give undefined results.
 *   - PDAKV_ERR_NO_DEVICE without a current HIP device. */
int paged_attn_decode_int8_noalloc(void* out, int out_dtype, int64_t out_stride_seq,
                                   int64_t out_stride_head, const void* q, int q_dtype,
                                   int64_t q_stride_seq, int64_t q_stride_head,
                                   const void* kv_pool, int64_t num_blocks, int block_size,
                                   const int32_t* block_tables, int64_t block_table_stride,
                                   const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int max_context_len,
                                   float sm_scale, int32_t* err_flag, void* stream);

/* Paged decode over 16-bit pages (the FP16-KV control; MoE-Infinity PR #183,
 * "What landed": the pre-existing FP16 paged-attention kernel). Same
 * arguments as paged_attn_decode_int8; kv_pool is a PDAKV_KV_16BIT pool whose
 * values have the dtype q_dtype. */
int paged_attn_decode_fp16(void* out, int out_dtype, int64_t out_stride_seq,
                           int64_t out_stride_head, const void* q, int q_dtype,
                           int64_t q_stride_seq, int64_t q_stride_head, const void* kv_pool,
                           int64_t num_blocks, int block_size, const int32_t* block_tables,
                           int64_t block_table_stride, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_context_len, float sm_scale, void* workspace,
                           size_t workspace_bytes, int32_t* err_flag, void* stream);

/* Fused decode step: append each sequence's newest token and attend
 * (InfiniLM PR #553 "fix: #552 int8 kv cache quantization cannot be enabled",
 * benchmark note after "Summary": separate per-step quantize kernels cost
 * INT8 decode 7-10%; here the quantize-on-write of the new token runs inside
 * the decode launch).
 * Same result as kv_quant_int8_sym_write of k_new/v_new with, for every
 * sequence b with context_lens[b] >= 1, the slot of position
 * context_lens[b] - 1 (page block_tables[b][(L - 1) / 16], offset (L - 1) % 16),
 * followed by paged_attn_decode_int8 over all L positions.
 *   k_new, v_new   device [num_seqs][num_kv_heads][head_dim] of q_dtype (F16
 *                  or BF16) through the given element strides; row b is
 *                  sequence b's newest token. Other arguments as
 *                  paged_attn_decode_int8.
 * A sequence with context length 0 gets zero rows and no write. A row whose
 * scale would exceed 65504, or that holds a NaN or an infinity, is flagged
 * PDAKV_EFLAG_SCALE_RANGE and not written, as kv_quant_int8_sym_write treats
 * it (the slot keeps its old contents, which the attention then reads). With an
 * out-of-range context length (flagged) the token is written at the clamped
 * length's last position. */
int paged_attn_decode_int8_append(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_head, const void* q,
    int q_dtype, int64_t q_stride_seq, int64_t q_stride_head, const void* k_new,
    const void* v_new, int64_t k_stride_seq, int64_t k_stride_head, int64_t k_stride_dim,
    int64_t v_stride_seq, int64_t v_stride_head, int64_t v_stride_dim, void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream);

/* The fused step over 16-bit pages (the control for the fused INT8 step):
 * kv_write_16bit of the newest tokens, then paged_attn_decode_fp16; same
 * arguments as paged_attn_decode_int8_append. */
int paged_attn_decode_fp16_append(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_head, const void* q,
    int q_dtype, int64_t q_stride_seq, int64_t q_stride_head, const void* k_new,
    const void* v_new, int64_t k_stride_seq, int64_t k_stride_head, int64_t k_stride_dim,
    int64_t v_stride_seq, int64_t v_stride_head, int64_t v_stride_dim, void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream);

/* Quantize-on-write with static scales (InfiniLM PR #553 "fix: #552 int8 kv
 * cache quantization cannot be enabled", "Summary": per-tensor
 * kv_cache_k_scale / kv_cache_v_scale; TensorRT-LLM PR #18953 "Add calibrated
 * INT8 KV cache to PyTorch backend", "Summary": positive finite float32
 * k_scale / v_scale). Same arguments as kv_quant_int8_sym_write plus
 *   k_scale, v_scale   host float, the layer's scales; each must be finite
 *                      and > 0, else PDAKV_ERR_INVALID_ARG.
 * kv_pool is a PDAKV_KV_INT8_STATIC pool. Every element gets
 * clamp(round_half_even(fl32(x / scale)), -127, 127); nothing is flagged for
 * saturation (it is part of the scheme). Non-finite inputs: +inf gives 127,
 * -inf gives -127 and a NaN gives -127 (the clamp ignores a NaN operand);
 * paged_attn_decode_int8_static_append stores the same codes. */
int kv_quant_int8_static_write(const void* k_src, const void* v_src, int src_dtype,
                               int64_t num_tokens, int num_kv_heads, int head_dim,
                               int64_t k_stride_tok, int64_t k_stride_head, int64_t k_stride_dim,
                               int64_t v_stride_tok, int64_t v_stride_head, int64_t v_stride_dim,
                               float k_scale, float v_scale, const int32_t* slot_mapping,
                               void* kv_pool, int64_t num_blocks, int block_size,
                               int32_t* err_flag, void* stream);

/* Paged decode over static-scale INT8 pages: the attention of
 * paged_attn_decode_int8 with k_t = code * k_scale and v_t = code * v_scale.
 * Same arguments as paged_attn_decode_int8 plus k_scale and v_scale (host
 * float, finite and > 0, and sm_scale * k_scale finite, else
 * PDAKV_ERR_INVALID_ARG); kv_pool is a PDAKV_KV_INT8_STATIC pool. */
int paged_attn_decode_int8_static(void* out, int out_dtype, int64_t out_stride_seq,
                                  int64_t out_stride_head, const void* q, int q_dtype,
                                  int64_t q_stride_seq, int64_t q_stride_head,
                                  const void* kv_pool, int64_t num_blocks, int block_size,
                                  const int32_t* block_tables, int64_t block_table_stride,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int max_context_len,
                                  float sm_scale, float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, int32_t* err_flag, void* stream);

/* The fused append + decode step over static-scale pages:
 * kv_quant_int8_static_write of the newest tokens (as for
 * paged_attn_decode_int8_append), then paged_attn_decode_int8_static. Same
 * arguments as paged_attn_decode_int8_append plus k_scale and v_scale. */
int paged_attn_decode_int8_static_append(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_head, const void* q,
    int q_dtype, int64_t q_stride_seq, int64_t q_stride_head, const void* k_new,
    const void* v_new, int64_t k_stride_seq, int64_t k_stride_head, int64_t k_stride_dim,
    int64_t v_stride_seq, int64_t v_stride_head, int64_t v_stride_dim, void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, float k_scale, float v_scale, void* workspace,
    size_t workspace_bytes, int32_t* err_flag, void* stream);

/* Decode with several query tokens per sequence: speculative verification
 * of draft tokens, or a short chunk decoded against the cache (mlxcel PR
 * #717, "Server integration": INT8 chunked prefill followed by decode; the
 * multi-token case of the paged decode of MoE-Infinity PR #183, "What
 * landed"). The num_query_tokens = T new tokens are the last T positions of
 * each sequence and must already be in the pool (written with
 * kv_quant_int8_sym_write); context_lens[b] counts them. Query token j of
 * sequence b sits at position context_lens[b] - T + j and attends to
 * positions 0 .. context_lens[b] - T + j (causal among the new tokens); a
 * token whose position is negative gets a zero row.
 *   out   device [num_seqs][T][num_q_heads][head_dim] of out_dtype through
 *         the strides out_stride_seq / _tok / _head (elements).
 *   q     device [num_seqs][T][num_q_heads][head_dim] of q_dtype through
 *         q_stride_seq / _tok / _head.
 *   workspace  at least pdakv_decode_multi_workspace_bytes() for the same
 *         sizes, 16-byte aligned.
 * Other arguments as paged_attn_decode_int8. The T x (num_q_heads /
 * num_kv_heads) query columns of a KV head are processed in tiles of 16
 * matrix-instruction columns; a KV head's pages are streamed once for every
 * run of up to 4 tiles (once in all for up to 64 columns).
 * Returns PDAKV_ERR_INVALID_ARG for num_query_tokens < 1. */
int paged_attn_decode_int8_multi(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_tok,
    int64_t out_stride_head, const void* q, int q_dtype, int64_t q_stride_seq,
    int64_t q_stride_tok, int64_t q_stride_head, int num_query_tokens, const void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream);

/* The several-token decode over 16-bit pages (the control); same arguments
 * as paged_attn_decode_int8_multi, kv_pool a PDAKV_KV_16BIT pool of q's
 * dtype. */
int paged_attn_decode_fp16_multi(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_tok,
    int64_t out_stride_head, const void* q, int q_dtype, int64_t q_stride_seq,
    int64_t q_stride_tok, int64_t q_stride_head, int num_query_tokens, const void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream);

/* Workspace of the several-token decode calls: the layout of
 * pdakv_decode_workspace_bytes with units of (sequence, KV head, run of up
 * to 4 tiles of 16 query columns), min(T * G, 64) columns per partial slot;
 * 0 when num_seqs, num_query_tokens or max_context_len is 0. With
 * num_query_tokens = 1 it equals pdakv_decode_workspace_bytes. */
size_t pdakv_decode_multi_workspace_bytes(int num_seqs, int num_query_tokens, int num_q_heads,
                                          int num_kv_heads, int head_dim, int max_context_len);

/* Page swap-out (MoE-Infinity PR #183, "What landed", serving-lifecycle
 * bullet: pages are swapped out of GPU memory and back in, INT8 scales
 * included). Copies page block_ids[i] of the pool (num_blocks pages of
 * page_bytes each; page_bytes = pdakv_page_bytes() of the pool's format, a
 * multiple of 16) to dst + i * page_bytes, for i < num_pages. Every format
 * keeps a token's scales inside its page, so whole pages carry them.
 *   dst        device memory, or pinned host memory (hipHostMalloc; passed
 *              as its host address, the library looks up the address the GPU
 *              uses); 16-byte aligned; num_pages * page_bytes bytes. Pageable
 *              host memory is rejected with PDAKV_ERR_INVALID_ARG.
 *   block_ids  device int32 [num_pages]; an id outside [0, num_blocks) is
 *              flagged PDAKV_EFLAG_BLOCK_RANGE and its entry left unwritten.
 * Rolling a swap back (the transaction of a residency change) is the
 * caller's: this call only moves bytes. */
int kv_pages_swap_out(const void* kv_pool, int64_t num_blocks, int64_t page_bytes,
                      const int32_t* block_ids, int64_t num_pages, void* dst, int32_t* err_flag,
                      void* stream);

/* Page swap-in: copies src + i * page_bytes into page block_ids[i] of the
 * pool (the pages may differ from the ones swapped out; the caller updates
 * its block tables). The ids must be distinct; out-of-range ids are flagged
 * and skipped. src is device or pinned host memory, 16-byte aligned. */
int kv_pages_swap_in(const void* src, int64_t num_pages, const int32_t* block_ids, void* kv_pool,
                     int64_t num_blocks, int64_t page_bytes, int32_t* err_flag, void* stream);

/* Front trim that keeps sink tokens (mlxcel PR #717 and its follow-up on the
 * same page: drop the n tokens after the first `keep` positions instead of
 * the n oldest, so the first tokens survive; the INT8 scales move with their
 * tokens). For every sequence b with L = context_lens[b] and
 * n = clamp(trim_lens[b], 0, max(L - keep, 0)), the tokens at positions
 * keep + n .. L - 1 move to positions keep .. L - n - 1 through the
 * sequence's block table, in place, and new_context_lens[b] = L - n. Slots at
 * or past the new length keep what they held; pages no longer needed are
 * the caller's to free. Cutting the end of a sequence (truncation) moves
 * nothing: it is a shorter context length.
 *   kv_format  any PDAKV_KV_* format; the pool layout above.
 *   trim_lens, context_lens   device int32 [num_seqs].
 *   new_context_lens  device int32 [num_seqs]; must not alias context_lens.
 *   keep       host int >= 0.
 * Pages the trim rewrites (positions >= keep) must belong to that sequence
 * alone. Context lengths beyond block_table_stride * 16 are clamped and
 * flagged; a token whose source or destination page is out of range is not
 * moved (flagged). */
int kv_trim_keep_sink(int kv_format, void* kv_pool, int64_t num_blocks, int block_size,
                      int num_kv_heads, int head_dim, const int32_t* block_tables,
                      int64_t block_table_stride, const int32_t* context_lens,
                      const int32_t* trim_lens, int num_seqs, int keep,
                      int32_t* new_context_lens, int32_t* err_flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PDAKV_H */
