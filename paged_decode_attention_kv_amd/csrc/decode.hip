// Paged decode attention over INT8 pages (codes + FP16 per-token scales, or
// codes only with static per-tensor scales) and over 16-bit pages (the
// control), for gfx950.
//
// What is computed (MoE-Infinity PR #183 "feat: opt-in INT8 KV-cache
// quantization", "What landed", native-kernel bullet): for sequence b and
// query head h reading KV head g = h / G,
//   out = sum_t softmax_t(sm_scale * <q, sK_t * cK_t>) * sV_t * cV_t
// with the INT8 codes and FP16 scales read straight from the pages,
// dequantized in registers, and an FP32 online softmax.
//
// Work decomposition
// ------------------
// The work of one call is the list of (sequence, KV head, page) items, in
// that order: KV head g of sequence b owns the items of its pages
// 0..ceil(L_b/16)-1 (a "unit"). Every wave of the grid takes an equal,
// contiguous run of P items (P = max(2, ceil(total / waves))), so all waves
// stream the same number of pages whatever the spread of context lengths, and
// they run independently (LDS is private to each wave; no barrier). Each wave
// derives the total and its start from the context lengths itself (a prefix
// sum over the batch, 64 sequences per step, in registers).
// A wave's run crosses one or more units ("segments"). It handles them in
// passes: a pass plans up to seg_cap segments, reads all their block ids at
// once, stages their q rows in LDS, and then streams every page of the pass
// through one pipeline; a segment switch only stashes the finished softmax
// state in LDS and loads the next q rows from LDS, so the page loads in
// flight are never waited for early. One page = 16 tokens = one 16x16 MFMA
// tile:
//  * QK: S[t][c] = sum_d K[t][d] * q_c[d] with K in the A operand (row t =
//    lane % 16) and up to 16 query columns in the B operand (column c =
//    lane % 16, zero-padded): the G query heads of the KV head, or with
//    several query tokens per sequence the (token, head) pairs of a tile.
//    Every K byte is fetched once and shared by all columns inside the
//    matrix instruction. INT8 codes become fp16 exactly; q is scaled by a
//    power of two into fp16 range (exact for fp16/bf16 inputs down to far
//    below any contributing term) and the scale is undone on the fp32
//    logits. Products are exact, sums fp32.
//  * The result tile holds, in lane l, tokens 4*(l/16)+j (j = 0..3) of column
//    l % 16 — exactly the B-operand layout the PV product needs, so the
//    probabilities never leave registers.
//  * PV: O^T[d][c] = sum_t V[t][d] * P[c][t]. The V codes of four tokens of
//    one dimension share a 32-bit word in the page: the A operand of one lane
//    of a 16x16x16 instruction. The fp32 probability (V scale folded in) is
//    split into a high and a low fp16 part (22 significant bits), contracted
//    by two instructions.
//  * Online softmax state (running max m, sum l, accumulator) lives in the
//    lanes of column l % 16. The V scale sV = f * 2^e (f in [0.5, 1)) enters
//    the logit as the base-2 exponent e, so the folded probabilities
//    P = 2^(s + e - m) * f never leave the fp16 range whatever the scales.
//    With static scales the K scale is part of the logit factor and the V
//    scale multiplies the output.
//  * Page pairs (one-token calls, groups of at most 8 heads, head size 128):
//    the 16 columns hold the group twice, columns 0-7 for the first page of
//    a pair and 8-15 for the second, so one softmax update covers 32 tokens.
//    QK runs on the integer matrix instructions with the codes as loaded and
//    q in three signed base-256 digits (exact int32 sums), each page meeting
//    q in its own half of the columns; PV takes both pages in one 16x16x32
//    instruction per dimension block and part, and the two column halves
//    are added when the segment ends.
// A segment that covers a whole unit writes the output rows directly;
// otherwise it writes a partial (max, sum, accumulator) into the slot
// wave + unit (unique: along the item order both indexes only grow and one of
// them grows at every segment boundary), and merge_kernel combines the
// partials of each unit that spans several waves. (Merging in the last
// arriving wave would need agent-scope fences, which write back and
// invalidate the L2 of the XCD: measured far dearer than the second launch.)
#include <type_traits>

#include "device_util.h"
#include "launch.h"
#include "quant_row.h"

namespace pdakv {

namespace {

// Probabilities are carried times 2^kPScale relative to the running max m; m
// is raised only when a new logit exceeds it by more than kTau (base-2
// units), so the accumulator is rescaled rarely and probabilities stay below
// 2^(kPScale + kTau) = 2^15, inside the fp16 range of the PV operand, with
// their low fp16 parts clear of the subnormal range.
constexpr float kTau = 8.0f;
constexpr float kPScale = 7.0f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int readlane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// ---------------------------------------------------------------------------
// Work partition
// ---------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// 64 sequences of the batch, one per lane: sequence 64 * c + lane.
struct SeqChunk {
  int c;     // chunk index
  int L;     // lane's clamped context length (0 past the batch)
  int np;    // lane's page count
  int excl;  // pages (per KV head) of all sequences before the lane's
};

// Context lengths are clamped to [0, max_ctx]; an out-of-range value is
// flagged when `report`.
__device__ __forceinline__ SeqChunk load_chunk(const DecodeArgs& a, int c, int base, bool report,
                                               int lane) {
  SeqChunk s;
  s.c = c;
  const int b = 64 * c + lane;
  int L = b < a.num_seqs ? a.ctx[b] : 0;
  if (L < 0 || L > a.max_ctx) {
    if (report) raise_flag(a.err, PDAKV_EFLAG_CONTEXT_RANGE);
    L = L < 0 ? 0 : a.max_ctx;
  }
  s.L = L;
  s.np = (L + kBlockSize - 1) / kBlockSize;
  s.excl = base + wave_incl_scan(s.np, lane) - s.np;
  return s;
}

// Pages (per KV head) of all sequences up to the end of the chunk.
__device__ __forceinline__ int chunk_end(const SeqChunk& s) { return readlane(s.excl + s.np, 63); }

__device__ __forceinline__ int pages_per_wave(int total, int waves) {
  const int p = (total + waves - 1) / waves;
  return p > kMinPagesPerWave ? p : kMinPagesPerWave;
}

// Zero output rows of the empty sequences of the chunk; sequence b is done by
// wave b % waves.
__device__ void zero_rows(const DecodeArgs& a, const SeqChunk& s, int wave, int D, int lane) {
  const int b = 64 * s.c + lane;
  uint64_t m = __ballot(b < a.num_seqs && s.np == 0 && b % a.num_waves == wave);
  while (m) {
    const int bb = 64 * s.c + __builtin_ctzll(m);
    m &= m - 1;
    const int rows = a.qtok * a.num_q_heads;  // (query token, head) rows
    for (int i = lane; i < rows * D; i += 64) {
      const int r = i / D;
      store_out(a.out, a.out_dtype,
                bb * a.out_ss + (r / a.num_q_heads) * a.out_st + (r % a.num_q_heads) * a.out_sh +
                    i % D,
                0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Online softmax state and shared helpers
// ---------------------------------------------------------------------------

// Eight consecutive 16-bit q elements (dims d0..d0+7) of query token j, head
// h, as four words. One 16-byte load when the host found q's pointer and
// strides 16-byte aligned, else eight 2-byte loads. Always issued (no per-lane
// branch), so the loads of a wave overlap.
__device__ __forceinline__ u4_t q_chunk8(const DecodeArgs& a, int b, int j, int h, int d0) {
  const uint16_t* row =
      static_cast<const uint16_t*>(a.q) + b * a.q_ss + j * a.q_st + h * a.q_sh + d0;
  if (a.q_vec16) return *reinterpret_cast<const u4_t*>(row);
  u4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = row[2 * i] | (static_cast<uint32_t>(row[2 * i + 1]) << 16);
  return w;
}

template <int ND>
struct SoftmaxState {
  float m;   // running max (base-2 units)
  float mk;  // m - kPScale
  float l;
  f4_t acc[ND];
};

// Start value of the running max: finite, so that a page whose tokens are all
// masked (logit -inf) adds exactly 0 before any token was seen.
constexpr float kMaxInit = -1e30f;

template <int ND>
__device__ __forceinline__ void softmax_init(SoftmaxState<ND>& st) {
  st.m = kMaxInit;
  st.mk = kMaxInit;
  st.l = 0.f;
#pragma unroll
  for (int k = 0; k < ND; ++k) st.acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};
}

// Lane i16 ^ 8 of the same 16-lane row (DPP row rotation by 8).
__device__ __forceinline__ float row_partner8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Pair: the tile's columns i16 and i16 ^ 8 hold one head on two pages and
// keep one running max, so that their accumulators add at the end.
template <bool Pair = false, int ND>
__device__ __forceinline__ void raise_max(SoftmaxState<ND>& st, float zmax) {
  zmax = col_max(zmax);
  if constexpr (Pair) zmax = max_fin(zmax, row_partner8(zmax));
  if (__any(zmax > st.m + kTau)) {
    const float m_new = fmaxf(st.m, zmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 on the first token
    st.m = m_new;
    st.mk = m_new - kPScale;
    st.l *= alpha;
#pragma unroll
    for (int k = 0; k < ND; ++k) st.acc[k] *= alpha;
  }
}

// Four int8 codes (byte i = element i) -> four fp16 values, exactly: bias the
// bytes to c + 128, place each in the mantissa of the fp16 constant 1024
// (0x6400) with one byte permute per pair, and subtract 1024 + 128.
__device__ __forceinline__ u2_t i8x4_to_f16x4_perm(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const h2_t bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  u2_t r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, lo) - bias);
  r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, hi) - bias);
  return r;
}

// q fragments as fp16 scaled by 2^kq so that max|q| of the head lies in
// [2^14, 2^15); fragment j holds the eight 16-bit values chunk(j). Lanes of
// padding heads (hvalid false) use zeros. Returns the factor that turns the
// MFMA dot products into base-2 logits.
template <int NJ, bool QBF16, typename ChunkFn>
__device__ __forceinline__ float load_q_scaled(const DecodeArgs& a, bool hvalid, ChunkFn chunk,
                                               h8_t* qf) {
  u4_t raw[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) raw[j] = chunk(j);
  float qv[NJ * 8];
  float qmax = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint16_t bits = static_cast<uint16_t>(raw[j][r / 2] >> (16 * (r % 2)));
      const float x = hvalid ? bits16_to_f32<QBF16>(bits) : 0.f;
      qv[j * 8 + r] = x;
      qmax = fmaxf(qmax, fabsf(x));
    }
  qmax = col_max(qmax);
  const int kq = qmax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(qmax) : 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r)
      qf[j][r] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(qv[j * 8 + r], kq));
  return __builtin_amdgcn_ldexpf(a.scale_log2, -kq);
}

// q for the integer matrix instructions of the page-pair kernels: the lane's
// 16 dims of each 64-dim chunk i (chunk(2i), chunk(2i + 1)) as integers
// qi = rint(q * 2^kq) with max|qi| of the head in [2^21, 2^22], in base 256
// with signed digits: qi = 2^16 a + 2^8 b + c (a, b, c in [-128, 127]; the
// bytes of qi + 0x808080 are a + 128, b + 128, c + 128), digit p of chunk i
// one byte per dim.
// The lanes of MFMA columns 0-7 keep the digits in qa (page a of a pair) and
// zeros in qb, those of columns 8-15 the reverse, so that one chain of matrix
// instructions over both pages leaves page a's sums in columns 0-7 and page
// b's in columns 8-15. Products and sums are exact in int32; rounding q costs
// at most 2^-22 of the head's largest element per element. (Two digits, 2^-14
// of the largest element, measured up to 0.2 off the exact attention on rows
// whose q has outlier channels: the small elements keep too few bits.)
// Returns the factor that turns 2^16 A + 2^8 B + C into base-2 logits.
typedef int i4_t __attribute__((ext_vector_type(4)));
template <int NI, bool QBF16, typename ChunkFn>
__device__ __forceinline__ float load_q_pieces(const DecodeArgs& a, bool hvalid, ChunkFn chunk,
                                               i4_t (*qa)[3], i4_t (*qb)[3]) {
  u4_t raw[2 * NI];
#pragma unroll
  for (int j = 0; j < 2 * NI; ++j) raw[j] = chunk(j);
  float qv[NI * 16];
  float qmax = 0.f;
#pragma unroll
  for (int j = 0; j < 2 * NI; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint16_t bits = static_cast<uint16_t>(raw[j][r / 2] >> (16 * (r % 2)));
      const float x = hvalid ? bits16_to_f32<QBF16>(bits) : 0.f;
      qv[j * 8 + r] = x;
      qmax = fmaxf(qmax, fabsf(x));
    }
  qmax = col_max(qmax);
  const int kq = qmax > 0.f ? 22 - __builtin_amdgcn_frexp_expf(qmax) : 0;
  const float f = __builtin_amdgcn_ldexpf(1.0f, kq);
  const bool hi = (lane_id() & 8) != 0;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[e] = static_cast<uint32_t>(static_cast<int>(rintf(qv[i * 16 + 4 * w + e] * f))) +
               0x808080u;
      // byte k of the four values into one word, offset removed (xor 0x80)
      auto digit = [&u](uint32_t lo_sel, uint32_t hi_sel) {
        return static_cast<int>((__builtin_amdgcn_perm(u[1], u[0], lo_sel) |
                                 __builtin_amdgcn_perm(u[3], u[2], hi_sel)) ^
                                0x80808080u);
      };
      const int d[3] = {digit(0x0c0c0602u, 0x06020c0cu),   // a
                        digit(0x0c0c0501u, 0x05010c0cu),   // b
                        digit(0x0c0c0400u, 0x04000c0cu)};  // c
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        qa[i][p][w] = hi ? 0 : d[p];
        qb[i][p][w] = hi ? d[p] : 0;
      }
    }
  return __builtin_amdgcn_ldexpf(a.scale_log2, -kq);
}

// ---------------------------------------------------------------------------
// INT8 pages
// ---------------------------------------------------------------------------
template <int D>
struct Int8Page {
  u4_t k[D / 64];  // K codes: token i16, dims 64*i + 16*kb + (0..15)
  u4_t v[D / 64];  // V codes: dims 64*i + 4*i16 + (0..3), tokens 4*kb + (0..3)
  u2_t ks, vs;     // scales of tokens 4*kb + (0..3)
};

// One KV head's part of a page: its code block (K then V; 16-bit values in
// the 16-bit format) and, for per-token INT8, the byte distance from there to
// the head's scale records (every head's code block comes first in an INT8
// page, then every head's scales, so that the code blocks stay aligned).
struct HeadRef {
  const uint8_t* code;
  int scales;
};
template <class K>
__device__ __forceinline__ HeadRef head_ref(const DecodeArgs& a, int blk, int g) {
  // (wave-uniform: the address stays in scalar registers, as the buffer
  // resource requires; a missing page (blk < 0) points at page 0)
  blk = __builtin_amdgcn_readfirstlane(blk);
  g = __builtin_amdgcn_readfirstlane(g);
  const int64_t page = blk >= 0 ? blk : 0;
  return {a.pool + page * a.page_bytes + g * K::kCodeBytes,
          (a.num_kv_heads - g) * K::kCodeBytes + g * K::kScaleBytes};
}

// Page reads go through a buffer resource made for each page's head (base
// in SGPRs, 32-bit lane offsets, constant parts in the instruction's offset
// field): no 64-bit per-lane address arithmetic, and a read outside the
// resource would return 0 instead of touching other memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_block(const uint8_t* hp, int bytes) {
  // (the size is wave-uniform; saying so keeps the resource in scalar
  // registers, without a loop over distinct lane values)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(hp), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Page bytes are read once per call: the loads carry the non-temporal
// (streaming) cache policy, so they do not displace what the caches hold for
// reuse (measured: the batched step's INT8 call 3% and its 16-bit call 11%
// faster, the 8K and 32K decodes unchanged).
constexpr int kStreamLoad = 2;  // cache-policy bits: nt
__device__ __forceinline__ u4_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamLoad));
}

// (the resource runs from the head's code block to the end of its scale
// records, all inside the page)
template <int D>
__device__ __forceinline__ void load_int8_page(Int8Page<D>& pg, HeadRef h, bool live, int i16,
                                               int kb) {
  const __amdgpu_buffer_rsrc_t r = head_block(h.code, live ? h.scales + 64 : 0);
  const uint32_t ko = i16 * D + 16 * kb;      // K: token i16
  const uint32_t vo = kb * 4 * D + 16 * i16;  // V: token group kb (after 16*D)
#pragma unroll
  for (int i = 0; i < D / 64; ++i) pg.k[i] = ld16(r, ko + 64 * i);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) pg.v[i] = ld16(r, vo + 16 * D + 256 * i);
  // the record of tokens 4*kb .. 4*kb+3: four K scales, then four V scales
  const u4_t sc = ld16(r, h.scales + 16 * kb);
  pg.ks = u2_t{sc.x, sc.y};
  pg.vs = u2_t{sc.z, sc.w};
}

// The matrix-instruction operands of a page's codes, converted where they
// are used: K fragment j (the A operand of QK instruction j: 8 codes of
// token i16) and V fragment k (the A operand of PV instruction k: one
// dimension of four tokens), as fp16.
template <class Pg>
__device__ __forceinline__ h8_t k_frag(const Pg& pg, int j) {
  const u2_t c0 = i8x4_to_f16x4_perm(pg.k[j / 2][2 * (j % 2)]);
  const u2_t c1 = i8x4_to_f16x4_perm(pg.k[j / 2][2 * (j % 2) + 1]);
  return __builtin_bit_cast(h8_t, u4_t{c0.x, c0.y, c1.x, c1.y});
}
template <class Pg>
__device__ __forceinline__ h4_t v_frag(const Pg& pg, int k) {
  return __builtin_bit_cast(h4_t, i8x4_to_f16x4_perm(pg.v[k / 4][k % 4]));
}

template <int D, class Pg>
__device__ __forceinline__ f4_t int8_qk(const Pg& pg, const h8_t* qf) {
  f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_frag(pg, j), qf[j], s, 0, 0, 0);
  return s;
}

// High fp16 parts of four binary32 probabilities (rounded toward zero, one
// conversion instruction per pair) and the fp16 rests p - hi, so that
// hi + lo carries 22 significant bits of p.
__device__ __forceinline__ h4_t split_hi(const float (&p)[4]) {
  const auto a = __builtin_amdgcn_cvt_pkrtz(p[0], p[1]);
  const auto b = __builtin_amdgcn_cvt_pkrtz(p[2], p[3]);
  return __builtin_bit_cast(h4_t, u2_t{__builtin_bit_cast(uint32_t, a),
                                       __builtin_bit_cast(uint32_t, b)});
}
__device__ __forceinline__ h4_t split_lo(const float (&p)[4], h4_t hi) {
  float lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) lo[j] = p[j] - static_cast<float>(hi[j]);
  return __builtin_bit_cast(h4_t, u2_t{pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3])});
}

// Position of this lane's first token in a page starting at page_tok: lane
// (i16, kb) holds tokens 4*kb + (0..3) of the tile.
__device__ __forceinline__ int lane_token(int page_tok) {
  return page_tok + 4 * static_cast<int>((threadIdx.x & 63) >> 4);
}

// Limits of one page step: tokens at or past L (wave-uniform: the context
// length, or the page start for a skipped page) hold no data; the lane's
// query column attends to tokens below Lc (<= L; below L only for the
// earlier tokens of a multi-token query); Lmin (wave-uniform) is the
// smallest Lc of the wave, so pages below it need no mask at all.

// One page starting at token page_tok (wave-uniform). The tokens at or past
// L get V scale 1.0 (their slots may hold anything); those at or past Lc get
// logit -inf. (A separate unmasked path for full pages costs more registers
// than the masks cost instructions.)
// The scale terms of the lane's four tokens 4*kb + (0..3): the K scale, and
// the V scale sV = f * 2^e (f in [0.5, 1)) as its exponent and mantissa;
// tokens at or past L (tail pages only) get V scale 1.0, as their slots may
// hold anything.
struct TokenScales {
  _Float16 sk[4];
  int e[4];
  _Float16 f[4];
};
__device__ __forceinline__ TokenScales token_scales_w(u2_t ks, u2_t vs, bool tail, int tok0,
                                                      int L) {
  const uint32_t ksw[2] = {ks.x, ks.y};
  uint32_t vsw[2] = {vs.x, vs.y};
  if (tail) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tok0 + j >= L) vsw[j / 2] = (vsw[j / 2] & (0xFFFF0000u >> (16 * (j % 2)))) |
                                      (0x3C00u << (16 * (j % 2)));
  }
  TokenScales ts;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ts.sk[j] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(ksw[j / 2] >> (16 * (j % 2))));
    const _Float16 sv =
        __builtin_bit_cast(_Float16, static_cast<uint16_t>(vsw[j / 2] >> (16 * (j % 2))));
    ts.e[j] = __builtin_amdgcn_frexp_exph(sv);
    ts.f[j] = __builtin_amdgcn_frexp_manth(sv);
  }
  return ts;
}
template <class Pg>
__device__ __forceinline__ TokenScales token_scales(const Pg& pg, bool tail, int tok0, int L) {
  return token_scales_w(pg.ks, pg.vs, tail, tok0, L);
}

// Softmax update of one query tile from its logit tile s: base-2 logits
// plus the V scale's exponent (P = 2^(z - m) * f), tokens at or past Lc
// masked, running max and sum, and the probabilities (V scale folded in) as
// high and low fp16 parts for the PV product.
template <bool Pair = false, int ND>
__device__ __forceinline__ void int8_probs(const f4_t& s, const TokenScales& ts, float qscale,
                                           bool tail, int tok0, int Lc, SoftmaxState<ND>& st,
                                           h4_t& ph, h4_t& pl) {
  // (the fp16 scale factors enter as mixed-precision fma operands; only a
  // tail page pays the mask, one compare per logit against the lane's count
  // of attendable tokens)
  float z[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    z[j] = fmaf(s[j] * qscale, static_cast<float>(ts.sk[j]), static_cast<float>(ts.e[j]));
  if (tail) {
    const int lim = Lc - tok0;
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = j < lim ? z[j] : -INFINITY;
  }
  raise_max<Pair>(st, fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
  float x[4], p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = __builtin_amdgcn_exp2f(z[j] - st.mk);  // 2^(kPScale + z - m)
    st.l += __builtin_amdgcn_ldexpf(x[j], -ts.e[j]);
    p[j] = fmaf(x[j], static_cast<float>(ts.f[j]), 0.f);  // = x * f (x, f >= 0)
  }
  // x * f = hi + lo to 22 bits: hi is p converted to fp16 once (by the
  // conversion instruction itself, so that the compiler cannot fold the
  // product into a second, differently rounded conversion), lo the exact
  // rest x * f - hi (one fma) rounded to fp16
  ph = split_hi(p);
  float lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    lo[j] = fmaf(x[j], static_cast<float>(ts.f[j]), -static_cast<float>(ph[j]));
  pl = __builtin_bit_cast(h4_t, u2_t{pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3])});
}

// One page starting at token page_tok (wave-uniform). The tokens at or past
// L get V scale 1.0 (their slots may hold anything); those at or past Lc get
// logit -inf. (A separate unmasked path for full pages costs more registers
// than the masks cost instructions.)
template <int D, class Pg>
__device__ __forceinline__ void int8_page_step(const Pg& pg, const h8_t* qf,
                                               float qscale, int page_tok, int L, int Lmin,
                                               int Lc, SoftmaxState<D / 16>& st) {
  constexpr int ND = D / 16;
  const f4_t s = int8_qk<D>(pg, qf);
  const bool tail = page_tok + kBlockSize > Lmin;
  const int tok0 = tail ? lane_token(page_tok) : 0;
  const TokenScales ts = token_scales(pg, tail, tok0, L);
  h4_t ph, pl;
  int8_probs(s, ts, qscale, tail, tok0, Lc, st, ph, pl);
  // O^T += V^T P^T; instruction k covers dims 64*(k/4) + 4*(row) + k%4, its
  // K-slots hold tokens 4*kb + (0..3)
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    const h4_t vw = v_frag(pg, k);
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, ph, st.acc[k], 0, 0, 0);
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, pl, st.acc[k], 0, 0, 0);
  }
}

// INT8 pages with static scales: the codes only, laid out as in the
// per-token page (one calibrated scalar for all of K and one for all of V;
// InfiniLM PR #553 "Summary", TensorRT-LLM PR #18953 "Summary"). The K scale
// is folded into the logit factor on the host and the V scale multiplies the
// final output, so a page step is the per-token step without the scales.
template <int D>
struct StaticPage {
  u4_t k[D / 64];  // as Int8Page
  u4_t v[D / 64];
};

template <int D>
__device__ __forceinline__ void load_static_page(StaticPage<D>& pg, HeadRef h, bool live, int i16,
                                                 int kb) {
  const __amdgpu_buffer_rsrc_t r = head_block(h.code, live ? 32 * D : 0);
  const uint32_t ko = i16 * D + 16 * kb;
  const uint32_t vo = kb * 4 * D + 16 * i16;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) pg.k[i] = ld16(r, ko + 64 * i);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) pg.v[i] = ld16(r, vo + 16 * D + 256 * i);
}

// Tokens at or past the limit L get logit -inf (probability 0; any byte in
// their slots is a finite code, so 0 * code adds nothing).
// Softmax update of one query tile over static-scale codes (the K scale is
// part of qscale): tokens at or past Lc masked (any byte in a slot past the
// context is a finite code, so 0 * code adds nothing), running max and sum,
// probabilities as high and low fp16 parts.
template <bool Pair = false, int ND>
__device__ __forceinline__ void static_probs(const f4_t& s, float qscale, bool tail, int tok0,
                                             int Lc, SoftmaxState<ND>& st, h4_t& ph, h4_t& pl) {
  float z[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = s[j] * qscale;
  if (tail) {
    const int lim = Lc - tok0;  // the lane's attendable tokens
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = j < lim ? z[j] : -INFINITY;
  }
  raise_max<Pair>(st, fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = __builtin_amdgcn_exp2f(z[j] - st.mk);  // 2^(kPScale + z - m)
    st.l += x[j];
  }
  ph = split_hi(x);
  pl = split_lo(x, ph);
}

template <int D, class Pg>
__device__ __forceinline__ void static_page_step(const Pg& pg, const h8_t* qf,
                                                 float qscale, int page_tok, int Lmin, int Lc,
                                                 SoftmaxState<D / 16>& st) {
  constexpr int ND = D / 16;
  const f4_t s = int8_qk<D>(pg, qf);
  const bool tail = page_tok + kBlockSize > Lmin;
  const int tok0 = tail ? lane_token(page_tok) : 0;
  h4_t ph, pl;
  static_probs(s, qscale, tail, tok0, Lc, st, ph, pl);
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    const h4_t vw = v_frag(pg, k);
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, ph, st.acc[k], 0, 0, 0);
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, pl, st.acc[k], 0, 0, 0);
  }
}

// Two consecutive pages a, b of one segment against one query tile for a
// group of at most 8 heads: the tile's 16 MFMA columns hold the heads twice,
// columns 0-7 (lanes with i16 < 8) for page a and 8-15 for page b, so one
// softmax update covers 32 tokens. In QK, page a's codes meet q in columns
// 0-7 only and page b's in columns 8-15 (zeros in the other half), so one
// chain of matrix instructions leaves each lane its own page's logits; in
// PV, page a's V meets
// the probabilities of the columns 0-7 only (zeros in the others) and page
// b's V those of columns 8-15, into one accumulator whose two column halves
// share the running max and add up when the segment ends (fold_pair).
// La, Lb: the pages' limits (a missing page gets its first token: masked).
// QK of a page pair on the integer matrix cores: the codes as they were
// loaded (K fragment i = the lane's 16 codes of chunk i) against the three q
// digits, page a's against qa and page b's against qb into the same three
// exact int32 sums per logit.
template <int D, class Pg>
__device__ __forceinline__ void int8_pair_qk(const Pg& pa, const Pg& pb, const i4_t (*qa)[3],
                                             const i4_t (*qb)[3], i4_t (&acc)[3]) {
#pragma unroll
  for (int p = 0; p < 3; ++p) acc[p] = i4_t{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
#pragma unroll
    for (int p = 0; p < 3; ++p)
      acc[p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, pa.k[i]), qa[i][p],
                                                     acc[p], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
#pragma unroll
    for (int p = 0; p < 3; ++p)
      acc[p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i4_t, pb.k[i]), qb[i][p],
                                                     acc[p], 0, 0, 0);
}
template <int D, bool Static, class Pg>
__device__ __forceinline__ void int8_pair_step(const Pg& pa, const Pg& pb, const i4_t (*qa)[3],
                                               const i4_t (*qb)[3], float qscale, int tok_a,
                                               int La, int Lb, SoftmaxState<D / 16>& st) {
  constexpr int ND = D / 16;
  const bool hi = (threadIdx.x & 8) != 0;
  i4_t acc[3];
  int8_pair_qk<D>(pa, pb, qa, qb, acc);
  // 2^16 A + 2^8 B + C (B and C combined exactly in int32, then one fp32
  // rounding each for the conversion and the fma)
  f4_t s;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    s[r] = fmaf(static_cast<float>(acc[0][r]), 65536.f,
                static_cast<float>(acc[1][r] * 256 + acc[2][r]));
  // (wave-uniform: a scalar branch)
  const bool tail = __builtin_amdgcn_readfirstlane(tok_a + 2 * kBlockSize > min(La, Lb));
  const int L = hi ? Lb : La;
  const int tok0 = tail ? lane_token(tok_a + (hi ? kBlockSize : 0)) : 0;
  h4_t ph, pl;
  if constexpr (Static) {
    static_probs<true>(s, qscale, tail, tok0, L, st, ph, pl);
  } else {
    const TokenScales ts =
        token_scales_w(hi ? pb.ks : pa.ks, hi ? pb.vs : pa.vs, tail, tok0, L);
    int8_probs<true>(s, ts, qscale, tail, tok0, L, st, ph, pl);
  }
  // PV over both pages in one 16x16x32 instruction per dim block and part:
  // the lane's eight K-slots hold its four tokens of page a, then the same
  // four of page b, in V and in P alike (P zero for the other page's half)
  const u2_t z2 = {0u, 0u};
  const u2_t ph2 = __builtin_bit_cast(u2_t, ph), pl2 = __builtin_bit_cast(u2_t, pl);
  const u2_t pha = hi ? z2 : ph2, pla = hi ? z2 : pl2;
  const u2_t phb = hi ? ph2 : z2, plb = hi ? pl2 : z2;
  const h8_t p_hi = __builtin_bit_cast(h8_t, u4_t{pha.x, pha.y, phb.x, phb.y});
  const h8_t p_lo = __builtin_bit_cast(h8_t, u4_t{pla.x, pla.y, plb.x, plb.y});
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    const u2_t va = __builtin_bit_cast(u2_t, v_frag(pa, k));
    const u2_t vb = __builtin_bit_cast(u2_t, v_frag(pb, k));
    const h8_t v8 = __builtin_bit_cast(h8_t, u4_t{va.x, va.y, vb.x, vb.y});
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v8, p_hi, st.acc[k], 0, 0, 0);
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v8, p_lo, st.acc[k], 0, 0, 0);
  }
}

// End of a pair segment: add the column halves (page a's and page b's
// tokens of each head; same running max), in every lane of the row.
template <int ND>
__device__ __forceinline__ void fold_pair(SoftmaxState<ND>& st) {
#pragma unroll
  for (int k = 0; k < ND; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) st.acc[k][j] += row_partner8(st.acc[k][j]);
  st.l += row_partner8(st.l);
}

// Fused append: the lane's D / 64 elements (dims lane * D / 64 + e) of the
// newest token's K and V rows of sequence b, KV head g (16-bit patterns).
template <int D>
struct NewRows {
  uint16_t k[D / 64], v[D / 64];
};
template <int D>
__device__ __forceinline__ NewRows<D> load_new_rows(const DecodeArgs& a, int b, int g, int lane) {
  constexpr int EPL = D / 64;
  const uint16_t* kn = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(a.v_new);
  NewRows<D> r;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int64_t d = lane * EPL + e;
    r.k[e] = kn[b * a.kn_st + g * a.kn_sh + d * a.kn_sd];
    r.v[e] = vn[b * a.vn_st + g * a.vn_sh + d * a.vn_sd];
  }
  return r;
}

// The INT8 page formats as seen by the decode loop: per-token FP16 scales in
// the page, or (Static) codes only with the layer's two scalar scales.
template <int D_, bool QBF16, int G_ = 1, bool Static = false, bool Pair = false>
struct Int8Kind {
  static constexpr int D = D_;
  static constexpr int kGroup = G_;  // pages per register buffer
  // pairs of pages per softmax update (one-token calls, groups of <= 8 heads)
  static constexpr bool kPair = Pair;
  static_assert(!Pair || G_ == 2, "a pair kind streams pages two by two");
  // the head of MFMA column i16
  static __device__ __forceinline__ int col_head(int i16) { return Pair ? (i16 & 7) : i16; }
  static constexpr int kCodeBytes = 32 * D;            // a head's K and V codes
  static constexpr int kScaleBytes = Static ? 0 : 64;  // a head's scale records
  using Page = typename std::conditional<Static, StaticPage<D>, Int8Page<D>>::type;
  h8_t qf[D / 32];                   // fp16 q fragments (one page per update)
  i4_t qa[D / 64][3], qb[D / 64][3];  // integer q digits for pages a, b (pair kinds)
  float qscale;

  // q of head i16 from the unit's rows in LDS ([G][D] 16-bit values)
  __device__ __forceinline__ void load_q(const DecodeArgs& a, const uint16_t* q_rows, int i16,
                                         int kb, bool hvalid) {
    const uint16_t* row = q_rows + (hvalid ? i16 : 0) * D;
    auto chunk = [row, kb](int j) {
      return *reinterpret_cast<const u4_t*>(row + 64 * (j / 2) + 16 * kb + 8 * (j % 2));
    };
    if constexpr (Pair)
      qscale = load_q_pieces<D / 64, QBF16>(a, hvalid, chunk, qa, qb);
    else
      qscale = load_q_scaled<D / 32, QBF16>(a, hvalid, chunk, qf);
  }
  static __device__ __forceinline__ void load(Page& pg, HeadRef h, bool live, int i16, int kb) {
    if constexpr (Static)
      load_static_page<D>(pg, h, live, i16, kb);
    else
      load_int8_page<D>(pg, h, live, i16, kb);
  }
  // one page against this query tile
  __device__ __forceinline__ void step(const Page& pg, int page_tok, int L, int Lmin, int Lc,
                                       SoftmaxState<D / 16>& st) const {
    if constexpr (Static)
      static_page_step<D>(pg, qf, qscale, page_tok, Lmin, Lc, st);
    else
      int8_page_step<D>(pg, qf, qscale, page_tok, L, Lmin, Lc, st);
  }
  // two consecutive pages of one segment (pair kinds)
  __device__ __forceinline__ void step_pair(const Page& pa, const Page& pb, int tok_a, int La,
                                            int Lb, SoftmaxState<D / 16>& st) const {
    int8_pair_step<D, Static>(pa, pb, qa, qb, qscale, tok_a, La, Lb, st);
  }
  // One page against the first nt of NT query tiles (tile c: q fragments
  // kd[c], state st[c], column limit Lc[c]), two tiles at a time: every K and
  // V fragment is converted once per pair of tiles and fed to the matrix
  // instructions of both, and the token scales are decoded once per pair.
  // (Four tiles at once need more registers than one wave has.)
  template <int NT>
  static __device__ __forceinline__ void step_tiles(const Page& pg, const Int8Kind* kd, int nt,
                                                    int page_tok, int L, int Lmin,
                                                    const int* Lc, SoftmaxState<D / 16>* st) {
    if constexpr (NT > 2) {
#pragma unroll
      for (int c = 0; c < NT; c += 2) {
        if (c < nt) step_tiles<2>(pg, kd + c, nt - c, page_tok, L, Lmin, Lc + c, st + c);
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    constexpr int ND = D / 16;
    f4_t s[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) s[c] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const h8_t kf = k_frag(pg, j);
#pragma unroll
      for (int c = 0; c < NT; ++c)
        if (c < nt) s[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, kd[c].qf[j], s[c], 0, 0, 0);
    }
    const bool tail = page_tok + kBlockSize > Lmin;
    const int tok0 = tail ? lane_token(page_tok) : 0;
    h4_t ph[NT], pl[NT];
    // (the tiles' softmax updates one after the other: interleaving them
    // costs registers)
    if constexpr (Static) {
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        if (c < nt) static_probs(s[c], kd[c].qscale, tail, tok0, Lc[c], st[c], ph[c], pl[c]);
      }
    } else {
      const TokenScales ts = token_scales(pg, tail, tok0, L);
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        if (c < nt) int8_probs(s[c], ts, kd[c].qscale, tail, tok0, Lc[c], st[c], ph[c], pl[c]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      const h4_t vw = v_frag(pg, k);
#pragma unroll
      for (int c = 0; c < NT; ++c)
        if (c < nt) {
          st[c].acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, ph[c], st[c].acc[k], 0, 0, 0);
          st[c].acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, pl[c], st[c].acc[k], 0, 0, 0);
        }
    }
  }
  // dimension of accumulator element acc[k][j] in lane (i16, kb)
  static __device__ __forceinline__ int acc_dim(int k, int j, int kb) {
    return 64 * (k / 4) + 16 * kb + 4 * j + (k % 4);
  }

  // Fused append, first half: quantize the newest token's K and V rows
  // (the lane's elements r, loaded by load_new_rows) with the
  // quantize-on-write rule into nt ([D] K codes, [D] V codes, K scale, V
  // scale) for patch() and store_new(). False when a scale would exceed FP16
  // or a row holds a NaN or an infinity (flagged; the slot is then left as it
  // was, as the separate write leaves it).
  static __device__ __forceinline__ bool quant_new(const DecodeArgs& a, const NewRows<D>& r,
                                                   uint8_t* nt, int lane) {
    constexpr int EPL = D / 64;
    float xk[EPL], xv[EPL];
    // row maxima as 16-bit magnitude patterns (sign bit cleared): FP16 and
    // BF16 magnitudes order like unsigned integers, with a NaN above the
    // infinity, so a NaN or an infinity reaches the scale check
    uint32_t mk = 0, mv = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xk[e] = bits16_to_f32<QBF16>(r.k[e]);
      xv[e] = bits16_to_f32<QBF16>(r.v[e]);
      mk = max(mk, static_cast<uint32_t>(r.k[e] & 0x7FFFu));
      mv = max(mv, static_cast<uint32_t>(r.v[e] & 0x7FFFu));
    }
    if constexpr (Static) {
      // the layer's scales: nothing can overflow
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        nt[d] = row_code(xk[e], a.k_scale);
        nt[D + d] = row_code(xv[e], a.v_scale);
      }
      return true;
    }
    const float ak = bits16_to_f32<QBF16>(static_cast<uint16_t>(wave_max_u32(mk)));
    const float av = bits16_to_f32<QBF16>(static_cast<uint16_t>(wave_max_u32(mv)));
    uint16_t skb, svb;
    const bool okk = row_scale(ak, skb), okv = row_scale(av, svb);
    if (!okk || !okv) {
      if (lane == 0) raise_flag(a.err, PDAKV_EFLAG_SCALE_RANGE);
      return false;
    }
    const float sk = f16_bits_to_f32(skb), sv = f16_bits_to_f32(svb);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane * EPL + e;
      nt[d] = row_code(xk[e], sk);
      nt[D + d] = row_code(xv[e], sv);
    }
    if (lane == 0) {
      *reinterpret_cast<uint16_t*>(nt + 2 * D) = skb;
      *reinterpret_cast<uint16_t*>(nt + 2 * D + 2) = svb;
    }
    return true;
  }
  static __device__ __forceinline__ bool prepare_new(const DecodeArgs& a, int b, int g,
                                                     uint8_t* nt, int lane) {
    return quant_new(a, load_new_rows<D>(a, b, g, lane), nt, lane);
  }

  // Fused append, second half (after the page loop): store the token from nt
  // at position pos of head h.
  static __device__ __forceinline__ void store_new(const DecodeArgs& a, const uint8_t* nt,
                                                   int pos, HeadRef h, int lane) {
    uint8_t* head = const_cast<uint8_t*>(h.code);
    for (int d = lane; d < D; d += 64) {
      head[pos * D + d] = nt[d];
      head[16 * D + (pos >> 2) * 4 * D + 4 * d + (pos & 3)] = nt[D + d];
    }
    if (!Static && lane == 0) {
      uint8_t* rec = head + h.scales + 16 * (pos >> 2) + 2 * (pos & 3);
      *reinterpret_cast<uint16_t*>(rec) = *reinterpret_cast<const uint16_t*>(nt + 2 * D);
      *reinterpret_cast<uint16_t*>(rec + 8) = *reinterpret_cast<const uint16_t*>(nt + 2 * D + 2);
    }
  }

  // Put the appended token (from nt) into the registers of its page as
  // loaded: K row in the lanes of token pos, V bytes and scales in the lanes
  // of its token group.
  static __device__ __forceinline__ void patch(Page& pg, const uint8_t* nt, int pos, int i16,
                                               int kb) {
    if (i16 == pos) {
#pragma unroll
      for (int i = 0; i < D / 64; ++i)
        pg.k[i] = *reinterpret_cast<const u4_t*>(nt + 64 * i + 16 * kb);
    }
    if (kb == (pos >> 2)) {
      const int sh = 8 * (pos & 3);
      const uint32_t keep = ~(0xFFu << sh);
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(nt + D + 64 * i + 4 * i16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pg.v[i][j] = (pg.v[i][j] & keep) | (((w >> (8 * j)) & 0xFFu) << sh);
      }
      if constexpr (!Static) patch_scales(pg, nt, pos);
    }
  }

  // the appended token's K and V scales into the scale words of its group
  static __device__ __forceinline__ void patch_scales(Page& pg, const uint8_t* nt, int pos) {
    const int hs = 16 * (pos & 1);
    const uint32_t hkeep = ~(0xFFFFu << hs);
    const uint32_t kbits = *reinterpret_cast<const uint16_t*>(nt + 2 * D);
    const uint32_t vbits = *reinterpret_cast<const uint16_t*>(nt + 2 * D + 2);
    if ((pos & 3) < 2) {
      pg.ks.x = (pg.ks.x & hkeep) | (kbits << hs);
      pg.vs.x = (pg.vs.x & hkeep) | (vbits << hs);
    } else {
      pg.ks.y = (pg.ks.y & hkeep) | (kbits << hs);
      pg.vs.y = (pg.vs.y & hkeep) | (vbits << hs);
    }
  }
};

// ---------------------------------------------------------------------------
// 16-bit pages (control)
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ f4_t mfma16x16x32(u4_t a_bits, u4_t b_bits, f4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a_bits),
                                                   __builtin_bit_cast(b8_t, b_bits), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a_bits),
                                                  __builtin_bit_cast(h8_t, b_bits), c, 0, 0, 0);
}

template <int D>
struct Page16 {
  u4_t k[D / 32];  // K: token i16, dims 32*j + 8*kb + (0..7)
  u4_t v[D / 32];  // V: dims 32*i + 2*i16 + (0,1), tokens 4*kb + (0..3)
};

template <int D>
__device__ __forceinline__ void load_page16(Page16<D>& pg, HeadRef h, bool live, int i16,
                                            int kb) {
  const __amdgpu_buffer_rsrc_t r = head_block(h.code, live ? 64 * D : 0);
  const uint32_t ko = i16 * 2 * D + 16 * kb;
  const uint32_t vo = 32 * D + kb * 8 * D + 16 * i16;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) pg.k[j] = ld16(r, ko + 64 * j);
#pragma unroll
  for (int i = 0; i < D / 32; ++i) pg.v[i] = ld16(r, vo + 256 * i);
}

template <bool BF16>
__device__ __forceinline__ f4_t mfma16x16x16(u2_t a_bits, u2_t b_bits, f4_t c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a_bits),
                                                     __builtin_bit_cast(s4_t, b_bits), c, 0, 0,
                                                     0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a_bits),
                                                 __builtin_bit_cast(h4_t, b_bits), c, 0, 0, 0);
}

template <int D, bool BF16>
__device__ __forceinline__ void page16_step(const Page16<D>& pg, const u4_t* qf,
                                            float scale_log2, int page_tok, int L, int Lmin,
                                            int Lc, SoftmaxState<D / 16>& st) {
  constexpr int NJ = D / 32, ND = D / 16;
  f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) s = mfma16x16x32<BF16>(pg.k[j], qf[j], s);
  const bool tail = page_tok + kBlockSize > Lmin;
  const int tok0 = tail ? lane_token(page_tok) : 0;
  float z[4];
  float zmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z[j] = s[j] * scale_log2;
    if (tail) z[j] = tok0 + j < Lc ? z[j] : -INFINITY;
    zmax = max_nc(zmax, z[j]);
  }
  raise_max(st, zmax);
  float pe[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pe[j] = __builtin_amdgcn_exp2f(z[j] - st.mk);
    st.l += pe[j];
  }
  // V of masked tokens -> 0 (a slot past the context may hold NaN bits, and
  // 0 * NaN would reach the accumulator). Word 2r + w of pg.v[i] holds
  // tokens 2w, 2w+1 of one dimension.
  u4_t v[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) v[i] = pg.v[i];
  if (tail) {
    const uint32_t m01 = (tok0 < L ? 0xFFFFu : 0u) | (tok0 + 1 < L ? 0xFFFF0000u : 0u);
    const uint32_t m23 = (tok0 + 2 < L ? 0xFFFFu : 0u) | (tok0 + 3 < L ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      v[i][0] &= m01;
      v[i][1] &= m23;
      v[i][2] &= m01;
      v[i][3] &= m23;
    }
  }
  if constexpr (BF16) {
    // exact three-way split into truncated bf16 parts (8 + 8 + 8 bits)
    uint32_t p1[4], p2[4], p3[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = __float_as_uint(pe[j]);
      p1[j] = u >> 16;
      const float r1 = pe[j] - __uint_as_float(u & 0xFFFF0000u);
      const uint32_t u1 = __float_as_uint(r1);
      p2[j] = u1 >> 16;
      const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
      p3[j] = __float_as_uint(r2) >> 16;
    }
    const u2_t w1 = {p1[0] | (p1[1] << 16), p1[2] | (p1[3] << 16)};
    const u2_t w2 = {p2[0] | (p2[1] << 16), p2[2] | (p2[3] << 16)};
    const u2_t w3 = {p3[0] | (p3[1] << 16), p3[2] | (p3[3] << 16)};
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      const u2_t vw = {v[k / 2][2 * (k % 2)], v[k / 2][2 * (k % 2) + 1]};
      st.acc[k] = mfma16x16x16<true>(vw, w1, st.acc[k]);
      st.acc[k] = mfma16x16x16<true>(vw, w2, st.acc[k]);
      st.acc[k] = mfma16x16x16<true>(vw, w3, st.acc[k]);
    }
  } else {
    float hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hi[j] = static_cast<float>(static_cast<_Float16>(pe[j]));
      lo[j] = pe[j] - hi[j];
    }
    const u2_t ph = {pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3])};
    const u2_t pl = {pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3])};
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      const u2_t vw = {v[k / 2][2 * (k % 2)], v[k / 2][2 * (k % 2) + 1]};
      st.acc[k] = mfma16x16x16<false>(vw, ph, st.acc[k]);
      st.acc[k] = mfma16x16x16<false>(vw, pl, st.acc[k]);
    }
  }
}

// The 16-bit page format as seen by the decode loop (q stays in K's dtype).
template <int D_, bool BF16, int G_ = 1>
struct F16Kind {
  static constexpr int D = D_;
  static constexpr int kGroup = G_;  // pages per register buffer
  static constexpr bool kPair = false;
  static __device__ __forceinline__ int col_head(int i16) { return i16; }
  static constexpr int kCodeBytes = 64 * D;  // a head's K and V values
  static constexpr int kScaleBytes = 0;
  using Page = Page16<D>;
  u4_t qf[D / 32];  // fragment j: dims 32*j + 8*kb + (0..7)
  float scale_log2;

  __device__ __forceinline__ void load_q(const DecodeArgs& a, const uint16_t* q_rows, int i16,
                                         int kb, bool hvalid) {
    const uint16_t* row = q_rows + (hvalid ? i16 : 0) * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) qf[j] = *reinterpret_cast<const u4_t*>(row + 32 * j + 8 * kb);
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
      if (!hvalid) qf[j] = u4_t{0u, 0u, 0u, 0u};
    scale_log2 = a.scale_log2;
  }
  static __device__ __forceinline__ void load(Page& pg, HeadRef h, bool live, int i16, int kb) {
    load_page16<D>(pg, h, live, i16, kb);
  }
  __device__ __forceinline__ void step(const Page& pg, int page_tok, int L, int Lmin, int Lc,
                                       SoftmaxState<D / 16>& st) const {
    page16_step<D, BF16>(pg, qf, scale_log2, page_tok, L, Lmin, Lc, st);
  }
  // One page against the first nt of NT query tiles: 16-bit values need no
  // conversion, so each tile runs its own step on the loaded page.
  template <int NT>
  static __device__ __forceinline__ void step_tiles(const Page& pg, const F16Kind* kd, int nt,
                                                    int page_tok, int L, int Lmin,
                                                    const int* Lc, SoftmaxState<D / 16>* st) {
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      if (c < nt) kd[c].step(pg, page_tok, L, Lmin, Lc[c], st[c]);
      // one tile after the other (interleaving them costs registers)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  static __device__ __forceinline__ int acc_dim(int k, int j, int kb) {
    return 32 * (k / 2) + 8 * kb + 2 * j + (k % 2);
  }

  // Fused append, first half: the newest token's K and V rows (the lane's
  // elements r, loaded by load_new_rows) into nt ([D] K, [D] V, 16-bit) for
  // patch() and store_new().
  static __device__ __forceinline__ bool quant_new(const DecodeArgs&, const NewRows<D>& r,
                                                   uint8_t* nt, int lane) {
    constexpr int EPL = D / 64;
    uint16_t* nt16 = reinterpret_cast<uint16_t*>(nt);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int d = lane * EPL + e;
      nt16[d] = r.k[e];
      nt16[D + d] = r.v[e];
    }
    return true;
  }
  static __device__ __forceinline__ bool prepare_new(const DecodeArgs& a, int b, int g,
                                                     uint8_t* nt, int lane) {
    return quant_new(a, load_new_rows<D>(a, b, g, lane), nt, lane);
  }

  // Fused append, second half (after the page loop): store the token from nt
  // at position pos of head h.
  static __device__ __forceinline__ void store_new(const DecodeArgs& a, const uint8_t* nt,
                                                   int pos, HeadRef h, int lane) {
    uint16_t* head = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(h.code));
    const uint16_t* nt16 = reinterpret_cast<const uint16_t*>(nt);
    for (int d = lane; d < D; d += 64) {
      head[pos * D + d] = nt16[d];
      head[16 * D + (pos >> 2) * 4 * D + 4 * d + (pos & 3)] = nt16[D + d];
    }
  }

  // Put the appended token (from nt) into the registers of its page.
  static __device__ __forceinline__ void patch(Page& pg, const uint8_t* nt, int pos, int i16,
                                               int kb) {
    const uint16_t* nt16 = reinterpret_cast<const uint16_t*>(nt);
    if (i16 == pos) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j)
        pg.k[j] = *reinterpret_cast<const u4_t*>(nt16 + 32 * j + 8 * kb);
    }
    if (kb == (pos >> 2)) {
      const int tt = pos & 3;
      const int hs = 16 * (tt & 1);
      const uint32_t keep = ~(0xFFFFu << hs);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        // V values of dims 32*i + 2*i16 and + 1: word (tt >> 1) and 2 + (tt >> 1)
        const uint32_t w = *reinterpret_cast<const uint32_t*>(nt16 + D + 32 * i + 2 * i16);
        const int w0 = tt >> 1;
        pg.v[i][w0] = (pg.v[i][w0] & keep) | ((w & 0xFFFFu) << hs);
        pg.v[i][2 + w0] = (pg.v[i][2 + w0] & keep) | ((w >> 16) << hs);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Decode loop
// ---------------------------------------------------------------------------

// Per-wave LDS staging of one pass: the q rows of each segment's unit
// ([C][D] 16-bit values, C = a.slot_cols columns) and each segment's result
// ([C][D + 2] floats: accumulator, running max, sum), a.seg_cap segments
// (offsets set on the host). One-token kernels keep the two in separate
// regions. The several-token kernels put the q slots at the top of the area
// and the result slots at its bottom: segment s's result, stashed when
// segment s + 1 starts and before s + 1's q rows are read, may cover the q
// slots up to s but never a later one, and the last segment's result is
// stashed in slot 0 once the others are written out (so a pass holds two
// 16-column segments where separate regions held one).
struct PassLds {
  uint16_t* q;   // [seg_cap][C][D]
  float* res;    // [C][D + 2] per slot
  uint8_t* nt;   // [seg_cap][kNewTokenBytes(D)]: appended token per segment
};

// The MFMA columns of unit vg of a sequence: KV head g, whose columns
// 0..n-1 are the (query token, head) pairs col0 + c with
// col = token * group + (head - g * group). One query token: all of KV
// head vg's query heads. Several: KV head vg / units_per_head, the
// unit_tiles tiles of 16 columns from tile (vg % units_per_head) * unit_tiles.
struct UnitCols {
  int g, col0, n;
};
template <bool Multi>
__device__ __forceinline__ UnitCols unit_cols(const DecodeArgs& a, int vg) {
  if constexpr (!Multi) {
    return {vg, 0, a.group};
  } else {
    const int w = 16 * a.unit_tiles;
    const int col0 = w * (vg % a.units_per_head);
    return {vg / a.units_per_head, col0, min(w, a.cols - col0)};
  }
}

// LDS bytes that hold one segment's appended token (16-bit K and V rows, or
// INT8 codes and scales); a multiple of 16.
__host__ __device__ constexpr int new_token_bytes(int D) { return 4 * D; }

// Copy the q rows of unit (b, vg) into LDS; 16-byte chunks dealt to the lanes.
template <int D, bool Multi>
__device__ __forceinline__ void stage_q(const DecodeArgs& a, int b, int vg, uint16_t* dst,
                                        int lane) {
  const UnitCols uc = unit_cols<Multi>(a, vg);
  const int chunks = uc.n * D / 8;
  for (int c = lane; c < chunks; c += 64) {
    const int cc = c / (D / 8), d0 = (c % (D / 8)) * 8;
    const int col = uc.col0 + cc;
    *reinterpret_cast<u4_t*>(dst + cc * D + d0) =
        q_chunk8(a, b, col / a.group, uc.g * a.group + col % a.group, d0);
  }
}

// Leave a segment's softmax state in LDS: [n][D + 2] for its n columns.
template <class K>
__device__ __forceinline__ void stash_result(const DecodeArgs& a, SoftmaxState<K::D / 16>& st,
                                             float* res, int i16, int kb, int n) {
  constexpr int D = K::D, ND = D / 16;
  if constexpr (K::kPair) fold_pair(st);
  const float l = col_sum(st.l);
  if (i16 >= n) return;
  float* r = res + i16 * (D + 2);
#pragma unroll
  for (int k = 0; k < ND; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) r[K::acc_dim(k, j, kb)] = st.acc[k][j];
  if (kb == 0) {
    r[D] = st.m;
    r[D + 1] = l;
  }
}

// Write a stashed result of unit (b, vg): the output rows when the segment
// covers its whole unit (zero rows when no token was attendable), else the
// partial of `slot`.
template <int D, bool Multi>
__device__ __forceinline__ void write_result(const DecodeArgs& a, const float* res, int b,
                                             int vg, int slot, bool whole, int lane) {
  const UnitCols uc = unit_cols<Multi>(a, vg);
  if (whole) {
    for (int e = lane; e < uc.n * D; e += 64) {
      const int cc = e / D, d = e % D;
      const int col = uc.col0 + cc;
      const float l = res[cc * (D + 2) + D + 1];
      const float v = l > 0.f ? res[cc * (D + 2) + d] / l * a.out_mul : 0.f;
      store_out(a.out, a.out_dtype,
                b * a.out_ss + (col / a.group) * a.out_st +
                    (uc.g * a.group + col % a.group) * a.out_sh + d,
                v);
    }
  } else {
    float* dst = a.ws + static_cast<int64_t>(slot) * a.slot_cols * (D + 2);
    for (int e = lane; e < uc.n * (D + 2); e += 64) dst[e] = res[e];
  }
}

// Walks the units of a wave's item range: (b, g, p) is the current position,
// np and L the current sequence's page count and length; lens holds the
// context lengths of sequences 64*c .. 64*c+63 (one per lane), hit the lane of b.
struct Cursor {
  int b, g, p, np, L, c, lens, hit;
};

// Move to the first page of the next unit with pages; false if the lengths
// changed under the call (no such unit).
__device__ __forceinline__ bool next_unit(const DecodeArgs& a, Cursor& cu, int nchunk, int vh,
                                          int lane) {
  cu.p = 0;
  if (++cu.g < vh) return true;
  cu.g = 0;
  while (true) {
    const uint64_t m = __ballot(cu.lens > 0 && lane > cu.hit);
    if (m) {
      cu.hit = __builtin_ctzll(m);
      break;
    }
    if (cu.c + 1 >= nchunk) return false;
    cu.lens = load_chunk(a, ++cu.c, 0, false, lane).L;
    cu.hit = -1;
  }
  cu.b = 64 * cu.c + cu.hit;
  cu.L = readlane(cu.lens, cu.hit);
  cu.np = (cu.L + kBlockSize - 1) / kBlockSize;
  return true;
}

// One pass over up to a.seg_cap segments (and up to 128 items) of the wave's
// range starting at item x: plan the segments, stage every segment's q rows in
// LDS and every item's block id in registers, stream all the pass's pages
// through one pipeline (segment switches inside it touch only registers and
// LDS, so the page loads in flight are never waited for early), then write
// the stashed results. Returns the number of items done (0: lengths changed).
template <class K, bool Multi>
__device__ __forceinline__ int run_pass(const DecodeArgs& a, K& kind, Cursor& cu, int x, int x1,
                                        int P, int wave, int nchunk, const PassLds& lds,
                                        int lane) {
  constexpr int D = K::D, ND = D / 16;
  const int i16 = lane & 15, kb = lane >> 4;
  const int hkv = a.num_kv_heads;
  const int vh = Multi ? a.vheads : hkv;  // units per sequence
  const int C = a.slot_cols;              // LDS columns per segment

  // plan: lane s keeps segment s's unit, first page, first item, length, L
  // (a pair kind pads each segment to whole pairs: `items` counts the
  // pass's page slots, holes included, `real` the wave's items done)
  constexpr bool kPair = K::kPair;
  int s_unit = 0, s_p = 0, s_start = 0, s_n = 0, s_L = 0, s_whole = 0, s_last = 0;
  int ns = 0, items = 0, real = 0;
  while (true) {
    // a segment is never cut by the end of a pass: its unit would come back
    // in the next pass of this wave, whose partial takes the same slot. One
    // that does not fit whole starts the next pass (the first one always
    // fits: at most P <= kMaxPagesPerWave pages, padded to an even count)
    const int want = min(cu.np - cu.p, x1 - (x + real));
    if (ns > 0 && items + (kPair ? want + (want & 1) : want) > kMaxPagesPerWave) break;
    const int n = min(want, kMaxPagesPerWave - items);
    const int u = cu.b * vh + cu.g;
    if (cu.p == 0 && lane == 0) {
      // this wave holds the unit's first item: record which waves cover it
      a.desc[u] = make_int2(wave, (x + real + cu.np - 1) / P - wave + 1);
    }
    if (lane == ns) {
      s_unit = u;
      s_p = cu.p;
      s_start = items;
      s_n = n;
      s_L = cu.L;
      s_whole = cu.p == 0 && n == cu.np;
      s_last = cu.p + n == cu.np;  // holds the unit's last page
    }
    ++ns;
    items += kPair ? n + (n & 1) : n;  // (items stays even for pairs: 128 - items > n)
    real += n;
    cu.p += n;
    if (cu.p == cu.np && x + real < x1 && !next_unit(a, cu, nchunk, vh, lane)) return 0;
    if (x + real >= x1 || ns == a.seg_cap || items >= kMaxPagesPerWave) break;
  }

  // pages of the items: lane i holds the block ids and KV heads of items i
  // and 64 + i; out-of-range block ids are flagged and become -1 (the page
  // is masked)
  // (slots that hold no item, the holes of pair padding, stay -1)
  int blk0 = -1, blk1 = -1, g0 = 0, g1 = 0;
  bool own0 = false, own1 = false;
  for (int s = 0; s < ns; ++s) {
    const int st = readlane(s_start, s), n = readlane(s_n, s);
    const int u = readlane(s_unit, s);
    const int32_t* row = a.bt + static_cast<int64_t>(u / vh) * a.bt_stride + readlane(s_p, s);
    const int g = unit_cols<Multi>(a, u % vh).g;
    if (lane >= st && lane < st + n) {
      blk0 = row[lane - st];
      g0 = g;
      own0 = true;
    }
    if (lane + 64 >= st && lane + 64 < st + n) {
      blk1 = row[lane + 64 - st];
      g1 = g;
      own1 = true;
    }
  }
  // the q rows go to LDS while the block ids are in flight
  for (int s = 0; s < ns; ++s) {
    const int u = readlane(s_unit, s);
    stage_q<D, Multi>(a, u / vh, u % vh, lds.q + s * C * D, lane);
  }
  if (own0 && (blk0 < 0 || blk0 >= a.num_blocks)) {
    raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    blk0 = -1;
  }
  if (own1 && (blk1 < 0 || blk1 >= a.num_blocks)) {
    raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    blk1 = -1;
  }
  auto block_of = [&](int i) { return i < 64 ? readlane(blk0, i) : readlane(blk1, i - 64); };
  auto head_of = [&](int i) { return i < 64 ? readlane(g0, i) : readlane(g1, i - 64); };
  // (a missing page is fully masked and loaded through an empty resource:
  // no memory access)

  // current segment: first page's token, first item, end item, length,
  // whether its last page gets the appended token, its column count and (for
  // several query tokens) the smallest and the lane's own attention limit
  int s_patch = 0;  // lane s: segment s's appended token is in LDS
  int cs = 0, c_tok = 0, c_start = 0, c_end = 0, c_endp = 0, c_L = 0, c_patch = 0;
  int c_n = a.group, c_Lmin = 0, c_Lc = 0;
  auto enter = [&](int sidx) {
    cs = sidx;
    c_tok = readlane(s_p, sidx) * kBlockSize;
    c_start = readlane(s_start, sidx);
    c_end = c_start + readlane(s_n, sidx);
    c_endp = kPair ? c_end + ((c_end - c_start) & 1) : c_end;  // with the hole
    c_L = readlane(s_L, sidx);
    c_patch = readlane(s_patch, sidx);
    if constexpr (Multi) {
      // query token j sits at position L - qtok + j and sees positions up to it
      const UnitCols uc = unit_cols<true>(a, readlane(s_unit, sidx) % vh);
      c_n = uc.n;
      c_Lmin = c_L - a.qtok + 1;
      c_Lc = min(c_Lmin + (uc.col0 + i16) / a.group, c_L);
    }
  };
  SoftmaxState<ND> st;

  // Two register buffers of G pages each, each refilled right after its pages
  // are consumed. Every refill issues the same load instructions (so the
  // compiler's waits count exactly the loads of the pages being consumed):
  // past the pass's last item, and for a missing page, the loads go through
  // an empty buffer resource, which returns zeros without a memory access.
  constexpr int G = K::kGroup;
  typename K::Page ga[G], gb[G];
  int ba[G], bb[G];
  auto fill = [&](typename K::Page* grp, int* blk, int first) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int q = first + j;
      blk[j] = q < items ? block_of(q) : -1;
      K::load(grp[j], head_ref<K>(a, blk[j], q < items ? head_of(q) : 0), blk[j] >= 0, i16, kb);
    }
  };
  // consume items first.. of a group; false once the pass's items are done
  auto consume = [&](typename K::Page* grp, const int* blk, int first) {
    if constexpr (kPair) {
      // the group is one pair of one segment
      const int i = first;
      if (i >= items) return false;
      if (i == c_endp) {  // next segment: only registers and LDS are touched
        stash_result<K>(a, st, lds.res + cs * C * (D + 2), i16, kb, c_n);
        enter(cs + 1);
        softmax_init(st);
        const int h = K::col_head(i16);
        kind.load_q(a, lds.q + cs * C * D, h, kb, h < c_n);
      }
      const int t = c_tok + (i - c_start) * kBlockSize;
      if (c_patch) {
        const int pos = (c_L - 1) % kBlockSize;
        const uint8_t* nt = lds.nt + cs * new_token_bytes(D);
        if (i == c_end - 1) K::patch(grp[0], nt, pos, i16, kb);
        if (i + 1 == c_end - 1) K::patch(grp[1], nt, pos, i16, kb);
      }
      kind.step_pair(grp[0], grp[1], t, blk[0] >= 0 ? c_L : t,
                     blk[1] >= 0 ? c_L : t + kBlockSize, st);
      return true;
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = first + j;
      if (i >= items) return false;
      if (i == c_end) {  // next segment: only registers and LDS are touched
        stash_result<K>(a, st, lds.res + cs * C * (D + 2), i16, kb, c_n);
        enter(cs + 1);
        softmax_init(st);
        kind.load_q(a, lds.q + cs * C * D, i16, kb, i16 < c_n);
      }
      const int t = c_tok + (i - c_start) * kBlockSize;
      if (!Multi && c_patch && i == c_end - 1)
        K::patch(grp[j], lds.nt + cs * new_token_bytes(D), (c_L - 1) % kBlockSize, i16, kb);
      // a missing page (blk < 0) is masked whole
      if constexpr (Multi) {
        const bool ok = blk[j] >= 0;
        kind.step(grp[j], t, ok ? c_L : t, ok ? c_Lmin : t, ok ? c_Lc : t, st);
      } else {
        const int Lv = blk[j] >= 0 ? c_L : t;
        kind.step(grp[j], t, Lv, Lv, Lv, st);
      }
    }
    return true;
  };
  fill(ga, ba, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep the groups' loads in order
  fill(gb, bb, G);
  __builtin_amdgcn_sched_barrier(0);
  // fused append (after the first pages are in flight): the wave holding a
  // unit's last page quantizes the sequence's newest token for that KV head,
  // patches it into the page as loaded and stores it into the page (nobody
  // else reads that slot during the call)
  // (its stores wait until after the page loop, so that the loop's waits
  // count page loads only). The first such unit's new rows are requested
  // before q is read from LDS and quantized after, so that their round trip
  // overlaps q's preparation instead of delaying it (one-token calls: c_n is
  // the group, whatever the segment).
  NewRows<D> first_rows{};
  int first_end = -1;
  if (!Multi && a.append) {
    const uint64_t ends = __ballot(lane < ns && s_last != 0);
    if (ends) {
      first_end = __builtin_ctzll(ends);
      const int u = readlane(s_unit, first_end);
      first_rows = load_new_rows<D>(a, u / hkv, u % hkv, lane);
    }
    // (a compiler barrier: keeps these loads here rather than next to their
    // use; it waits for nothing)
    asm volatile("" ::: "memory");
  }
  if constexpr (!Multi) kind.load_q(a, lds.q, K::col_head(i16), kb, K::col_head(i16) < c_n);
  if (!Multi && a.append) {
    for (int s = 0; s < ns; ++s) {
      if (!readlane(s_last, s)) continue;
      const int u = readlane(s_unit, s);
      uint8_t* nt = lds.nt + s * new_token_bytes(D);
      const bool ok = s == first_end ? K::quant_new(a, first_rows, nt, lane)
                                     : K::prepare_new(a, u / hkv, u % hkv, nt, lane);
      if (lane == s) s_patch = ok;
    }
  }
  enter(0);
  softmax_init(st);
  if constexpr (Multi) kind.load_q(a, lds.q, K::col_head(i16), kb, K::col_head(i16) < c_n);
  for (int i = 0;; i += 2 * G) {
    if (!consume(ga, ba, i)) break;
    __builtin_amdgcn_sched_barrier(0);
    fill(ga, ba, i + 2 * G);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = consume(gb, bb, i + G);
    __builtin_amdgcn_sched_barrier(0);
    fill(gb, bb, i + 3 * G);
    __builtin_amdgcn_sched_barrier(0);
    if (!more || i + 2 * G >= items) break;
  }
  if constexpr (!Multi) stash_result<K>(a, st, lds.res + cs * C * (D + 2), i16, kb, c_n);

  if (!Multi && a.append) {
    for (int s = 0; s < ns; ++s) {
      const int it = readlane(s_start, s) + readlane(s_n, s) - 1;  // its last page
      const int blk = block_of(it);
      if (!readlane(s_patch, s) || blk < 0) continue;
      K::store_new(a, lds.nt + s * new_token_bytes(D), (readlane(s_L, s) - 1) % kBlockSize,
                   head_ref<K>(a, blk, head_of(it)), lane);
    }
  }
  if constexpr (Multi) {
    // the earlier segments' results from their slots, then the last one's
    // (still in registers) through slot 0
    for (int s = 0; s <= ns - 1; ++s) {
      if (s == ns - 1) stash_result<K>(a, st, lds.res, i16, kb, c_n);
      const int u = readlane(s_unit, s);
      write_result<D, Multi>(a, lds.res + (s == ns - 1 ? 0 : s) * C * (D + 2), u / vh, u % vh,
                             wave + u, readlane(s_whole, s) != 0, lane);
    }
  } else {
    for (int s = 0; s < ns; ++s) {
      const int u = readlane(s_unit, s);
      write_result<D, Multi>(a, lds.res + s * C * (D + 2), u / vh, u % vh, wave + u,
                             readlane(s_whole, s) != 0, lane);
    }
  }
  return real;
}

// Write tile i's softmax state straight from registers (after the page
// loop): the output rows of its columns when the segment covers the whole
// unit (zero rows when no token was attendable), else the columns of the
// unit's partial in `slot` (accumulator, running max, sum).
template <class K>
__device__ __forceinline__ void write_tile(const DecodeArgs& a, SoftmaxState<K::D / 16>& st,
                                           int b, const UnitCols& uc, int tile, int slot,
                                           bool whole, int i16, int kb) {
  constexpr int D = K::D, ND = D / 16;
  const float l = col_sum(st.l);
  const int cc = 16 * tile + i16;  // column inside the unit
  if (cc >= uc.n) return;
  if (whole) {
    const int col = uc.col0 + cc;
    const int64_t o = b * a.out_ss + (col / a.group) * a.out_st +
                      (uc.g * a.group + col % a.group) * a.out_sh;
    const float f = l > 0.f ? a.out_mul / l : 0.f;
#pragma unroll
    for (int k = 0; k < ND; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) store_out(a.out, a.out_dtype, o + K::acc_dim(k, j, kb),
                                            st.acc[k][j] * f);
  } else {
    float* r = a.ws + (static_cast<int64_t>(slot) * a.slot_cols + cc) * (D + 2);
#pragma unroll
    for (int k = 0; k < ND; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) r[K::acc_dim(k, j, kb)] = st.acc[k][j];
    if (kb == 0) {
      r[D] = st.m;
      r[D + 1] = l;
    }
  }
}

// A pass of the several-token kernels with NT tiles per unit: the rest of
// the current unit inside the wave's range (up to kMaxPagesPerWave items),
// every page converted once and used by all NT query tiles, whose softmax
// states stay in registers and are written after the page loop. Returns the
// number of items done (0: the lengths changed under the call).
template <class K, int NT>
__device__ __forceinline__ int run_pass_wide(const DecodeArgs& a, K* kind, Cursor& cu, int x,
                                             int x1, int P, int wave, int nchunk,
                                             uint16_t* q_lds, int lane) {
  constexpr int D = K::D, ND = D / 16;
  const int i16 = lane & 15, kb = lane >> 4;
  const int vh = a.vheads;
  const int items = min(min(cu.np - cu.p, x1 - x), kMaxPagesPerWave);
  const int u = cu.b * vh + cu.g;
  if (cu.p == 0 && lane == 0) a.desc[u] = make_int2(wave, (x + cu.np - 1) / P - wave + 1);
  const int b = cu.b, vg = cu.g, p0 = cu.p, L = cu.L;
  const bool whole = cu.p == 0 && items == cu.np;
  const UnitCols uc = unit_cols<true>(a, vg);
  // block ids of the pass (lane i: items i and 64 + i), flagged and masked
  // when out of range; then the q rows of every tile go to LDS
  const int32_t* row = a.bt + static_cast<int64_t>(b) * a.bt_stride + p0;
  int blk0 = lane < items ? row[lane] : 0;
  int blk1 = lane + 64 < items ? row[lane + 64] : 0;
  stage_q<D, true>(a, b, vg, q_lds, lane);
  if (blk0 < 0 || blk0 >= a.num_blocks) {
    raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    blk0 = -1;
  }
  if (blk1 < 0 || blk1 >= a.num_blocks) {
    raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    blk1 = -1;
  }
  auto block_of = [&](int i) { return i < 64 ? readlane(blk0, i) : readlane(blk1, i - 64); };
  cu.p += items;
  if (cu.p == cu.np && x + items < x1 && !next_unit(a, cu, nchunk, vh, lane)) return 0;

  // query token j of the sequence sits at position L - qtok + j and sees the
  // positions up to it; Lmin: the first query token's limit
  const int Lmin = L - a.qtok + 1;
  const int nt = (uc.n + 15) / 16;  // tiles of the unit (wave-uniform)
  int Lc[NT];
  SoftmaxState<ND> st[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    Lc[i] = min(Lmin + (uc.col0 + 16 * i + i16) / a.group, L);
    softmax_init(st[i]);
    if (16 * i < uc.n) kind[i].load_q(a, q_lds + 16 * i * D, i16, kb, 16 * i + i16 < uc.n);
  }

  constexpr int G = K::kGroup;
  typename K::Page ga[G], gb[G];
  int ba[G], bb[G];
  auto fill = [&](typename K::Page* grp, int* blk, int first) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int q = first + j;
      blk[j] = q < items ? block_of(q) : -1;
      K::load(grp[j], head_ref<K>(a, blk[j], uc.g), blk[j] >= 0, i16, kb);
    }
  };
  auto consume = [&](typename K::Page* grp, const int* blk, int first) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int i = first + j;
      if (i >= items) return false;
      const int t = (p0 + i) * kBlockSize;
      const bool ok = blk[j] >= 0;  // a missing page is masked whole
      int lim[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) lim[c] = ok ? Lc[c] : t;
      K::template step_tiles<NT>(grp[j], kind, nt, t, ok ? L : t, ok ? Lmin : t, lim, st);
    }
    return true;
  };
  fill(ga, ba, 0);
  __builtin_amdgcn_sched_barrier(0);
  fill(gb, bb, G);
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0;; i += 2 * G) {
    if (!consume(ga, ba, i)) break;
    __builtin_amdgcn_sched_barrier(0);
    fill(ga, ba, i + 2 * G);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = consume(gb, bb, i + G);
    __builtin_amdgcn_sched_barrier(0);
    fill(gb, bb, i + 3 * G);
    __builtin_amdgcn_sched_barrier(0);
    if (!more || i + 2 * G >= items) break;
  }
#pragma unroll
  for (int c = 0; c < NT; ++c)
    if (16 * c < uc.n) write_tile<K>(a, st[c], b, uc, c, wave + u, whole, i16, kb);
  return items;
}

template <class K, bool Multi, int NT = 1>
__device__ __forceinline__ void decode_wave(const DecodeArgs& a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kWaves + wid;
  const int vh = Multi ? a.vheads : a.num_kv_heads;  // units per sequence
  PassLds lds;
  lds.q = reinterpret_cast<uint16_t*>(smem + wid * a.lds_wave_bytes + a.lds_q_off);
  lds.res = reinterpret_cast<float*>(smem + wid * a.lds_wave_bytes + a.lds_res_off);
  lds.nt = smem + wid * a.lds_wave_bytes + a.lds_nt_off;

  // total pages; zero rows of empty sequences
  const int nchunk = (a.num_seqs + 63) / 64;
  SeqChunk s = load_chunk(a, 0, 0, wave == 0, lane);
  zero_rows(a, s, wave, K::D, lane);
  int pages = chunk_end(s);
  for (int c = 1; c < nchunk; ++c) {
    const SeqChunk t = load_chunk(a, c, pages, wave == 0, lane);
    zero_rows(a, t, wave, K::D, lane);
    pages = chunk_end(t);
  }
  const int total = pages * vh;
  const int P = pages_per_wave(total, a.num_waves);
  const int x0 = wave * P;
  if (x0 >= total) return;
  const int x1 = min(x0 + P, total);

  // the sequence holding item x0: items of sequence b are
  // [vh * excl_b, vh * (excl_b + np_b))
  int hit;
  while (true) {
    const int lo = vh * s.excl;
    const uint64_t m = __ballot(s.np > 0 && lo <= x0 && x0 < lo + vh * s.np);
    if (m) {
      hit = __builtin_ctzll(m);
      break;
    }
    if (s.c + 1 >= nchunk) return;  // only if the lengths changed under the call
    s = load_chunk(a, s.c + 1, chunk_end(s), false, lane);
  }
  Cursor cu;
  cu.c = s.c;
  cu.lens = s.L;
  cu.hit = hit;
  cu.b = 64 * s.c + hit;
  cu.L = readlane(s.L, hit);
  cu.np = (cu.L + kBlockSize - 1) / kBlockSize;
  const int off = x0 - vh * readlane(s.excl, hit);
  cu.g = off / cu.np;
  cu.p = off - cu.g * cu.np;

  if constexpr (NT == 1) {
    K kind;
    for (int x = x0; x < x1;) {
      const int done = run_pass<K, Multi>(a, kind, cu, x, x1, P, wave, nchunk, lds, lane);
      if (done == 0) return;
      x += done;
    }
  } else {
    K kind[NT];
    for (int x = x0; x < x1;) {
      const int done = run_pass_wide<K, NT>(a, kind, cu, x, x1, P, wave, nchunk, lds.q, lane);
      if (done == 0) return;
      x += done;
    }
  }
}

// ---------------------------------------------------------------------------
// Calls with few units: one workgroup per (sequence, KV head)
// ---------------------------------------------------------------------------
// With few units (a short batch: latency-bound), the even split over a whole
// grid pays a context-length scan, partials in HBM and a second launch for
// their merge, all in series with a small amount of streaming. Here workgroup
// u takes unit u = (b, g) alone: its kUnitWaves waves split the unit's pages
// evenly, each streams its share through the page pipeline of the large-call
// kernels, leaves its softmax state (acc, max, sum per column) in LDS, and
// after a barrier the workgroup merges the waves' states and writes the
// output rows: one launch, no HBM round trip between the waves and the merge.
// (It pays while each wave has a few pages: a wave streams its share alone.)
template <class K>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a) {
  constexpr int D = K::D;
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i16 = lane & 15, kb = lane >> 4;
  const int G = a.group;
  const int b = blockIdx.x / a.num_kv_heads, g = blockIdx.x % a.num_kv_heads;
  // LDS: every wave's q rows [G][D] (16-bit), then every wave's state
  // [G][D + 2], then every wave's appended token (new_token_bytes(D))
  uint16_t* q_lds = reinterpret_cast<uint16_t*>(smem) + w * G * D;
  float* res_all = reinterpret_cast<float*>(smem + kUnitWaves * G * D * 2);
  float* res = res_all + w * G * (D + 2);
  uint8_t* nt = smem + kUnitWaves * G * (D * 2 + (D + 2) * 4) + w * new_token_bytes(D);

  int L = a.ctx[b];
  if (L < 0 || L > a.max_ctx) {
    if (g == 0 && w == 0 && lane == 0) raise_flag(a.err, PDAKV_EFLAG_CONTEXT_RANGE);
    L = L < 0 ? 0 : a.max_ctx;
  }
  const int np = (L + kBlockSize - 1) / kBlockSize;
  const int per = (np + kUnitWaves - 1) / kUnitWaves;  // at most 128 (host-checked)
  const int p0 = min(w * per, np);
  const int items = min(per, np - p0);

  // the wave's block ids (lane i: items i and 64 + i), flagged and masked
  // when out of range; the q rows go to LDS meanwhile
  const int32_t* row = a.bt + static_cast<int64_t>(b) * a.bt_stride + p0;
  int blk0 = lane < items ? row[lane] : 0;
  int blk1 = lane + 64 < items ? row[lane + 64] : 0;
  stage_q<D, false>(a, b, g, q_lds, lane);
  if (blk0 < 0 || blk0 >= a.num_blocks) {
    raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    blk0 = -1;
  }
  if (blk1 < 0 || blk1 >= a.num_blocks) {
    raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    blk1 = -1;
  }
  auto block_of = [&](int i) { return i < 64 ? readlane(blk0, i) : readlane(blk1, i - 64); };

  K kind;
  SoftmaxState<D / 16> st;
  softmax_init(st);
  constexpr int GP = K::kGroup;
  typename K::Page ga[GP], gb[GP];
  int ba[GP], bb[GP];
  auto fill = [&](typename K::Page* grp, int* blk, int first) {
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      const int q = first + j;
      blk[j] = q < items ? block_of(q) : -1;
      K::load(grp[j], head_ref<K>(a, blk[j], g), blk[j] >= 0, i16, kb);
    }
  };
  // fused append: the wave holding the unit's last page quantizes the
  // sequence's newest token for KV head g, patches it into that page as
  // loaded and stores it after the loop (nobody else reads that slot)
  const bool owner = a.append && items > 0 && p0 + items == np;
  bool patched = false;
  const int pos = (L - 1) % kBlockSize;
  auto consume = [&](typename K::Page* grp, const int* blk, int first) {
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      const int i = first + j;
      if (i >= items) return false;
      const int t = (p0 + i) * kBlockSize;
      if (patched && i == items - 1) K::patch(grp[j], nt, pos, i16, kb);
      const int Lv = blk[j] >= 0 ? L : t;  // a missing page is masked whole
      kind.step(grp[j], t, Lv, Lv, Lv, st);
    }
    return true;
  };
  fill(ga, ba, 0);
  __builtin_amdgcn_sched_barrier(0);
  fill(gb, bb, GP);
  __builtin_amdgcn_sched_barrier(0);
  // (after the first pages are in flight; its stores wait until after the
  // page loop, so that the loop's waits count page loads only)
  if (owner) patched = K::prepare_new(a, b, g, nt, lane);
  kind.load_q(a, q_lds, i16, kb, i16 < G);
  for (int i = 0;; i += 2 * GP) {
    if (!consume(ga, ba, i)) break;
    __builtin_amdgcn_sched_barrier(0);
    fill(ga, ba, i + 2 * GP);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = consume(gb, bb, i + GP);
    __builtin_amdgcn_sched_barrier(0);
    fill(gb, bb, i + 3 * GP);
    __builtin_amdgcn_sched_barrier(0);
    if (!more || i + 2 * GP >= items) break;
  }
  stash_result<K>(a, st, res, i16, kb, G);
  if (patched) {
    const int blk = block_of(items - 1);
    if (blk >= 0) K::store_new(a, nt, pos, head_ref<K>(a, blk, g), lane);
  }
  __syncthreads();

  // out[c][d] = sum_w 2^(m_w - m) acc_w[c][d] / sum_w 2^(m_w - m) l_w (m = max_w m_w;
  // a wave without pages has m_w = kMaxInit and adds nothing; no token at
  // all gives a zero row)
  for (int e = threadIdx.x; e < G * D; e += 64 * kUnitWaves) {
    const int c = e / D, d = e % D;
    float m = kMaxInit;
#pragma unroll
    for (int v = 0; v < kUnitWaves; ++v) m = fmaxf(m, res_all[(v * G + c) * (D + 2) + D]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int v = 0; v < kUnitWaves; ++v) {
      const float* r = res_all + (v * G + c) * (D + 2);
      const float f = __builtin_amdgcn_exp2f(r[D] - m);
      num += f * r[d];
      den += f * r[D + 1];
    }
    store_out(a.out, a.out_dtype, b * a.out_ss + (g * G + c) * a.out_sh + d,
              den > 0.f ? num / den * a.out_mul : 0.f);
  }
}

// The register budget per wave (waves per SIMD) sets how many pages a
// buffer group holds; the host plans one resident round of waves for it.
// Pair: groups of at most 8 heads take two pages per softmax update
template <int D, bool QBF16, bool Pair>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    kInt8WavesPerSimd))) void decode_int8_kernel(DecodeArgs a) {
  decode_wave<Int8Kind<D, QBF16, kInt8PageGroup, false, Pair>, false>(a);
}

template <int D, bool QBF16>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    kInt8WavesPerSimd))) void decode_int8_multi_kernel(DecodeArgs a) {
  decode_wave<Int8Kind<D, QBF16, kInt8PageGroup>, true>(a);
}

// Several query tiles per unit, one page per register buffer; the waves per
// SIMD that the registers of NT tiles' softmax states and q fragments allow
// (wide_waves_per_simd, which the host plans with)
template <int D, bool QBF16, int NT>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    wide_waves_per_simd(PDAKV_KV_INT8_SYM, NT)))) void decode_int8_wide_kernel(DecodeArgs a) {
  decode_wave<Int8Kind<D, QBF16, 1>, true, NT>(a);
}

template <int D, bool BF16, int NT>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    wide_waves_per_simd(PDAKV_KV_16BIT, NT)))) void decode_16bit_wide_kernel(DecodeArgs a) {
  decode_wave<F16Kind<D, BF16, 1>, true, NT>(a);
}

template <int D, bool QBF16, bool Pair>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    kInt8WavesPerSimd))) void decode_int8_static_kernel(DecodeArgs a) {
  decode_wave<Int8Kind<D, QBF16, kInt8PageGroup, true, Pair>, false>(a);
}

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    k16WavesPerSimd))) void decode_16bit_kernel(DecodeArgs a) {
  decode_wave<F16Kind<D, BF16, k16PageGroup>, false>(a);
}

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(
    k16WavesPerSimd))) void decode_16bit_multi_kernel(DecodeArgs a) {
  decode_wave<F16Kind<D, BF16, k16PageGroup>, true>(a);
}

// One workgroup per unit (small calls), at the occupancy of the large-call
// kernels of the same format (two waves per SIMD).
template <int D, bool QBF16>
__global__ __launch_bounds__(64 * kUnitWaves) __attribute__((amdgpu_waves_per_eu(
    kInt8WavesPerSimd))) void decode_int8_unit_kernel(DecodeArgs a) {
  decode_unit<Int8Kind<D, QBF16, kInt8PageGroup>>(a);
}
template <int D, bool QBF16>
__global__ __launch_bounds__(64 * kUnitWaves) __attribute__((amdgpu_waves_per_eu(
    kInt8WavesPerSimd))) void decode_int8_static_unit_kernel(DecodeArgs a) {
  decode_unit<Int8Kind<D, QBF16, kInt8PageGroup, true>>(a);
}
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kUnitWaves) __attribute__((amdgpu_waves_per_eu(
    k16WavesPerSimd))) void decode_16bit_unit_kernel(DecodeArgs a) {
  decode_unit<F16Kind<D, BF16, k16PageGroup>>(a);
}

// Combine the partials of a unit that spans several waves, per (query token,
// query head) column: out = sum_i 2^(m_i - m) acc_i / sum_i 2^(m_i - m) l_i
// over the waves i that cover the unit (m = max_i m_i), as recorded by the
// unit's first wave. One workgroup per MC columns of a unit (64 / MC lanes
// per column, lane l of a column holding dims l, l + 64 / MC, ...) with
// a.merge_waves waves: wave w folds the partials w, w + waves, ... into a
// running (max, sum, accumulator), kMergeBatch partials per round trip; the
// waves then combine through LDS. Four columns per workgroup pay off once a
// unit has 16 columns (several query tokens): a quarter of the workgroups,
// each with four times the loads in flight.
constexpr int kMergeBatch = 8;

template <int MC>
__host__ __device__ constexpr int merge_groups(int slot_cols) {
  return (slot_cols + MC - 1) / MC;
}

template <int D, int MC>
__global__ __launch_bounds__(64 * kMaxMergeWaves) void merge_kernel(DecodeArgs a) {
  constexpr int LPC = 64 / MC;   // lanes per column
  constexpr int DPL = D / LPC;   // dims per lane
  // with several waves: per wave and column the accumulator, max and sum
  // ([waves][MC][D + 2] floats, sized at launch)
  extern __shared__ float merge_lds[];
  const int lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int groups = merge_groups<MC>(a.slot_cols);
  const int per_seq = a.vheads * groups;
  const int b = blockIdx.x / per_seq, vg = blockIdx.x % per_seq / groups;
  const int grp = blockIdx.x % groups;
  const int u = b * a.vheads + vg;
  // the unit's record is this call's only if the sequence has pages (its
  // first wave wrote it)
  const int2 rec = a.desc[u];
  const int L = a.ctx[b];
  if (L <= 0 || rec.y <= 1) return;  // no pages, or written directly
  const UnitCols uc = unit_cols<true>(a, vg);
  const int ci = lane / LPC, li = lane % LPC;
  const int cc = grp * MC + ci;  // column inside the unit
  const bool valid = cc < uc.n;
  const int n = rec.y;
  const int64_t stride = static_cast<int64_t>(a.slot_cols) * (D + 2);
  const float* base = a.ws + (static_cast<int64_t>(rec.x) + u) * stride +
                      (valid ? cc : 0) * (D + 2) + li;

  float mw = kMaxInit, lw = 0.f, acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  for (int i0 = w; i0 < n; i0 += nw * kMergeBatch) {
    float m[kMergeBatch], l[kMergeBatch], v[kMergeBatch][DPL];
#pragma unroll
    for (int r = 0; r < kMergeBatch; ++r) {
      // entries past n repeat the last partial's loads and are zeroed
      const int i = i0 + r * nw;
      const float* pi = base + (i < n ? i : n - 1) * stride;
      m[r] = i < n ? pi[D - li] : kMaxInit;
      l[r] = i < n ? pi[D + 1 - li] : 0.f;
#pragma unroll
      for (int k = 0; k < DPL; ++k) v[r][k] = i < n ? pi[LPC * k] : 0.f;
    }
    float mn = mw;
#pragma unroll
    for (int r = 0; r < kMergeBatch; ++r) mn = fmaxf(mn, m[r]);
    const float c = exp2f(mw - mn);
    lw *= c;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] *= c;
#pragma unroll
    for (int r = 0; r < kMergeBatch; ++r) {
      const float e = exp2f(m[r] - mn);
      lw += e * l[r];
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] += e * v[r][k];
    }
    mw = mn;
  }
  const int col = uc.col0 + (valid ? cc : 0);
  const int64_t o = b * a.out_ss + (col / a.group) * a.out_st +
                    (uc.g * a.group + col % a.group) * a.out_sh;
  if (nw == 1) {
    // lw == 0: no attendable token in the unit
    if (valid) {
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        store_out(a.out, a.out_dtype, o + li + LPC * k, lw > 0.f ? acc[k] / lw * a.out_mul : 0.f);
    }
    return;
  }
  auto slot = [&](int wave) { return merge_lds + (wave * MC + ci) * (D + 2); };
  float* mine = slot(w);
  if (li == 0) {
    mine[D] = mw;
    mine[D + 1] = lw;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) mine[li + LPC * k] = acc[k];
  __syncthreads();
  if (!valid || w != 0) return;
  float ms = kMaxInit;
  for (int j = 0; j < nw; ++j) ms = fmaxf(ms, slot(j)[D]);
  float den = 0.f;
  for (int j = 0; j < nw; ++j) den += exp2f(slot(j)[D] - ms) * slot(j)[D + 1];
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    float num = 0.f;
    for (int j = 0; j < nw; ++j) num += exp2f(slot(j)[D] - ms) * slot(j)[li + LPC * k];
    store_out(a.out, a.out_dtype, o + li + LPC * k, den > 0.f ? num / den * a.out_mul : 0.f);
  }
}

template <int D, int MC>
hipError_t launch_merge_cols(const DecodeArgs& a, hipStream_t s) {
  const size_t lds =
      a.merge_waves > 1 ? static_cast<size_t>(a.merge_waves) * MC * (D + 2) * 4 : 0;
  hipLaunchKernelGGL((merge_kernel<D, MC>),
                     dim3(a.num_seqs * a.vheads * merge_groups<MC>(a.slot_cols)),
                     dim3(64 * a.merge_waves), lds, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  if (a.max_ctx == 0) return hipSuccess;
  return a.slot_cols > 8 ? launch_merge_cols<D, 4>(a, s) : launch_merge_cols<D, 1>(a, s);
}

// The decode grid (one resident round of waves, planned on the host) with its
// LDS, then the merge of the units split over several waves.
using DecodeKernel = void (*)(DecodeArgs);

// A call of few units: one workgroup per unit (no merge launch).
hipError_t launch_unit(DecodeKernel k, const DecodeArgs& a, int head_dim, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kUnitWaves) *
                     (a.group * (head_dim * 2 + (head_dim + 2) * 4) + new_token_bytes(head_dim));
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(a.num_seqs) * a.num_kv_heads),
                     dim3(64 * kUnitWaves), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_pair(DecodeKernel k, const DecodeArgs& a, int head_dim, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kWaves) * a.lds_wave_bytes;
  hipLaunchKernelGGL(k, dim3(a.num_waves / kWaves), dim3(64 * kWaves), lds, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return head_dim == 128 ? launch_merge<128>(a, s) : launch_merge<64>(a, s);
}

// The one-token INT8 grid kernel for a head size, q type and scale format:
// head size 128 with a group that fits the pair tile takes two pages per
// softmax update (measured: batched step 126 -> 122 us back to back, 32K
// 112 -> 105 us); head size 64 keeps one (its smaller pages gained nothing:
// the small-head configuration measured 22.2 -> 22.5 us).
constexpr int kPairMaxGroup = 8;
template <bool Static, int D, bool B>
DecodeKernel int8_kernel(bool pair) {
  if constexpr (Static)
    return pair ? decode_int8_static_kernel<D, B, true> : decode_int8_static_kernel<D, B, false>;
  else
    return pair ? decode_int8_kernel<D, B, true> : decode_int8_kernel<D, B, false>;
}
template <bool Static>
DecodeKernel pick_int8(int head_dim, int group, bool q_bf16) {
  const bool pair = group <= kPairMaxGroup;
  if (head_dim == 128)
    return q_bf16 ? int8_kernel<Static, 128, true>(pair) : int8_kernel<Static, 128, false>(pair);
  if constexpr (Static)
    return q_bf16 ? decode_int8_static_kernel<64, true, false>
                  : decode_int8_static_kernel<64, false, false>;
  else
    return q_bf16 ? decode_int8_kernel<64, true, false> : decode_int8_kernel<64, false, false>;
}

}  // namespace

hipError_t launch_decode_int8(const DecodeArgs& a, int head_dim, bool q_bf16, hipStream_t s) {
  if (a.unit_path) {
    const DecodeKernel k = head_dim == 128 ? (q_bf16 ? decode_int8_unit_kernel<128, true>
                                                     : decode_int8_unit_kernel<128, false>)
                                           : (q_bf16 ? decode_int8_unit_kernel<64, true>
                                                     : decode_int8_unit_kernel<64, false>);
    return launch_unit(k, a, head_dim, s);
  }
  const DecodeKernel k = pick_int8<false>(head_dim, a.group, q_bf16);
  return launch_pair(k, a, head_dim, s);
}

// units of 2 or 4 tiles (a unit of 3 runs in the 4-tile kernel)
template <template <int, bool, int> class W, int D, bool B>
DecodeKernel wide_kernel(int unit_tiles) {
  return unit_tiles == 2 ? W<D, B, 2>::kernel : W<D, B, kMaxUnitTiles>::kernel;
}
template <int D, bool B, int NT>
struct Int8Wide {
  static constexpr DecodeKernel kernel = decode_int8_wide_kernel<D, B, NT>;
};
template <int D, bool B, int NT>
struct Bits16Wide {
  static constexpr DecodeKernel kernel = decode_16bit_wide_kernel<D, B, NT>;
};

hipError_t launch_decode_int8_multi(const DecodeArgs& a, int head_dim, bool q_bf16,
                                    hipStream_t s) {
  DecodeKernel k;
  if (a.unit_tiles == 1)
    k = head_dim == 128
            ? (q_bf16 ? decode_int8_multi_kernel<128, true> : decode_int8_multi_kernel<128, false>)
            : (q_bf16 ? decode_int8_multi_kernel<64, true> : decode_int8_multi_kernel<64, false>);
  else
    k = head_dim == 128 ? (q_bf16 ? wide_kernel<Int8Wide, 128, true>(a.unit_tiles)
                                  : wide_kernel<Int8Wide, 128, false>(a.unit_tiles))
                        : (q_bf16 ? wide_kernel<Int8Wide, 64, true>(a.unit_tiles)
                                  : wide_kernel<Int8Wide, 64, false>(a.unit_tiles));
  return launch_pair(k, a, head_dim, s);
}

hipError_t launch_decode_int8_static(const DecodeArgs& a, int head_dim, bool q_bf16,
                                     hipStream_t s) {
  if (a.unit_path) {
    const DecodeKernel k = head_dim == 128 ? (q_bf16 ? decode_int8_static_unit_kernel<128, true>
                                                     : decode_int8_static_unit_kernel<128, false>)
                                           : (q_bf16 ? decode_int8_static_unit_kernel<64, true>
                                                     : decode_int8_static_unit_kernel<64, false>);
    return launch_unit(k, a, head_dim, s);
  }
  const DecodeKernel k = pick_int8<true>(head_dim, a.group, q_bf16);
  return launch_pair(k, a, head_dim, s);
}

hipError_t launch_decode_16bit(const DecodeArgs& a, int head_dim, bool kv_bf16,
                               hipStream_t s) {
  if (a.unit_path) {
    const DecodeKernel k = head_dim == 128 ? (kv_bf16 ? decode_16bit_unit_kernel<128, true>
                                                      : decode_16bit_unit_kernel<128, false>)
                                           : (kv_bf16 ? decode_16bit_unit_kernel<64, true>
                                                      : decode_16bit_unit_kernel<64, false>);
    return launch_unit(k, a, head_dim, s);
  }
  const DecodeKernel k =
      head_dim == 128
          ? (kv_bf16 ? decode_16bit_kernel<128, true> : decode_16bit_kernel<128, false>)
          : (kv_bf16 ? decode_16bit_kernel<64, true> : decode_16bit_kernel<64, false>);
  return launch_pair(k, a, head_dim, s);
}

hipError_t launch_decode_16bit_multi(const DecodeArgs& a, int head_dim, bool kv_bf16,
                                     hipStream_t s) {
  DecodeKernel k;
  if (a.unit_tiles == 1)
    k = head_dim == 128 ? (kv_bf16 ? decode_16bit_multi_kernel<128, true>
                                   : decode_16bit_multi_kernel<128, false>)
                        : (kv_bf16 ? decode_16bit_multi_kernel<64, true>
                                   : decode_16bit_multi_kernel<64, false>);
  else
    k = head_dim == 128 ? (kv_bf16 ? wide_kernel<Bits16Wide, 128, true>(a.unit_tiles)
                                   : wide_kernel<Bits16Wide, 128, false>(a.unit_tiles))
                        : (kv_bf16 ? wide_kernel<Bits16Wide, 64, true>(a.unit_tiles)
                                   : wide_kernel<Bits16Wide, 64, false>(a.unit_tiles));
  return launch_pair(k, a, head_dim, s);
}

}  // namespace pdakv
