// Paged decode attention over INT8 pages (codes + FP16 per-token scales) and
// over 16-bit pages (the control), for gfx950.
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
// grid = (split, KV head, sequence); a workgroup of four waves owns one
// (sequence, KV head) and a run of `pages_per_split` pages; wave w takes the
// pages w, w+4, w+8, ... and keeps the next page's loads in flight while it
// computes the current one. One page = 16 tokens = one 16x16 MFMA tile:
//  * QK: S[t][h] = sum_d K[t][d] * q[h][d] with K in the A operand (row t =
//    lane % 16) and the G query heads of the group in the B operand (column
//    h = lane % 16, zero-padded to 16). Every K byte is fetched once and
//    shared by the whole GQA group inside the matrix instruction. INT8 codes
//    become fp16 exactly; q is scaled by a power of two into fp16 range
//    (exact for fp16/bf16 inputs down to far below any contributing term) and
//    the scale is undone on the fp32 logits. Products are exact, sums fp32.
//  * The result tile holds, in lane l, tokens 4*(l/16)+j (j = 0..3) of head
//    l % 16 — exactly the B-operand layout the PV product needs, so the
//    probabilities never leave registers.
//  * PV: O^T[d][h] = sum_t V[t][d] * P[h][t]. The V codes of four tokens of
//    one dimension share a 32-bit word in the page: the A operand of one lane
//    of a 16x16x16 instruction. The fp32 probability (V scale folded in) is
//    split into a high and a low fp16 part (22 significant bits), contracted
//    by two instructions.
//  * Online softmax state (running max m, sum l, accumulator) lives in the
//    lanes of head l % 16. The V scale sV = f * 2^e (f in [0.5, 1)) enters
//    the logit as the base-2 exponent e, so the folded probabilities
//    P = 2^(s + e - m) * f never leave the fp16 range whatever the scales.
// After the page loop the four waves combine through LDS. A sequence with a
// single split writes its rows directly; otherwise every split writes a
// partial (max, sum, accumulator) and merge_splits_kernel combines them.
// (Merging in the last-arriving workgroup would need device-scope fences,
// which write back and invalidate the L2 of the XCD: far dearer than the
// second launch.)
#include "device_util.h"
#include "launch.h"

namespace pdakv {

namespace {

// Probabilities are carried times 2^kPScale relative to the running max m; m
// is raised only when a new logit exceeds it by more than kTau (base-2
// units), so the accumulator is rescaled rarely and probabilities stay below
// 2^(kPScale + kTau) = 2^15, inside the fp16 range of the PV operand, with
// their low fp16 parts clear of the subnormal range.
constexpr float kTau = 8.0f;
constexpr float kPScale = 7.0f;

template <int D>
struct DecodeShared {
  int blk[kMaxPagesPerSplit];
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  float acc[kWaves][kMaxGroup][D];
};

// Eight consecutive 16-bit q elements (dims d0..d0+7) of head h, as four
// words. One 16-byte load when the host found q's pointer and strides 16-byte
// aligned, else eight 2-byte loads. Always issued (no per-lane branch), so the
// loads of a wave overlap.
__device__ __forceinline__ u4_t q_chunk8(const DecodeArgs& a, int b, int h, int d0) {
  const uint16_t* row = static_cast<const uint16_t*>(a.q) + b * a.q_ss + h * a.q_sh + d0;
  if (a.q_vec16) return *reinterpret_cast<const u4_t*>(row);
  u4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = row[2 * i] | (static_cast<uint32_t>(row[2 * i + 1]) << 16);
  return w;
}

// Clamped context length of sequence b (flags an out-of-range value).
__device__ __forceinline__ int context_len(const DecodeArgs& a, int b, bool report) {
  int L = a.ctx[b];
  if (L < 0 || L > a.max_ctx) {
    if (report) raise_flag(a.err, PDAKV_EFLAG_CONTEXT_RANGE);
    L = L < 0 ? 0 : a.max_ctx;
  }
  return L;
}

// Load this split's block-table entries into LDS (invalid ids -> -1).
__device__ __forceinline__ void load_block_ids(const DecodeArgs& a, int* sblk, int b, int p0,
                                               int np) {
  if (static_cast<int>(threadIdx.x) < np) {
    int blk = a.bt[static_cast<int64_t>(b) * a.bt_stride + p0 + threadIdx.x];
    if (blk < 0 || blk >= a.num_blocks) {
      raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
      blk = -1;
    }
    sblk[threadIdx.x] = blk;
  }
}

// Zero output rows of (b, group g): empty context.
__device__ void write_zero_rows(const DecodeArgs& a, int b, int g, int D) {
  for (int i = threadIdx.x; i < a.group * D; i += blockDim.x) {
    const int h = g * a.group + i / D;
    store_out(a.out, a.out_dtype, b * a.out_ss + h * a.out_sh + i % D, 0.f);
  }
}

// Combine the four waves' (m, l, acc); write the final rows (the sequence has
// a single split) or this split's partial for merge_splits_kernel.
template <int D>
__device__ void finish(const DecodeArgs& a, DecodeShared<D>& sh, int b, int g, int split,
                       int nsplit) {
  const bool direct = nsplit == 1;
  for (int i = threadIdx.x; i < a.group * D; i += blockDim.x) {
    const int hh = i / D, d = i % D;
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, sh.m[w][hh]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = exp2f(sh.m[w][hh] - ms);  // 0 for a wave without pages
      num += c * sh.acc[w][hh][d];
      den += c * sh.l[w][hh];
    }
    const int h = g * a.group + hh;
    if (direct) {
      store_out(a.out, a.out_dtype, b * a.out_ss + h * a.out_sh + d, num / den);
    } else {
      float* p = a.ws + ((static_cast<int64_t>(b) * a.num_q_heads + h) * a.max_splits + split) *
                            (D + 2);
      p[d] = num;
      if (d == 0) {
        p[D] = ms;
        p[D + 1] = den;
      }
    }
  }
}

template <int ND>
struct SoftmaxState {
  float m;   // running max (base-2 units)
  float mk;  // m - kPScale
  float l;
  f4_t acc[ND];
};

template <int ND>
__device__ __forceinline__ void softmax_init(SoftmaxState<ND>& st) {
  st.m = -INFINITY;
  st.mk = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int k = 0; k < ND; ++k) st.acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};
}

template <int ND>
__device__ __forceinline__ void raise_max(SoftmaxState<ND>& st, float zmax) {
  zmax = col_max(zmax);
  if (__any(zmax > st.m + kTau)) {
    const float m_new = fmaxf(st.m, zmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 on the first page
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
// [2^14, 2^15); fragment j, slot r holds dim qdim0(j) + r. Lanes of padding
// heads (hvalid false) read head h_load and use zeros. Returns the factor that
// turns the MFMA dot products into base-2 logits.
template <int NJ, bool QBF16, typename DimFn>
__device__ __forceinline__ float load_q_scaled(const DecodeArgs& a, int b, int h_load,
                                               bool hvalid, DimFn qdim0, h8_t* qf) {
  u4_t raw[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) raw[j] = q_chunk8(a, b, h_load, qdim0(j));
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

// ---------------------------------------------------------------------------
// INT8 pages
// ---------------------------------------------------------------------------
template <int D>
struct Int8Page {
  u4_t k[D / 64];  // K codes: token i16, dims 64*i + 16*kb + (0..15)
  u4_t v[D / 64];  // V codes: dims 64*i + 4*i16 + (0..3), tokens 4*kb + (0..3)
  u2_t ks, vs;     // scales of tokens 4*kb + (0..3)
};

template <int D>
__device__ __forceinline__ void load_int8_page(Int8Page<D>& pg, const uint8_t* hp, int i16,
                                               int kb) {
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    pg.k[i] = *reinterpret_cast<const u4_t*>(hp + i16 * D + 64 * i + 16 * kb);
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    pg.v[i] = *reinterpret_cast<const u4_t*>(hp + 16 * D + kb * 4 * D + 256 * i + 16 * i16);
  pg.ks = *reinterpret_cast<const u2_t*>(hp + 32 * D + 8 * kb);
  pg.vs = *reinterpret_cast<const u2_t*>(hp + 32 * D + 32 + 8 * kb);
}

template <int D>
__device__ __forceinline__ f4_t int8_qk(const Int8Page<D>& pg, const h8_t* qf) {
  f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    const u2_t c0 = i8x4_to_f16x4_perm(pg.k[j / 2][2 * (j % 2)]);
    const u2_t c1 = i8x4_to_f16x4_perm(pg.k[j / 2][2 * (j % 2) + 1]);
    const u4_t kw = {c0.x, c0.y, c1.x, c1.y};
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, kw), qf[j], s, 0, 0, 0);
  }
  return s;
}

// One page; tok0 = position of this lane's first token (4*kb within the
// page). MASK: the page may extend past L (its last page); then the V scales of
// the tokens past L are replaced by 1.0 (the slots may hold anything) and their
// logits by -inf.
template <int D, bool MASK>
__device__ __forceinline__ void int8_page_step(const Int8Page<D>& pg, bool valid, const h8_t* qf,
                                               float qscale, int tok0, int L,
                                               SoftmaxState<D / 16>& st) {
  constexpr int ND = D / 16;
  const f4_t s = int8_qk<D>(pg, qf);
  const uint32_t ksw[2] = {pg.ks.x, pg.ks.y};
  uint32_t vsw[2] = {pg.vs.x, pg.vs.y};
  const bool tail = MASK && tok0 - 4 * static_cast<int>((threadIdx.x & 63) >> 4) + kBlockSize > L;
  if (tail) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tok0 + j >= L) vsw[j / 2] = (vsw[j / 2] & (0xFFFF0000u >> (16 * (j % 2)))) |
                                      (0x3C00u << (16 * (j % 2)));
  }
  float z[4];
  int e[4];
  _Float16 f[4];
  float zmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sk = f16_bits_to_f32(static_cast<uint16_t>(ksw[j / 2] >> (16 * (j % 2))));
    const _Float16 sv =
        __builtin_bit_cast(_Float16, static_cast<uint16_t>(vsw[j / 2] >> (16 * (j % 2))));
    e[j] = __builtin_amdgcn_frexp_exph(sv);
    f[j] = __builtin_amdgcn_frexp_manth(sv);
    // base-2 logit plus the exponent of the V scale: P = 2^(z - m) * f
    z[j] = s[j] * sk * qscale + static_cast<float>(e[j]);
    if (tail) z[j] = tok0 + j < L ? z[j] : -INFINITY;
    zmax = max_nc(zmax, z[j]);
  }
  raise_max(st, zmax);
  float hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x = __builtin_amdgcn_exp2f(z[j] - st.mk);  // 2^(kPScale + z - m)
    st.l += __builtin_amdgcn_ldexpf(x, -e[j]);
    const float p = x * static_cast<float>(f[j]);
    hi[j] = static_cast<float>(static_cast<_Float16>(p));
    lo[j] = p - hi[j];
  }
  const h4_t ph = __builtin_bit_cast(h4_t, u2_t{pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3])});
  const h4_t pl = __builtin_bit_cast(h4_t, u2_t{pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3])});
  // O^T += V^T P^T; instruction k covers dims 64*(k/4) + 4*(row) + k%4, its
  // K-slots hold tokens 4*kb + (0..3)
#pragma unroll
  for (int k = 0; k < ND; ++k) {
    const h4_t vw = __builtin_bit_cast(h4_t, i8x4_to_f16x4_perm(pg.v[k / 4][k % 4]));
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, ph, st.acc[k], 0, 0, 0);
    st.acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(vw, pl, st.acc[k], 0, 0, 0);
  }
}

// Load page p of the split into pg. The loads are issued unconditionally (a
// missing or flagged page reads page 0, which exists, and is then skipped) so
// that the number of loads in flight is the same on every path and the
// compiler can wait for the current page only.
template <int D>
__device__ __forceinline__ bool int8_load(Int8Page<D>& pg, const DecodeShared<D>& sh, int p,
                                          int np, const uint8_t* base, int64_t page_bytes,
                                          int i16, int kb) {
  const int blk = p < np ? sh.blk[p] : -1;
  load_int8_page<D>(pg, base + (blk >= 0 ? blk : 0) * page_bytes, i16, kb);
  return blk >= 0;
}

// page_tok = position of the page's first token. (A separate unmasked path
// for full pages costs more registers than the masks cost instructions.)
template <int D>
__device__ __forceinline__ void int8_step(const Int8Page<D>& pg, bool valid, const h8_t* qf,
                                          float qscale, int page_tok, int kb, int L,
                                          SoftmaxState<D / 16>& st) {
  if (!valid) return;  // missing or flagged page: nothing to attend
  int8_page_step<D, true>(pg, true, qf, qscale, page_tok + 4 * kb, L, st);
}

// 4 waves per SIMD: the compiler keeps this kernel within 128 VGPRs
template <int D, bool QBF16>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(4))) void
decode_int8_kernel(DecodeArgs a) {
  constexpr int HB = 32 * D + 64;  // head block bytes
  constexpr int NJ = D / 32;       // QK instructions (16x16x32)
  constexpr int ND = D / 16;       // PV output blocks of 16 dims
  __shared__ DecodeShared<D> sh;

  const int split = a.heads_fastest ? blockIdx.y : blockIdx.x;
  const int g = a.heads_fastest ? blockIdx.x : blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, i16 = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int L = context_len(a, b, threadIdx.x == 0 && split == 0);
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = split * a.pages_per_split;
  if (p0 >= npages) {
    if (npages == 0 && split == 0) write_zero_rows(a, b, g, D);
    return;
  }
  const int nsplit = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const int np = min(npages - p0, a.pages_per_split);
  load_block_ids(a, sh.blk, b, p0, np);

  const bool hvalid = i16 < a.group;
  h8_t qf[NJ];
  const float qscale = load_q_scaled<NJ, QBF16>(
      a, b, g * a.group + (hvalid ? i16 : 0), hvalid,
      [kb](int j) { return 64 * (j / 2) + 16 * kb + 8 * (j % 2); }, qf);

  SoftmaxState<ND> st;
  softmax_init(st);
  __syncthreads();

  // Ping-pong register buffers: page i+4's loads are in flight while page i
  // is computed. Wave w owns pages w, w+4, w+8, ... of the split.
  const uint8_t* base = a.pool + static_cast<int64_t>(g) * HB;
  Int8Page<D> pa, pb;
  int p = wave;
  bool va = int8_load<D>(pa, sh, p, np, base, a.page_bytes, i16, kb);
  while (p < np) {
    const int p1 = p + kWaves;
    const bool vb = int8_load<D>(pb, sh, p1, np, base, a.page_bytes, i16, kb);
    int8_step<D>(pa, va, qf, qscale, (p0 + p) * kBlockSize, kb, L, st);
    if (p1 >= np) break;
    const int p2 = p1 + kWaves;
    va = int8_load<D>(pa, sh, p2, np, base, a.page_bytes, i16, kb);
    int8_step<D>(pb, vb, qf, qscale, (p0 + p1) * kBlockSize, kb, L, st);
    p = p2;
  }

  st.l = col_sum(st.l);
  if (hvalid) {
    if (kb == 0) {
      sh.m[wave][i16] = st.m;
      sh.l[wave][i16] = st.l;
    }
#pragma unroll
    for (int k = 0; k < ND; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sh.acc[wave][i16][64 * (k / 4) + 16 * kb + 4 * j + (k % 4)] = st.acc[k][j];
  }
  __syncthreads();
  finish<D>(a, sh, b, g, split, nsplit);
}

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
__device__ __forceinline__ void load_page16(Page16<D>& pg, const uint8_t* hp, int i16, int kb) {
#pragma unroll
  for (int j = 0; j < D / 32; ++j)
    pg.k[j] = *reinterpret_cast<const u4_t*>(hp + i16 * 2 * D + 64 * j + 16 * kb);
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    pg.v[i] = *reinterpret_cast<const u4_t*>(hp + 32 * D + kb * 8 * D + 256 * i + 16 * i16);
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

template <int D, bool BF16, bool MASK>
__device__ __forceinline__ void page16_step(const Page16<D>& pg, bool valid, const u4_t* qf,
                                            float scale_log2, int tok0, int L,
                                            SoftmaxState<D / 16>& st) {
  constexpr int NJ = D / 32, ND = D / 16;
  f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) s = mfma16x16x32<BF16>(pg.k[j], qf[j], s);
  const bool tail = MASK && tok0 - 4 * static_cast<int>((threadIdx.x & 63) >> 4) + kBlockSize > L;
  float z[4];
  float zmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z[j] = s[j] * scale_log2;
    if (tail) z[j] = tok0 + j < L ? z[j] : -INFINITY;
    zmax = max_nc(zmax, z[j]);
  }
  raise_max(st, zmax);
  float pe[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pe[j] = __builtin_amdgcn_exp2f(z[j] - st.mk);
    st.l += pe[j];
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
      const u2_t vw = {pg.v[k / 2][2 * (k % 2)], pg.v[k / 2][2 * (k % 2) + 1]};
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
      const u2_t vw = {pg.v[k / 2][2 * (k % 2)], pg.v[k / 2][2 * (k % 2) + 1]};
      st.acc[k] = mfma16x16x16<false>(vw, ph, st.acc[k]);
      st.acc[k] = mfma16x16x16<false>(vw, pl, st.acc[k]);
    }
  }
}

// Unconditional loads, as int8_load.
template <int D>
__device__ __forceinline__ bool load16(Page16<D>& pg, const DecodeShared<D>& sh, int p, int np,
                                       const uint8_t* base, int64_t page_bytes, int i16,
                                       int kb) {
  const int blk = p < np ? sh.blk[p] : -1;
  load_page16<D>(pg, base + (blk >= 0 ? blk : 0) * page_bytes, i16, kb);
  return blk >= 0;
}

template <int D, bool BF16>
__device__ __forceinline__ void step16(const Page16<D>& pg, bool valid, const u4_t* qf,
                                       float scale_log2, int page_tok, int kb, int L,
                                       SoftmaxState<D / 16>& st) {
  if (!valid) return;  // missing or flagged page: nothing to attend
  page16_step<D, BF16, true>(pg, valid, qf, scale_log2, page_tok + 4 * kb, L, st);
}

// 3 waves per SIMD: the compiler keeps this kernel within 168 VGPRs
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3))) void
decode_16bit_kernel(DecodeArgs a) {
  constexpr int HB = 64 * D;  // head block bytes
  constexpr int NJ = D / 32;  // QK instructions
  constexpr int ND = D / 16;  // PV output blocks
  __shared__ DecodeShared<D> sh;

  const int split = a.heads_fastest ? blockIdx.y : blockIdx.x;
  const int g = a.heads_fastest ? blockIdx.x : blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, i16 = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int L = context_len(a, b, threadIdx.x == 0 && split == 0);
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = split * a.pages_per_split;
  if (p0 >= npages) {
    if (npages == 0 && split == 0) write_zero_rows(a, b, g, D);
    return;
  }
  const int nsplit = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const int np = min(npages - p0, a.pages_per_split);
  load_block_ids(a, sh.blk, b, p0, np);

  // q fragment j: dims 32*j + 8*kb + r (raw 16-bit values, same dtype as K)
  const bool hvalid = i16 < a.group;
  const int h_load = g * a.group + (hvalid ? i16 : 0);
  u4_t qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) qf[j] = q_chunk8(a, b, h_load, 32 * j + 8 * kb);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (!hvalid) qf[j] = u4_t{0u, 0u, 0u, 0u};

  SoftmaxState<ND> st;
  softmax_init(st);
  __syncthreads();

  // Ping-pong register buffers, as in the INT8 kernel.
  const uint8_t* base = a.pool + static_cast<int64_t>(g) * HB;
  Page16<D> pa, pb;
  int p = wave;
  bool va = load16<D>(pa, sh, p, np, base, a.page_bytes, i16, kb);
  while (p < np) {
    const int p1 = p + kWaves;
    const bool vb = load16<D>(pb, sh, p1, np, base, a.page_bytes, i16, kb);
    step16<D, BF16>(pa, va, qf, a.scale_log2, (p0 + p) * kBlockSize, kb, L, st);
    if (p1 >= np) break;
    const int p2 = p1 + kWaves;
    va = load16<D>(pa, sh, p2, np, base, a.page_bytes, i16, kb);
    step16<D, BF16>(pb, vb, qf, a.scale_log2, (p0 + p1) * kBlockSize, kb, L, st);
    p = p2;
  }

  st.l = col_sum(st.l);
  if (hvalid) {
    if (kb == 0) {
      sh.m[wave][i16] = st.m;
      sh.l[wave][i16] = st.l;
    }
#pragma unroll
    for (int k = 0; k < ND; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sh.acc[wave][i16][32 * (k / 2) + 8 * kb + 2 * j + (k % 2)] = st.acc[k][j];
  }
  __syncthreads();
  finish<D>(a, sh, b, g, split, nsplit);
}

// split merge: out = sum_i 2^(m_i - m) acc_i / sum_i 2^(m_i - m) l_i for the
// sequences with more than one split (the others were written directly)
template <int D>
__global__ __launch_bounds__(D) void merge_splits_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.num_q_heads, h = bh % a.num_q_heads;
  const int d = threadIdx.x;
  const int L = context_len(a, b, false);
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int n = (npages + a.pages_per_split - 1) / a.pages_per_split;
  if (n <= 1) return;
  const float* p = a.ws + static_cast<int64_t>(bh) * a.max_splits * (D + 2);
  float ms = -INFINITY;
  for (int i = 0; i < n; ++i) ms = fmaxf(ms, p[i * (D + 2) + D]);
  float num = 0.f, den = 0.f;
  for (int i = 0; i < n; ++i) {
    const float c = exp2f(p[i * (D + 2) + D] - ms);
    num += c * p[i * (D + 2) + d];
    den += c * p[i * (D + 2) + D + 1];
  }
  store_out(a.out, a.out_dtype, b * a.out_ss + h * a.out_sh + d, num / den);
}

template <int D>
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  if (a.max_splits == 1) return hipSuccess;
  hipLaunchKernelGGL((merge_splits_kernel<D>), dim3(a.num_seqs * a.num_q_heads), dim3(D), 0, s,
                     a);
  return hipGetLastError();
}

dim3 decode_grid(const DecodeArgs& a) {
  return a.heads_fastest ? dim3(a.num_kv_heads, a.max_splits, a.num_seqs)
                         : dim3(a.max_splits, a.num_kv_heads, a.num_seqs);
}

}  // namespace

hipError_t launch_decode_int8(const DecodeArgs& a, int head_dim, bool q_bf16, hipStream_t s) {
  const dim3 grid = decode_grid(a), block(64 * kWaves);
  if (head_dim == 128) {
    if (q_bf16)
      hipLaunchKernelGGL((decode_int8_kernel<128, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_int8_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (q_bf16)
      hipLaunchKernelGGL((decode_int8_kernel<64, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_int8_kernel<64, false>), grid, block, 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return head_dim == 128 ? launch_merge<128>(a, s) : launch_merge<64>(a, s);
}

hipError_t launch_decode_16bit(const DecodeArgs& a, int head_dim, bool kv_bf16,
                               hipStream_t s) {
  const dim3 grid = decode_grid(a), block(64 * kWaves);
  if (head_dim == 128) {
    if (kv_bf16)
      hipLaunchKernelGGL((decode_16bit_kernel<128, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_16bit_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (kv_bf16)
      hipLaunchKernelGGL((decode_16bit_kernel<64, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_16bit_kernel<64, false>), grid, block, 0, s, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return head_dim == 128 ? launch_merge<128>(a, s) : launch_merge<64>(a, s);
}

}  // namespace pdakv
