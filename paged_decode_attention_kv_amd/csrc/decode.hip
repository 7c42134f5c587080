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
// pages w, w+4, ... of that run. One page = 16 tokens = one 16x16 MFMA tile:
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
//    one dimension share a 32-bit word in the page, which is the A operand of
//    one lane. The fp32 probability (with the V scale folded in) is split into
//    a high and a low fp16 part (22 significant bits), both contracted in one
//    16x16x32 instruction.
//  * Online softmax state (running max M, sum l, accumulator) lives in the
//    lanes of head l % 16; the V scale sV = f * 2^e (f in [0.5, 1)) enters
//    the running max as a base-2 exponent so that the folded probabilities
//    P = 2^(s + e - M) * f stay in [0, 1] (times 2^12 to keep the low fp16
//    parts out of the subnormal range).
// After the page loop the four waves combine through LDS; one split either
// writes the final row (single-split launches) or a partial (max, sum,
// accumulator) that merge_splits_kernel combines.
#include "device_util.h"
#include "launch.h"

namespace pdakv {

namespace {

constexpr float kPScale = 12.0f;  // probabilities are carried times 2^12

template <int D>
struct DecodeShared {
  int blk[kMaxPagesPerSplit];
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  float acc[kWaves][kMaxGroup][D];
};

// Element loads of q (any stride, 2-byte aligned).
__device__ __forceinline__ uint16_t q_bits(const DecodeArgs& a, int b, int h, int d) {
  return static_cast<const uint16_t*>(a.q)[b * a.q_ss + h * a.q_sh + d];
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

// Write zeros to the G output rows of (b, group g): empty context.
__device__ void write_zero_rows(const DecodeArgs& a, int b, int g, int D) {
  for (int i = threadIdx.x; i < a.group * D; i += blockDim.x) {
    const int h = g * a.group + i / D;
    store_out(a.out, a.out_dtype, b * a.out_ss + h * a.out_sh + i % D, 0.f);
  }
}

// Combine the four waves' (m, l, acc) of this workgroup and emit the final
// rows or a split partial.
template <int D>
__device__ void combine_and_store(const DecodeArgs& a, DecodeShared<D>& sh, int b, int g,
                                  int split) {
  const bool direct = a.max_splits == 1;
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

// ---------------------------------------------------------------------------
// INT8 pages
// ---------------------------------------------------------------------------
template <int D, bool QBF16>
__global__ __launch_bounds__(64 * kWaves) void decode_int8_kernel(DecodeArgs a) {
  constexpr int HB = 32 * D + 64;  // head block bytes
  constexpr int NJ = D / 32;       // QK instructions (16x16x32)
  constexpr int NK = D / 64;       // 16-byte K loads per lane
  constexpr int ND = D / 16;       // PV instructions (one per 16 output dims)
  constexpr int NV = D / 64;       // 16-byte V loads per lane
  __shared__ DecodeShared<D> sh;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, i16 = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int L = context_len(a, b, threadIdx.x == 0 && split == 0);
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = split * a.pages_per_split;
  if (p0 >= npages) {
    if (a.max_splits == 1 && split == 0) write_zero_rows(a, b, g, D);
    return;
  }
  const int np = min(npages - p0, a.pages_per_split);
  load_block_ids(a, sh.blk, b, p0, np);

  // q fragment for QK instruction j: dims 64*(j/2) + 16*kb + 8*(j%2) + r,
  // the same dims the K loads below place in the A operand.
  const bool hvalid = i16 < a.group;
  const int h = g * a.group + i16;
  float qv[NJ * 8];
  float qmax = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int d = 64 * (j / 2) + 16 * kb + 8 * (j % 2) + r;
      const float x = hvalid ? bits16_to_f32<QBF16>(q_bits(a, b, h, d)) : 0.f;
      qv[j * 8 + r] = x;
      qmax = fmaxf(qmax, fabsf(x));
    }
  qmax = col_max(qmax);
  // power of two putting max|q| in [2^14, 2^15): exact for fp16 and bf16 q
  const int kq = qmax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(qmax) : 0;
  h8_t qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r)
      qf[j][r] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(qv[j * 8 + r], kq));
  const float qscale = __builtin_amdgcn_ldexpf(a.scale_log2, -kq);

  float m_run = -INFINITY, l_run = 0.f;
  f4_t acc[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};

  __syncthreads();

  for (int pi = wave; pi < np; pi += kWaves) {
    const int blk = sh.blk[pi];
    if (blk < 0) continue;  // flagged page: skipped
    const uint8_t* hp = a.pool + static_cast<int64_t>(blk) * a.page_bytes + g * HB;
    u4_t kr[NK], vr[NV];
#pragma unroll
    for (int i = 0; i < NK; ++i)
      kr[i] = *reinterpret_cast<const u4_t*>(hp + i16 * D + 64 * i + 16 * kb);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      vr[i] = *reinterpret_cast<const u4_t*>(hp + 16 * D + kb * 4 * D + 256 * i + 16 * i16);
    const u2_t ksr = *reinterpret_cast<const u2_t*>(hp + 32 * D + 8 * kb);
    const u2_t vsr = *reinterpret_cast<const u2_t*>(hp + 32 * D + 32 + 8 * kb);

    // S = K q^T for 16 tokens x 16 (padded) heads
    f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const u2_t c0 = i8x4_to_f16x4(kr[j / 2][2 * (j % 2)]);
      const u2_t c1 = i8x4_to_f16x4(kr[j / 2][2 * (j % 2) + 1]);
      const u4_t kw = {c0.x, c0.y, c1.x, c1.y};
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, kw), qf[j], s, 0, 0, 0);
    }

    // lane holds tokens tok0 + j of head i16
    const int tok0 = (p0 + pi) * kBlockSize + 4 * kb;
    const uint16_t skb[4] = {static_cast<uint16_t>(ksr.x), static_cast<uint16_t>(ksr.x >> 16),
                             static_cast<uint16_t>(ksr.y), static_cast<uint16_t>(ksr.y >> 16)};
    const uint16_t svb[4] = {static_cast<uint16_t>(vsr.x), static_cast<uint16_t>(vsr.x >> 16),
                             static_cast<uint16_t>(vsr.y), static_cast<uint16_t>(vsr.y >> 16)};
    float z[4], f[4];
    int e[4];
    float zmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = tok0 + j < L;
      const float sv = f16_bits_to_f32(svb[j]);
      const float logit2 = s[j] * f16_bits_to_f32(skb[j]) * qscale;
      const int ej = __builtin_amdgcn_frexp_expf(sv);
      e[j] = valid ? ej : 0;
      f[j] = valid ? __builtin_amdgcn_frexp_mantf(sv) : 0.f;
      z[j] = valid ? logit2 + static_cast<float>(ej) : -INFINITY;
      zmax = fmaxf(zmax, z[j]);
    }
    zmax = col_max(zmax);
    const float m_new = fmaxf(m_run, zmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int k = 0; k < ND; ++k) acc[k] *= alpha;

    float hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pe = exp2f(z[j] - m_new + kPScale);          // <= 2^12
      l_run += __builtin_amdgcn_ldexpf(pe, -e[j]);            // 2^(12 + logit2 - M)
      const float p = pe * f[j];                               // 2^(12 - M) 2^logit2 sV
      const _Float16 ph = static_cast<_Float16>(p);
      hi[j] = static_cast<float>(ph);
      lo[j] = p - hi[j];
    }
    const u4_t pw = {pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]),
                     pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3])};
    const h8_t pf = __builtin_bit_cast(h8_t, pw);

    // O^T += V^T P^T: instruction k covers dims 64*(k/4) + 4*(row) + k%4
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      const u2_t c = i8x4_to_f16x4(vr[k / 4][k % 4]);
      const u4_t vw = {c.x, c.y, c.x, c.y};
      acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, vw), pf, acc[k],
                                                      0, 0, 0);
    }
  }

  l_run = col_sum(l_run);
  if (hvalid) {
    if (kb == 0) {
      sh.m[wave][i16] = m_run;
      sh.l[wave][i16] = l_run;
    }
#pragma unroll
    for (int k = 0; k < ND; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sh.acc[wave][i16][64 * (k / 4) + 16 * kb + 4 * j + (k % 4)] = acc[k][j];
  }
  __syncthreads();
  combine_and_store<D>(a, sh, b, g, split);
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

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kWaves) void decode_16bit_kernel(DecodeArgs a) {
  constexpr int HB = 64 * D;  // head block bytes
  constexpr int NJ = D / 32;  // QK instructions; also 16-byte K loads per lane
  constexpr int ND = D / 16;  // PV instructions
  constexpr int NV = D / 32;  // 16-byte V loads per lane (two instructions each)
  __shared__ DecodeShared<D> sh;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, i16 = lane & 15, kb = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int L = context_len(a, b, threadIdx.x == 0 && split == 0);
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int p0 = split * a.pages_per_split;
  if (p0 >= npages) {
    if (a.max_splits == 1 && split == 0) write_zero_rows(a, b, g, D);
    return;
  }
  const int np = min(npages - p0, a.pages_per_split);
  load_block_ids(a, sh.blk, b, p0, np);

  // q fragment j: dims 32*j + 8*kb + r (raw 16-bit values, same dtype as K)
  const bool hvalid = i16 < a.group;
  const int h = g * a.group + i16;
  u4_t qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = 32 * j + 8 * kb + 2 * r;
      const uint32_t x0 = hvalid ? q_bits(a, b, h, d) : 0u;
      const uint32_t x1 = hvalid ? q_bits(a, b, h, d + 1) : 0u;
      w[r] = x0 | (x1 << 16);
    }
    qf[j] = u4_t{w[0], w[1], w[2], w[3]};
  }

  float m_run = -INFINITY, l_run = 0.f;
  f4_t acc[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};

  __syncthreads();

  for (int pi = wave; pi < np; pi += kWaves) {
    const int blk = sh.blk[pi];
    if (blk < 0) continue;
    const uint8_t* hp = a.pool + static_cast<int64_t>(blk) * a.page_bytes + g * HB;
    u4_t kr[NJ], vr[NV];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      kr[j] = *reinterpret_cast<const u4_t*>(hp + i16 * 2 * D + 64 * j + 16 * kb);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      vr[i] = *reinterpret_cast<const u4_t*>(hp + 32 * D + kb * 8 * D + 256 * i + 16 * i16);

    f4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) s = mfma16x16x32<BF16>(kr[j], qf[j], s);

    const int tok0 = (p0 + pi) * kBlockSize + 4 * kb;
    float z[4];
    float zmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[j] = tok0 + j < L ? s[j] * a.scale_log2 : -INFINITY;
      zmax = fmaxf(zmax, z[j]);
    }
    zmax = col_max(zmax);
    const float m_new = fmaxf(m_run, zmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int k = 0; k < ND; ++k) acc[k] *= alpha;

    float pe[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pe[j] = exp2f(z[j] - m_new + kPScale);
      l_run += pe[j];
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
      const u4_t pa = {p1[0] | (p1[1] << 16), p1[2] | (p1[3] << 16), p2[0] | (p2[1] << 16),
                       p2[2] | (p2[3] << 16)};
      const u4_t pb = {p3[0] | (p3[1] << 16), p3[2] | (p3[3] << 16), 0u, 0u};
#pragma unroll
      for (int k = 0; k < ND; ++k) {
        const uint32_t w0 = vr[k / 2][2 * (k % 2)], w1 = vr[k / 2][2 * (k % 2) + 1];
        const u4_t vw = {w0, w1, w0, w1};
        acc[k] = mfma16x16x32<true>(vw, pa, acc[k]);
        acc[k] = mfma16x16x32<true>(vw, pb, acc[k]);
      }
    } else {
      float hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hi[j] = static_cast<float>(static_cast<_Float16>(pe[j]));
        lo[j] = pe[j] - hi[j];
      }
      const u4_t pw = {pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]),
                       pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3])};
#pragma unroll
      for (int k = 0; k < ND; ++k) {
        const uint32_t w0 = vr[k / 2][2 * (k % 2)], w1 = vr[k / 2][2 * (k % 2) + 1];
        const u4_t vw = {w0, w1, w0, w1};
        acc[k] = mfma16x16x32<false>(vw, pw, acc[k]);
      }
    }
  }

  l_run = col_sum(l_run);
  if (hvalid) {
    if (kb == 0) {
      sh.m[wave][i16] = m_run;
      sh.l[wave][i16] = l_run;
    }
#pragma unroll
    for (int k = 0; k < ND; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sh.acc[wave][i16][32 * (k / 2) + 8 * kb + 2 * j + (k % 2)] = acc[k][j];
  }
  __syncthreads();
  combine_and_store<D>(a, sh, b, g, split);
}

// ---------------------------------------------------------------------------
// split merge: out = sum_i 2^(m_i - m) acc_i / sum_i 2^(m_i - m) l_i
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void merge_splits_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.num_q_heads, h = bh % a.num_q_heads;
  const int d = threadIdx.x;
  const int L = context_len(a, b, false);
  const int npages = (L + kBlockSize - 1) / kBlockSize;
  const int n = (npages + a.pages_per_split - 1) / a.pages_per_split;
  const float* p = a.ws + static_cast<int64_t>(bh) * a.max_splits * (D + 2);
  float ms = -INFINITY;
  for (int i = 0; i < n; ++i) ms = fmaxf(ms, p[i * (D + 2) + D]);
  float num = 0.f, den = 0.f;
  for (int i = 0; i < n; ++i) {
    const float c = exp2f(p[i * (D + 2) + D] - ms);
    num += c * p[i * (D + 2) + d];
    den += c * p[i * (D + 2) + D + 1];
  }
  store_out(a.out, a.out_dtype, b * a.out_ss + h * a.out_sh + d, n > 0 ? num / den : 0.f);
}

template <int D>
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  if (a.max_splits == 1) return hipSuccess;
  hipLaunchKernelGGL((merge_splits_kernel<D>), dim3(a.num_seqs * a.num_q_heads), dim3(D), 0, s,
                     a);
  return hipGetLastError();
}

dim3 decode_grid(const DecodeArgs& a) {
  return dim3(a.max_splits, a.num_kv_heads, a.num_seqs);
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
  hipError_t e = hipGetLastError();
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return head_dim == 128 ? launch_merge<128>(a, s) : launch_merge<64>(a, s);
}

}  // namespace pdakv
