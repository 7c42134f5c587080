// Quantize-on-write and 16-bit write into paged KV pools (gfx950).
//
// One wave (64 lanes) owns one to three consecutive spans of about four
// tokens of the call (each aligned to the V groups of the pages, below) for
// one KV head and handles their K and V rows; a workgroup holds four waves.
// Three pool formats: per-token INT8 (codes + FP16 scales), static-scale INT8
// (codes only) and 16-bit. The row quantizer (quant_row.h) follows
// MoE-Infinity PR #183 "feat: opt-in INT8 KV-cache quantization" ("What
// landed", format-contract bullet; "Precision & memory") and the zero-token
// rule of mlxcel PR #717 ("The Int8 bug and fix"). Four tokens that fill one
// V group of a page are stored with whole group words, so a prefill writes
// whole cache lines instead of a byte scatter. Every lane holds 8 elements
// of one row (D = 64: two KV heads per wave), so the per-row reductions and
// scale arithmetic of all the wave's rows run side by side in the same
// instructions.
#include <type_traits>

#include "device_util.h"
#include "launch.h"
#include "quant_row.h"

namespace pdakv {

namespace {

constexpr int kWriteWaves = 4;
constexpr int kQuad = 4;  // tokens per span: one V group of the page layout

// A KV head's code block in a page: element size E (1: INT8 codes, 2: 16-bit
// values), K rows at pos * D elements, V grouped four tokens at a time from
// 16 * D elements on (dimension d of tokens 4g .. 4g+3 in one group word).
// Every head's code block comes first in a page; per-token INT8 pages then
// hold every head's fp16 scales, a 16-byte record per four tokens (K scales
// of tokens 4g .. 4g+3, then their V scales).
template <int D, int E, bool Scales>
struct HeadLayout {
  static constexpr int kBytes = 32 * D * E;      // a head's code block
  static constexpr int kV = kBlockSize * D * E;  // byte offset of the V groups
  static constexpr int kScaleBytes = 64;         // a head's scale records
  // K scale of token pos, from the head's scale records (V: 8 bytes on)
  static __device__ __forceinline__ int ks_off(int pos) { return 16 * (pos / 4) + 2 * (pos % 4); }
};

// Tokens are dealt out four at a time, with each boundary between the fours
// moved back to the start of the V group its token lands in: boundary b
// moves to b - k when token b's slot is 4g + k and tokens b - k .. b - 1 hold
// slots 4g .. 4g + k - 1. Both sides of a boundary compute the same move, so
// every token is handled once; inside a run of consecutive slots (a prefill
// chunk, whatever its start offset in the page) every span then holds whole
// V groups. A wave takes N consecutive fours (spans) and reads the slots of
// tokens 4q - 4 .. 4q + 4N + 3 at once (one per lane), which covers all of
// its boundaries and tokens.
struct Span {
  int64_t t0;       // first token
  int n;            // tokens (1 .. 7; 0 or less past the call's end)
  int32_t slot[8];  // their slots (-1: padding or out of range)
};
template <int N>
__device__ __forceinline__ void load_spans(const WriteArgs& a, int64_t qd, int lane,
                                           Span (&sp)[N]) {
  constexpr int NS = kQuad * (N + 2);
  static_assert(NS <= 64, "one slot per lane");
  const int64_t base = qd * kQuad - kQuad, T = a.num_tokens;
  const int64_t cap = a.num_blocks * kBlockSize;
  // one load per lane, then every lane reads the slots
  const int64_t tl = base + lane;
  int32_t mine = a.slots[tl < 0 ? 0 : (tl >= T ? T - 1 : tl)];
  if (tl < 0 || tl >= T) mine = -1;
  int32_t S[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) S[j] = __builtin_amdgcn_readlane(mine, j);
  // boundary at token base + c
  auto bnd = [&](int c) -> int64_t {
    const int64_t b = base + c;
    if (b <= 0 || b >= T) return b;
    const int32_t s = S[c];
    const int k = s & 3;
    if (s < 0 || s >= cap || k == 0) return b;
    bool run = b >= k;
#pragma unroll
    for (int j = 1; j < kQuad; ++j) run = run && (j > k || S[c - j] == s - j);
    return run ? b - k : b;
  };
  bool bad = false;
  int64_t lo = bnd(kQuad);
#pragma unroll
  for (int p = 0; p < N; ++p) {
    const int64_t hi = bnd(kQuad * (p + 2));
    sp[p].t0 = lo;
    sp[p].n = static_cast<int>(min(hi, T) - lo);
    // token t0 + j is S[4p + off + j], off in 1 .. 4 (selected with constant
    // indexes: S stays in registers)
    const int off = static_cast<int>(lo - base) - kQuad * p;
    const int32_t* Sp = S + kQuad * p;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int32_t s = off == 1 ? Sp[1 + j] : off == 2 ? Sp[2 + j] : off == 3 ? Sp[3 + j] : Sp[4 + j];
      if (j >= sp[p].n) s = -1;
      bad = bad || s >= cap;
      sp[p].slot[j] = s >= cap ? -1 : s;
    }
    lo = hi;
  }
  if (bad && lane == 0) raise_flag(a.err, PDAKV_EFLAG_SLOT_RANGE);
}

// Up to four consecutive tokens t0 .. t0+nt-1 of a wave and their slots.
struct Quad {
  int32_t slot[kQuad];
  int nt;
};
template <int Round>
__device__ __forceinline__ Quad quad_of(const Span& sp) {
  Quad q;
  q.nt = min(kQuad, sp.n - kQuad * Round);
#pragma unroll
  for (int j = 0; j < kQuad; ++j) q.slot[j] = sp.slot[kQuad * Round + j];
  return q;
}

template <int D, int E, bool Scales>
__device__ __forceinline__ uint8_t* head_of(const WriteArgs& a, int32_t slot, int h) {
  return a.pool + static_cast<int64_t>(slot / kBlockSize) * a.page_bytes +
         static_cast<int64_t>(h) * HeadLayout<D, E, Scales>::kBytes;
}
// a head's scale records, from its code block
template <int D, int E, bool Scales>
__device__ __forceinline__ int scales_from_code(const WriteArgs& a, int h) {
  using L = HeadLayout<D, E, Scales>;
  return (a.num_kv_heads - h) * L::kBytes + h * L::kScaleBytes;
}

// Max over each group of LPT lanes (16: DPP rotations inside a 16-lane row;
// 8: swaps inside quads, then the mirror inside each half row; 4: swaps
// inside quads) of unsigned values; VALU only, and every lane of the group
// gets it.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x), Ctrl, 0xF, 0xF, false));
}
template <int LPT>
__device__ __forceinline__ uint32_t group_max(uint32_t x) {
  if constexpr (LPT == 16) {
    x = max(x, dpp<0x128>(x));  // row_ror:8
    x = max(x, dpp<0x124>(x));  // row_ror:4
    x = max(x, dpp<0x122>(x));  // row_ror:2
    return max(x, dpp<0x121>(x));  // row_ror:1
  } else {
    static_assert(LPT == 8 || LPT == 4, "4, 8 or 16 lanes per token");
    x = max(x, dpp<0xB1>(x));   // quad_perm [1, 0, 3, 2]
    x = max(x, dpp<0x4E>(x));   // quad_perm [2, 3, 0, 1]
    if constexpr (LPT == 4) return x;
    return max(x, dpp<0x141>(x));  // row_half_mirror
  }
}

// Largest magnitude of the eight FP16 or BF16 values in w, as the 16-bit
// pattern of |x|: without the sign bit both formats order like unsigned
// integers (a NaN above the infinity, the infinity above every finite
// value), so this is an integer max of packed halves.
__device__ __forceinline__ uint32_t max_magnitude(const u4_t& w) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  auto m = [](uint32_t x) { return __builtin_bit_cast(us2, x & 0x7fff7fffu); };
  const us2 r = __builtin_elementwise_max(__builtin_elementwise_max(m(w[0]), m(w[1])),
                                          __builtin_elementwise_max(m(w[2]), m(w[3])));
  return max(static_cast<uint32_t>(r.x), static_cast<uint32_t>(r.y));
}

// Per-token scale of a row with absolute maximum a (an FP16 or BF16 value):
// the row rule of quant_row.h with a / 127 taken without a division: q0 =
// a * fl(1/127) is within an ulp, and one residual step (the residual is
// exact in an fma) gives fl32(a / 127) for every FP16 and BF16 magnitude
// (checked for all of them). False when the scale is beyond FP16 or a is not
// finite.
__device__ __forceinline__ bool row_scale_token(float a, uint16_t& bits) {
  constexpr float r = 1.0f / 127.0f;
  const float q0 = a * r;
  const float s32 = fmaf(fmaf(-q0, 127.0f, a), r, q0);
  if (!(s32 <= 65504.0f)) return false;
  bits = a == 0.f ? 0x3C00 : round_up_f16(s32);
  return true;
}

// Codes of the eight FP16 or BF16 values in w for a per-token scale s (an
// FP16 value with |x| <= 127 s), equal to clamp(rint(fl32(x / s)), -127, 127)
// but without a division; recip = the hardware reciprocal of s (within one
// ulp). Why these are the same codes:
// * q = x / s is a ratio of two integers of at most 11 bits times a power of
//   two, so fl32(q) is q itself or q lies at least about 2^-36 |q| away from
//   every rounding boundary of fp32; |q| <= 127, so no clamp is needed.
// * q0 = x * recip is within a few ulps of q, so e = x - q0 s is exact in an
//   fma and q0 + e * recip (one more fma) is within about 2^-45 |q| of q:
//   rounded once, it is fl32(q) (one Markstein step).
// * fl32(q) + 1.5 * 2^23 rounds to the nearest integer, ties to even, as
//   rint does; the low byte of its bits is the two's-complement code.
// (Checked against IEEE division for every FP16 and BF16 x and FP16 s, with
// the reciprocal anywhere within one ulp; four VALU instructions per
// element, x entering the two fmas that read it as an FP16 operand.)
template <bool BF16>
__device__ __forceinline__ uint64_t codes_token(const u4_t& w, float s, float recip) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  uint32_t f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = bits16_to_f32<BF16>(static_cast<uint16_t>(w[e / 2] >> (16 * (e % 2))));
    const float q0 = fmaf(x, recip, 0.0f);
    const float q1 = fmaf(fmaf(-q0, s, x), recip, q0);
    f[e] = __float_as_uint(q1 + kMagic);
  }
  // low bytes of f[0..3] and f[4..7] into two words (byte-select 0x0c: zero)
  auto pack = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
  };
  return pack(f[0], f[1], f[2], f[3]) |
         (static_cast<uint64_t>(pack(f[4], f[5], f[6], f[7])) << 32);
}

// Codes of the eight FP16 or BF16 values in w for a static scale s in
// [2^-64, 2^64] and r = fl(1/s), equal to clamp(rint(fl32(x / s)), -127,
// 127) without a division: q0 = x r is within an ulp of x / s, the residual
// x - q0 s is exact in an fma, and q0 + residual * r rounds to fl32(x / s)
// (Markstein's theorem for a correctly rounded reciprocal). q0 is first
// clamped to +-128 (one median of three): inside the range nothing changes,
// beyond it q1 stays at or past +-128 and saturates to +-127 as the division
// does, an infinity (x r infinite, or a finite bf16 x whose x r overflows)
// gives +-127, and a NaN gives -127, the code the division-based rule gives
// it too (the hardware's median of three takes the smaller bound for a quiet
// NaN; the product and the fmas quiet any NaN). The clamped quotient plus
// 1.5 * 2^23 rounds to nearest even, and its low byte is the code. (Checked
// against IEEE division for every FP16 and BF16 x, infinities and NaNs
// included, over scales across the window. FP16 values enter the products
// as mixed-precision operands, without a conversion of their own.)
__host__ __device__ __forceinline__ bool static_window(float s) {
  return s >= 0x1p-64f && s <= 0x1p64f;
}

template <bool BF16>
__device__ __forceinline__ uint64_t codes_static(const u4_t& w, float s, float r) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  uint32_t f[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = bits16_to_f32<BF16>(static_cast<uint16_t>(w[e / 2] >> (16 * (e % 2))));
    const float q0 = __builtin_amdgcn_fmed3f(fmaf(x, r, 0.0f), -128.0f, 128.0f);
    const float q1 = fmaf(fmaf(-q0, s, x), r, q0);
    f[e] = __float_as_uint(__builtin_amdgcn_fmed3f(q1, -127.0f, 127.0f) + kMagic);
  }
  auto pack = [](uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
  };
  return pack(f[0], f[1], f[2], f[3]) |
         (static_cast<uint64_t>(pack(f[4], f[5], f[6], f[7])) << 32);
}

// kInt8StaticDiv: static scales outside the division-free window (one IEEE
// division per element), a kernel of its own so that the window's kernel
// carries no division code
enum WriteFormat { kInt8Sym = 0, kInt8Static = 1, kBits16 = 2, kInt8StaticDiv = 3 };

// Spans per wave of a large call (measured on 262K- and 296K-token
// prefills): with 8 elements per lane the INT8 writers gain 5-8% from three
// spans' loads in flight at D = 128 (two at D = 64, where more registers
// cost occupancy). With 16 elements per lane both INT8 writers are fastest
// with one span (eight waves per SIMD; 296K-token prefill: per-token 361 us
// against 384 us with two and 390 with three, static scales 373-376 us
// against 407 us with two); the 16-bit writer, already near the copy rate,
// is 10% slower with more than one. A call of fewer than kManySpanWaves
// one-span waves (a decode step's append) keeps one span per wave: its time
// is one wave's latency, which more spans per wave lengthen (64 tokens: 6 us
// with one span, 10 us with three). (A persistent form, each wave looping
// over items with the next item's slots and rows in flight, measured 12-30%
// slower.)
constexpr int spans_per_wave(int D, int F, int epl) {
  return F == kBits16 || epl == 16 ? 1 : D == 128 && epl == 8 ? 3 : 2;
}
constexpr int64_t kManySpanWaves = 2048;

// Elements of a row each lane holds: 16 for the INT8 formats when the KV
// heads fill whole waves at that width (twice the row work per lane, so the
// per-row scale, address and store instructions are shared by twice the
// bytes: the INT8 writers are instruction-bound), else 8.
constexpr int kWideEpl = 16;
constexpr int heads_per_wave(int D, int epl) { return 16 * epl / D; }

// A lane's EPL raw 16-bit K and V elements, as EPL / 8 vectors of eight.
template <int EPL>
struct Rows {
  u4_t k[EPL / 8], v[EPL / 8];
};

// Loads of the rows of up to four consecutive tokens t0 .. t0 + nt - 1
// (nt >= 1): lane (head hh, token r, i) gets elements EPL*i .. EPL*i + EPL-1
// of token r's rows of KV head h0 + hh; past the call's end the last token,
// and past the last head the last head, are loaded again.
// (QPW = 2: the wave's lane groups of HPW / 2 heads each take one of two
// quads, q and t0 being those of the lane's quad)
template <int D, int EPL, bool Vec, int QPW = 1>
__device__ __forceinline__ Rows<EPL> load_rows(const WriteArgs& a, const Quad& q, int64_t t0,
                                               int h0, int lane) {
  constexpr int NV = EPL / 8, LPT = D / EPL, LPH = kQuad * LPT;
  constexpr int HQ = heads_per_wave(D, EPL) / QPW;  // heads per quad
  const int hh = lane / LPH % HQ, r = lane % LPH / LPT, i = lane % LPT;
  const int h = h0 + hh;
  const int hl = h < a.num_kv_heads ? h : a.num_kv_heads - 1;
  const int64_t t = t0 + (r < q.nt ? r : q.nt - 1);
  const uint16_t* kr = static_cast<const uint16_t*>(a.k) + t * a.k_st + hl * a.k_sh;
  const uint16_t* vr = static_cast<const uint16_t*>(a.v) + t * a.v_st + hl * a.v_sh;
  Rows<EPL> in;
  if constexpr (Vec) {
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      in.k[c] = *reinterpret_cast<const u4_t*>(kr + EPL * i + 8 * c);
      in.v[c] = *reinterpret_cast<const u4_t*>(vr + EPL * i + 8 * c);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      uint32_t kw[4] = {}, vw[4] = {};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t d = EPL * i + 8 * c + e;
        kw[e / 2] |= static_cast<uint32_t>(kr[d * a.k_sd]) << (16 * (e % 2));
        vw[e / 2] |= static_cast<uint32_t>(vr[d * a.v_sd]) << (16 * (e % 2));
      }
      in.k[c] = u4_t{kw[0], kw[1], kw[2], kw[3]};
      in.v[c] = u4_t{vw[0], vw[1], vw[2], vw[3]};
    }
  }
  return in;
}

// Codes of eight FP16 or BF16 values with a static scale outside the
// division-free window: one IEEE division per element.
template <bool BF16>
__device__ __forceinline__ uint64_t codes_static_div(const u4_t& w, float s) {
  uint64_t c = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    c |= static_cast<uint64_t>(
             row_code(bits16_to_f32<BF16>(static_cast<uint16_t>(w[e / 2] >> (16 * (e % 2)))), s))
         << (8 * e);
  return c;
}

// Write of the K and V rows (loaded by load_rows) of up to four consecutive
// tokens of the call, for HPW = 16 * EPL / D KV heads at once: quantize-on-
// write into INT8 pages (kInt8Sym: per-token scales; kInt8Static: the
// layer's scales) or a plain copy into 16-bit pages (kBits16). Every lane
// holds EPL elements of one row: lane (head hh, token r, i) holds elements
// EPL*i .. EPL*i + EPL-1 of token r's rows of KV head h0 + hh (LPT = D / EPL
// lanes per token), so a row's absolute maximum is an LPT-lane reduction and
// the per-row scale work of all the wave's rows shares instructions. The
// per-row rules (MoE-Infinity PR #183 "feat: opt-in INT8 KV-cache
// quantization", "What landed", format-contract bullet; zero rows per mlxcel
// PR #717 "The Int8 bug and fix"; static scales per InfiniLM PR #553
// "Summary"):
//   per-token: a = max|x|; s = 1.0 if a == 0 else the smallest FP16 >=
//   fl32(a/127); code = clamp(rint(fl32(x / s)), -127, 127);
//   static: code = clamp(rint(fl32(x / scale)), -127, 127).
// A token with a negative slot is padding (skipped); an out-of-range slot, a
// per-token scale beyond FP16 or a NaN or infinity in a row (per-token
// format) is flagged and that (token, head) is left unwritten. K rows are
// stored per token (EPL contiguous elements per lane). When the four tokens
// are one whole V group of a head, the elements go through LDS to become
// group words (one dimension of the four tokens) and every lane stores
// EPL / 4 whole words; otherwise each token's V elements are stored one by
// one.
// QPW = 2: two quads at once, the lane groups of the first HPW / 2 heads on
// q's first quad and the others on its second (q is the lane's own quad).
template <int D, int EPL, int F, bool BF16, int QPW = 1>
__device__ __forceinline__ void write_quad(const WriteArgs& a, const Quad& q,
                                           const Rows<EPL>& in, int h0, u4_t* s_elems,
                                           int lane) {
  constexpr int NV = EPL / 8;       // vectors of eight elements per lane
  constexpr int LPT = D / EPL;      // lanes per token row
  constexpr int LPH = kQuad * LPT;  // lanes per head
  constexpr int HQ = heads_per_wave(D, EPL) / QPW;  // heads per quad
  constexpr int E = F == kBits16 ? 2 : 1;  // bytes per stored element
  constexpr bool Scales = F == kInt8Sym;
  static_assert(NV * 8 * E <= 16, "a lane's V elements fit its 16 LDS bytes");
  using L = HeadLayout<D, E, Scales>;
  using Packed = typename std::conditional<E == 2, u4_t, uint64_t>::type;  // eight elements
  const int hg = lane / LPH;  // the lane group of one head and one quad
  const int hh = hg % HQ, r = lane % LPH / LPT, i = lane % LPT;
  const int h = h0 + hh;
  const bool hvalid = h < a.num_kv_heads;
  const int32_t my_slot = r == 0 ? q.slot[0] : r == 1 ? q.slot[1] : r == 2 ? q.slot[2] : q.slot[3];

  bool ok = my_slot >= 0 && hvalid;
  Packed kc[NV], vc[NV];
  uint16_t skb = 0, svb = 0;
  if constexpr (F == kBits16) {
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      kc[c] = in.k[c];
      vc[c] = in.v[c];
    }
  } else if constexpr (F == kInt8Sym) {
    // row maxima as magnitude bits, reduced over the row's lanes (a NaN
    // stays the largest and is flagged with the scale)
    uint32_t mk = max_magnitude(in.k[0]), mv = max_magnitude(in.v[0]);
#pragma unroll
    for (int c = 1; c < NV; ++c) {
      mk = max(mk, max_magnitude(in.k[c]));
      mv = max(mv, max_magnitude(in.v[c]));
    }
    const float ak = bits16_to_f32<BF16>(static_cast<uint16_t>(group_max<LPT>(mk)));
    const float av = bits16_to_f32<BF16>(static_cast<uint16_t>(group_max<LPT>(mv)));
    const bool okk = row_scale_token(ak, skb), okv = row_scale_token(av, svb);
    if (ok && !(okk && okv)) {
      if (i == 0) raise_flag(a.err, PDAKV_EFLAG_SCALE_RANGE);
      ok = false;
    }
    const float sk = f16_bits_to_f32(skb), sv = f16_bits_to_f32(svb);
    const float rk = __builtin_amdgcn_rcpf(sk), rv = __builtin_amdgcn_rcpf(sv);
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      kc[c] = codes_token<BF16>(in.k[c], sk, rk);
      vc[c] = codes_token<BF16>(in.v[c], sv, rv);
    }
  } else if constexpr (F == kInt8Static) {
    // (scales inside [2^-64, 2^64]; the reciprocals are fl(1/s), from the host)
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      kc[c] = codes_static<BF16>(in.k[c], a.k_scale, a.k_rcp);
      vc[c] = codes_static<BF16>(in.v[c], a.v_scale, a.v_rcp);
    }
  } else {
    // scales outside [2^-64, 2^64]: one IEEE division per element
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      kc[c] = codes_static_div<BF16>(in.k[c], a.k_scale);
      vc[c] = codes_static_div<BF16>(in.v[c], a.v_scale);
    }
  }
  // whole V group of this lane's head: all four tokens stored (uniform over
  // the head's lanes)
  const uint64_t stored = __ballot(ok);
  const uint64_t head_lanes = LPH == 64 ? ~0ull : ((1ull << LPH) - 1) << (LPH * hg);
  const bool whole = q.nt == kQuad && (stored & head_lanes) == head_lanes &&
                     q.slot[0] % 4 == 0 && q.slot[1] == q.slot[0] + 1 &&
                     q.slot[2] == q.slot[0] + 2 && q.slot[3] == q.slot[0] + 3;
  const int pos = my_slot % kBlockSize;
  uint8_t* head = head_of<D, E, Scales>(a, ok ? my_slot : 0, ok ? h : 0);
  if (ok) {
    uint8_t* krow = head + (pos * D + EPL * i) * E;
    if constexpr (E == 1 && NV == 2) {
      *reinterpret_cast<u4_t*>(krow) =
          u4_t{static_cast<uint32_t>(kc[0]), static_cast<uint32_t>(kc[0] >> 32),
               static_cast<uint32_t>(kc[1]), static_cast<uint32_t>(kc[1] >> 32)};
    } else {
#pragma unroll
      for (int c = 0; c < NV; ++c) *reinterpret_cast<Packed*>(krow + 8 * c * E) = kc[c];
    }
    if constexpr (Scales) {
      if (i == 0) {
        uint8_t* rec = head + scales_from_code<D, E, Scales>(a, h) + L::ks_off(pos);
        *reinterpret_cast<uint16_t*>(rec) = skb;
        *reinterpret_cast<uint16_t*>(rec + 8) = svb;
      }
    }
  }
  // (every lane passes the LDS exchange, so that the wave stays together;
  // the barrier keeps this store after the reads of an earlier span)
  __builtin_amdgcn_wave_barrier();
  if constexpr (E == 1 && NV == 2) {
    s_elems[lane] = u4_t{static_cast<uint32_t>(vc[0]), static_cast<uint32_t>(vc[0] >> 32),
                         static_cast<uint32_t>(vc[1]), static_cast<uint32_t>(vc[1] >> 32)};
  } else {
    *reinterpret_cast<Packed*>(&s_elems[lane]) = vc[0];
  }
  __builtin_amdgcn_wave_barrier();
  if (whole) {
    // lane (hh, r, i) builds the group words of EPL / 4 dimensions of its
    // head (one element of each token per word): it reads from each token's
    // lane (hh, j, i) the word that holds those dimensions' elements and
    // gathers them with byte selects
    const uint32_t* ew = reinterpret_cast<const uint32_t*>(s_elems + LPH * hg + i);
    uint32_t d[kQuad];
    if constexpr (E == 1 && NV == 2) {
      // dims 16i + 4r .. 16i + 4r + 3: word r of each token's 16 codes; a
      // 4 x 4 byte transpose turns the four words into four group words
#pragma unroll
      for (int j = 0; j < kQuad; ++j) d[j] = ew[4 * LPT * j + r];
      const uint32_t t01l = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u);  // d0.0 d1.0 d0.1 d1.1
      const uint32_t t01h = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u);  // d0.2 d1.2 d0.3 d1.3
      const uint32_t t23l = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
      const uint32_t t23h = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
      uint8_t* vg = head + L::kV + (pos / 4) * 4 * D + 4 * (EPL * i + 4 * r);
      *reinterpret_cast<u4_t*>(vg) = u4_t{__builtin_amdgcn_perm(t23l, t01l, 0x05040100u),
                                          __builtin_amdgcn_perm(t23l, t01l, 0x07060302u),
                                          __builtin_amdgcn_perm(t23h, t01h, 0x05040100u),
                                          __builtin_amdgcn_perm(t23h, t01h, 0x07060302u)};
    } else {
      // dims 8i + 2r and 8i + 2r + 1
#pragma unroll
      for (int j = 0; j < kQuad; ++j) d[j] = ew[4 * LPT * j + (E == 2 ? r : r >> 1)];
      uint8_t* vg = head + L::kV + ((pos / 4) * 4 * D + 4 * (EPL * i + 2 * r)) * E;
      if constexpr (E == 2) {
        // word j holds elements 2r (low half) and 2r + 1 (high half) of token j
        *reinterpret_cast<u4_t*>(vg) = u4_t{__builtin_amdgcn_perm(d[1], d[0], 0x05040100u),
                                            __builtin_amdgcn_perm(d[3], d[2], 0x05040100u),
                                            __builtin_amdgcn_perm(d[1], d[0], 0x07060302u),
                                            __builtin_amdgcn_perm(d[3], d[2], 0x07060302u)};
      } else {
        // elements 2r and 2r + 1 are bytes b and b + 1 of word j
        const uint32_t b = 2 * (r & 1);
        const uint32_t sel = b | (b + 4) << 8 | (b + 1) << 16 | (b + 5) << 24;
        const uint32_t t01 = __builtin_amdgcn_perm(d[1], d[0], sel);  // d0.b d1.b d0.b+1 d1.b+1
        const uint32_t t23 = __builtin_amdgcn_perm(d[3], d[2], sel);
        *reinterpret_cast<uint64_t*>(vg) =
            __builtin_amdgcn_perm(t23, t01, 0x05040100u) |
            static_cast<uint64_t>(__builtin_amdgcn_perm(t23, t01, 0x07060302u)) << 32;
      }
    }
  } else if (ok) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      uint8_t* dst = head + L::kV + ((pos / 4) * 4 * D + 4 * (EPL * i + e) + pos % 4) * E;
      const int c = e / 8, ee = e % 8;
      if constexpr (E == 2)
        *reinterpret_cast<uint16_t*>(dst) =
            static_cast<uint16_t>(vc[c][ee / 2] >> (16 * (ee % 2)));
      else
        *dst = static_cast<uint8_t>(vc[c] >> (8 * ee));
    }
  }
}

// One wave per kSpans spans of about four tokens (boundaries moved to V
// groups) and 16 * EPL / D KV heads. The rows of all its spans are loaded
// before the first is quantized and stored, so a wave keeps kSpans times the
// bytes in flight; a span across two runs of slots takes a second round.
// QPW = 2 (two quads per wave, kSpans = 2): the wave's first HPW / 2 heads'
// lane groups take span 0 and the others span 1, side by side in one round,
// so that the 16-element form serves a head count that fills only half a
// wave (two KV heads at D = 64, an odd count at D = 128).
template <int D, int F, bool BF16, bool Vec, int kSpans, int EPL, int QPW = 1>
__global__ __launch_bounds__(64 * kWriteWaves) void write_kernel(WriteArgs a) {
  constexpr int HPW = heads_per_wave(D, EPL) / QPW;  // KV heads per wave
  static_assert(QPW == 1 || kSpans == 2, "two quads: the wave's two spans side by side");
  __shared__ u4_t s_elems[kWriteWaves][64];  // a lane's V elements
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (wave-uniform, so the slots are scalar loads)
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWriteWaves + wv;
  const int64_t quads = (a.num_tokens + kQuad - 1) / kQuad;
  const int64_t groups = (quads + kSpans - 1) / kSpans;
  const int hgroups = (a.num_kv_heads + HPW - 1) / HPW;
  if (w >= groups * hgroups) return;
  const int64_t g = w / hgroups;
  const int h0 = static_cast<int>(w - g * hgroups) * HPW;
  Span sp[kSpans];
  load_spans<kSpans>(a, g * kSpans, lane, sp);
  if constexpr (QPW == 2) {
    constexpr int LPH = kQuad * D / EPL;
    const bool second = lane >= LPH * HPW;  // the lane's quad: span 1
    // a quad with nothing to store for the lane: span 0's tokens (valid
    // rows to load), no slots
    auto idle = [](Quad q) {
#pragma unroll
      for (int j = 0; j < kQuad; ++j) q.slot[j] = -1;
      return q;
    };
    auto pick = [&](const Quad& q0, int64_t t0, const Quad& q1, int64_t t1, Quad& q,
                    int64_t& t) {
      t = second ? t1 : t0;
      q.nt = second ? q1.nt : q0.nt;
#pragma unroll
      for (int j = 0; j < kQuad; ++j) q.slot[j] = second ? q1.slot[j] : q0.slot[j];
    };
    const Quad a0 = quad_of<0>(sp[0]);
    const bool has1 = sp[1].n > 0;
    Quad q;
    int64_t t;
    pick(a0, sp[0].t0, has1 ? quad_of<0>(sp[1]) : idle(a0), has1 ? sp[1].t0 : sp[0].t0, q, t);
    const Rows<EPL> in = load_rows<D, EPL, Vec, 2>(a, q, t, h0, lane);
    write_quad<D, EPL, F, BF16, 2>(a, q, in, h0, s_elems[wv], lane);
    const bool more0 = sp[0].n > kQuad, more1 = sp[1].n > kQuad;
    if (more0 || more1) {  // a span across two runs of slots: its second round
      pick(more0 ? quad_of<1>(sp[0]) : idle(a0), more0 ? sp[0].t0 + kQuad : sp[0].t0,
           more1 ? quad_of<1>(sp[1]) : idle(a0), more1 ? sp[1].t0 + kQuad : sp[0].t0, q, t);
      const Rows<EPL> in1 = load_rows<D, EPL, Vec, 2>(a, q, t, h0, lane);
      write_quad<D, EPL, F, BF16, 2>(a, q, in1, h0, s_elems[wv], lane);
    }
    return;
  }
  Rows<EPL> in[kSpans];
#pragma unroll
  for (int p = 0; p < kSpans; ++p)
    if (sp[p].n > 0) in[p] = load_rows<D, EPL, Vec>(a, quad_of<0>(sp[p]), sp[p].t0, h0, lane);
#pragma unroll
  for (int p = 0; p < kSpans; ++p)
    if (sp[p].n > 0)
      write_quad<D, EPL, F, BF16>(a, quad_of<0>(sp[p]), in[p], h0, s_elems[wv], lane);
#pragma unroll
  for (int p = 0; p < kSpans; ++p)
    if (sp[p].n > kQuad) {  // a span across two runs of slots
      const Quad q = quad_of<1>(sp[p]);
      const Rows<EPL> in1 = load_rows<D, EPL, Vec>(a, q, sp[p].t0 + kQuad, h0, lane);
      write_quad<D, EPL, F, BF16>(a, q, in1, h0, s_elems[wv], lane);
    }
}

// Waves of a call at `spans` spans per wave and `epl` elements per lane
// (qpw = 2: the two spans side by side, half the heads per wave).
int64_t write_waves(const WriteArgs& a, int head_dim, int spans, int epl, int qpw = 1) {
  const int hpw = heads_per_wave(head_dim, epl) / qpw;
  const int64_t quads = (a.num_tokens + kQuad - 1) / kQuad;
  return (quads + spans - 1) / spans * ((a.num_kv_heads + hpw - 1) / hpw);
}

// Whole-row vector loads: unit element stride, every row start aligned to
// `bytes`
bool vec_rows(const WriteArgs& a, int bytes) {
  const int64_t el = bytes / 2;
  auto al = [el](int64_t x) { return x % el == 0; };
  return a.k_sd == 1 && a.v_sd == 1 && al(a.k_st) && al(a.k_sh) && al(a.v_st) && al(a.v_sh) &&
         (reinterpret_cast<uintptr_t>(a.k) % bytes) == 0 &&
         (reinterpret_cast<uintptr_t>(a.v) % bytes) == 0;
}

template <int D, int F, bool BF16, int S, int EPL, int QPW = 1>
hipError_t launch_spans(const WriteArgs& a, hipStream_t s) {
  const int64_t waves = write_waves(a, D, S, EPL, QPW);
  const dim3 grid(static_cast<unsigned>((waves + kWriteWaves - 1) / kWriteWaves)),
      block(64 * kWriteWaves);
  // lanes load 16 bytes of a row
  if (vec_rows(a, 16))
    hipLaunchKernelGGL((write_kernel<D, F, BF16, true, S, EPL, QPW>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((write_kernel<D, F, BF16, false, S, EPL, QPW>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D, int F, bool BF16, int EPL>
hipError_t launch_epl(const WriteArgs& a, hipStream_t s) {
  constexpr int S = spans_per_wave(D, F, EPL);
  if (S > 1 && write_waves(a, D, 1, EPL) >= kManySpanWaves)
    return launch_spans<D, F, BF16, S, EPL>(a, s);
  return launch_spans<D, F, BF16, 1, EPL>(a, s);
}

template <int D, int F, bool BF16>
hipError_t launch_dim(const WriteArgs& a, hipStream_t s) {
  if constexpr (F != kBits16) {
    constexpr int hpw = heads_per_wave(D, kWideEpl);
    if (a.num_kv_heads % hpw == 0) return launch_epl<D, F, BF16, kWideEpl>(a, s);
    // heads that fill half a wave: two quads per wave
    if (a.num_kv_heads % (hpw / 2) == 0) return launch_spans<D, F, BF16, 2, kWideEpl, 2>(a, s);
  }
  return launch_epl<D, F, BF16, 8>(a, s);
}

template <int F, bool BF16>
hipError_t launch_format(const WriteArgs& a, int head_dim, hipStream_t s) {
  return head_dim == 128 ? launch_dim<128, F, BF16>(a, s) : launch_dim<64, F, BF16>(a, s);
}

}  // namespace

hipError_t launch_quant_write_int8(const WriteArgs& a, int head_dim, bool src_bf16,
                                   hipStream_t s) {
  return src_bf16 ? launch_format<kInt8Sym, true>(a, head_dim, s)
                  : launch_format<kInt8Sym, false>(a, head_dim, s);
}

hipError_t launch_quant_write_static(const WriteArgs& a, int head_dim, bool src_bf16,
                                     hipStream_t s) {
  if (static_window(a.k_scale) && static_window(a.v_scale))
    return src_bf16 ? launch_format<kInt8Static, true>(a, head_dim, s)
                    : launch_format<kInt8Static, false>(a, head_dim, s);
  return src_bf16 ? launch_format<kInt8StaticDiv, true>(a, head_dim, s)
                  : launch_format<kInt8StaticDiv, false>(a, head_dim, s);
}

hipError_t launch_write_16bit(const WriteArgs& a, int head_dim, hipStream_t s) {
  return launch_format<kBits16, false>(a, head_dim, s);
}

}  // namespace pdakv
