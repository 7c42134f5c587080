// Page lifecycle operations on the paged KV pools (gfx950).
//
// * Page copies for swap-out / swap-in (MoE-Infinity PR #183 "feat: opt-in
//   INT8 KV-cache quantization", "What landed", serving-lifecycle bullet:
//   pages leave the GPU and come back with their INT8 scales). A token's
//   scales live in its page, so whole-page copies move codes and scales
//   together. One workgroup per page, 16-byte vector copies; the far side
//   may be device memory or pinned host memory.
// * Front trim that keeps sink tokens (mlxcel PR #717 and its follow-up on
//   the same page: drop the n tokens after the first `keep` positions, the
//   INT8 scales moving with their tokens). Every later token moves n
//   positions toward the front through the sequence's own block table. One
//   workgroup per (sequence, KV head) moves the tokens in rounds of 128 in
//   increasing position order, each round read completely (K rows as
//   16-byte vectors, V as words holding a dimension of four tokens) into
//   LDS before any of it is written: a round's destinations lie below its
//   sources and below every later round's sources, so no token is
//   overwritten before it has been read.
#include "device_util.h"
#include "launch.h"

namespace pdakv {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte vectors in flight per thread

__global__ __launch_bounds__(kCopyThreads) void page_copy_kernel(PageCopyArgs a) {
  const int64_t i = blockIdx.x;
  const int32_t id = a.ids[i];
  if (id < 0 || id >= a.num_blocks) {
    if (threadIdx.x == 0) raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    return;
  }
  const int64_t pb = a.page_bytes;
  const uint8_t* src = a.gather ? a.pool + id * pb : a.packed + i * pb;
  uint8_t* dst = a.gather ? a.packed + i * pb : a.pool + id * pb;
  const int64_t nvec = pb / 16;
  for (int64_t v0 = threadIdx.x; v0 < nvec; v0 += kCopyThreads * kCopyUnroll) {
    u4_t w[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t v = v0 + u * kCopyThreads;
      if (v < nvec) w[u] = reinterpret_cast<const u4_t*>(src)[v];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t v = v0 + u * kCopyThreads;
      if (v < nvec) reinterpret_cast<u4_t*>(dst)[v] = w[u];
    }
  }
}

constexpr int kTrimThreads = 256;
// tokens moved per round (a multiple of 4); rounds of 512 were measured no
// faster, and the smaller LDS footprint lets several workgroups share a CU
template <int E>
constexpr int trim_chunk() {
  return 128;
}

// Token layout of a head block: element size E (1: INT8 codes, 2: 16-bit
// values), K row of D elements at pos * D, V grouped four tokens at a time
// (element d of token pos at 16 * D + (pos / 4) * 4 * D + 4 * d + pos % 4,
// so one "V word" of 4 * E bytes holds dimension d of a whole group), and
// for per-token INT8 the fp16 K and V scales after the codes.
template <int D, int E, bool Scales>
struct TokenLayout {
  static constexpr int kHeadBytes = 32 * D * E + (Scales ? 64 : 0);
  static constexpr int kRowBytes = D * E;
  static __device__ __forceinline__ int k_off(int pos) { return pos * D * E; }
  static __device__ __forceinline__ int vword_off(int group, int d) {  // group of the page
    return (16 * D + group * 4 * D + 4 * d) * E;
  }
  static __device__ __forceinline__ int ks_off(int pos) { return 32 * D + 2 * pos; }
  static __device__ __forceinline__ int vs_off(int pos) { return 32 * D + 32 + 2 * pos; }
};

template <int E>
struct Elem;
template <>
struct Elem<1> {
  using T = uint8_t;   // one element
  using W = uint32_t;  // one V word (4 elements)
};
template <>
struct Elem<2> {
  using T = uint16_t;
  using W = uint64_t;
};

template <int D, int E, bool Scales>
__global__ __launch_bounds__(kTrimThreads) void trim_keep_sink_kernel(TrimArgs a) {
  using Lay = TokenLayout<D, E, Scales>;
  using T = typename Elem<E>::T;
  using W = typename Elem<E>::W;
  constexpr int C = trim_chunk<E>();
  constexpr int KV = Lay::kRowBytes / 16;  // 16-byte vectors per K row
  constexpr int KPT = (C * KV + kTrimThreads - 1) / kTrimThreads;  // K vectors per thread
  constexpr int VG = C / 4 + 1;  // source groups a round touches
  constexpr int VPT = (VG * D + kTrimThreads - 1) / kTrimThreads;  // V words per thread
  constexpr int TPT = (C + kTrimThreads - 1) / kTrimThreads;        // tokens per thread
  __shared__ u4_t s_k[C][KV];
  __shared__ T s_v[C][D];
  __shared__ uint32_t s_sc[C];        // K scale | V scale << 16
  // head-block index of each token's source page (-1: missing) and of its
  // destination page (-1: missing, or the token is not moved)
  __shared__ int s_src[C], s_dst[C];

  const int b = blockIdx.x / a.num_kv_heads, g = blockIdx.x % a.num_kv_heads;
  const int tid = threadIdx.x;
  int L = a.ctx[b];
  const int64_t cap = a.bt_stride * kBlockSize;
  if (L < 0 || L > cap) {
    if (tid == 0 && g == 0) raise_flag(a.err, PDAKV_EFLAG_CONTEXT_RANGE);
    L = L < 0 ? 0 : static_cast<int>(cap);
  }
  const int room = L > a.keep ? L - a.keep : 0;
  int n = a.trim[b];
  n = n < 0 ? 0 : (n > room ? room : n);
  if (g == 0 && tid == 0) a.new_ctx[b] = L - n;
  const int count = L - a.keep - n;  // tokens that move
  if (n == 0 || count <= 0) return;
  const int32_t* row = a.bt + static_cast<int64_t>(b) * a.bt_stride;
  auto head = [&](int hb) { return a.pool + static_cast<int64_t>(hb) * Lay::kHeadBytes; };

  for (int c0 = 0; c0 < count; c0 += C) {
    const int m = min(C, count - c0);
    const int s0 = a.keep + n + c0;  // first source position of the round
    const int q0 = a.keep + c0;      // its destination
    for (int i = tid; i < m; i += kTrimThreads) {
      const int32_t bs = row[(s0 + i) / kBlockSize], bd = row[(q0 + i) / kBlockSize];
      const bool src_ok = bs >= 0 && bs < a.num_blocks;
      const bool dst_ok = bd >= 0 && bd < a.num_blocks;
      if (!src_ok || !dst_ok) raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
      // the four tokens of a source group share its page, so they share
      // src_ok: a group's V word is read whenever one of them is moved
      s_src[i] = src_ok ? bs * a.num_kv_heads + g : -1;
      s_dst[i] = src_ok && dst_ok ? bd * a.num_kv_heads + g : -1;
    }
    __syncthreads();

    // read the round: every load is issued before any is used
    u4_t kreg[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int e = tid + r * kTrimThreads;
      const int i = e / KV, c = e % KV;
      if (e < m * KV && s_src[i] >= 0) {
        const uint8_t* h = head(s_src[i]) + Lay::k_off((s0 + i) % kBlockSize);
        kreg[r] = reinterpret_cast<const u4_t*>(h)[c];
      }
    }
    const int gfirst = s0 / 4, ngroups = (s0 + m - 1) / 4 - gfirst + 1;
    W vreg[VPT];
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int e = tid + r * kTrimThreads;
      const int gi = e / D, d = e % D;
      const int p = max(4 * (gfirst + gi), s0);  // an in-round token of the group
      if (e < ngroups * D && s_src[p - s0] >= 0)
        vreg[r] = *reinterpret_cast<const W*>(head(s_src[p - s0]) +
                                              Lay::vword_off((p % kBlockSize) / 4, d));
    }
    uint32_t sc[TPT];
    if constexpr (Scales) {
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        const int i = tid + r * kTrimThreads;
        if (i < m && s_src[i] >= 0) {
          const int pos = (s0 + i) % kBlockSize;
          const uint8_t* h = head(s_src[i]);
          sc[r] = *reinterpret_cast<const uint16_t*>(h + Lay::ks_off(pos)) |
                  (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(h + Lay::vs_off(pos)))
                   << 16);
        }
      }
    }
    // into LDS, token-major
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int e = tid + r * kTrimThreads;
      if (e < m * KV) s_k[e / KV][e % KV] = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int e = tid + r * kTrimThreads;
      if (e >= ngroups * D) continue;
      const int gi = e / D, d = e % D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = 4 * (gfirst + gi) + j;
        if (p >= s0 && p < s0 + m) s_v[p - s0][d] = static_cast<T>(vreg[r] >> (8 * E * j));
      }
    }
    if constexpr (Scales) {
#pragma unroll
      for (int r = 0; r < TPT; ++r) {
        const int i = tid + r * kTrimThreads;
        if (i < m) s_sc[i] = sc[r];
      }
    }
    __syncthreads();

    // write the round n positions further to the front: whole V words where
    // all four tokens of the destination group move in this round, single
    // elements at the edges (the other tokens of such a word are a sink
    // token, a token of the next round, or past the new length)
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int e = tid + r * kTrimThreads;
      const int i = e / KV, c = e % KV;
      if (e < m * KV && s_dst[i] >= 0) {
        uint8_t* h = head(s_dst[i]) + Lay::k_off((q0 + i) % kBlockSize);
        reinterpret_cast<u4_t*>(h)[c] = s_k[i][c];
      }
    }
    const int hfirst = q0 / 4, nhead = (q0 + m - 1) / 4 - hfirst + 1;
    for (int e = tid; e < nhead * D; e += kTrimThreads) {
      const int gi = e / D, d = e % D;
      const int p0 = 4 * (hfirst + gi);  // first destination position of the group
      bool whole = p0 >= q0 && p0 + 3 < q0 + m;
      if (whole) {
#pragma unroll
        for (int j = 0; j < 4; ++j) whole = whole && s_dst[p0 + j - q0] >= 0;
      }
      if (whole) {
        W w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w |= static_cast<W>(s_v[p0 + j - q0][d]) << (8 * E * j);
        uint8_t* h = head(s_dst[p0 - q0]) + Lay::vword_off((p0 % kBlockSize) / 4, d);
        *reinterpret_cast<W*>(h) = w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = p0 + j;
          if (p < q0 || p >= q0 + m || s_dst[p - q0] < 0) continue;
          *reinterpret_cast<T*>(head(s_dst[p - q0]) +
                                Lay::vword_off((p % kBlockSize) / 4, d) + j * E) = s_v[p - q0][d];
        }
      }
    }
    if constexpr (Scales) {
      for (int i = tid; i < m; i += kTrimThreads) {
        if (s_dst[i] < 0) continue;
        const int pos = (q0 + i) % kBlockSize;
        uint8_t* h = head(s_dst[i]);
        *reinterpret_cast<uint16_t*>(h + Lay::ks_off(pos)) = static_cast<uint16_t>(s_sc[i]);
        *reinterpret_cast<uint16_t*>(h + Lay::vs_off(pos)) = static_cast<uint16_t>(s_sc[i] >> 16);
      }
    }
    __syncthreads();  // the next round reuses the LDS
  }
}

}  // namespace

hipError_t launch_page_copy(const PageCopyArgs& a, hipStream_t s) {
  if (a.num_pages == 0) return hipSuccess;
  hipLaunchKernelGGL(page_copy_kernel, dim3(static_cast<unsigned>(a.num_pages)),
                     dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_trim_keep_sink(const TrimArgs& a, int kv_format, int head_dim, hipStream_t s) {
  using Kern = void (*)(TrimArgs);
  Kern k;
  if (kv_format == PDAKV_KV_INT8_SYM)
    k = head_dim == 128 ? trim_keep_sink_kernel<128, 1, true> : trim_keep_sink_kernel<64, 1, true>;
  else if (kv_format == PDAKV_KV_INT8_STATIC)
    k = head_dim == 128 ? trim_keep_sink_kernel<128, 1, false>
                        : trim_keep_sink_kernel<64, 1, false>;
  else
    k = head_dim == 128 ? trim_keep_sink_kernel<128, 2, false>
                        : trim_keep_sink_kernel<64, 2, false>;
  hipLaunchKernelGGL(k, dim3(a.num_seqs * a.num_kv_heads), dim3(kTrimThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pdakv
