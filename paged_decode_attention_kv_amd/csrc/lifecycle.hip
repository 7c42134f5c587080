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
//   workgroup per (sequence, KV head) moves the tokens in chunks in
//   increasing position order, each chunk read completely into LDS before
//   any of it is written: a chunk's destinations lie below its sources and
//   below every later chunk's sources, so no token is overwritten before it
//   has been read.
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
constexpr int kTrimChunk = 64;  // tokens moved per round

// Token layout of a head block: element size E (1: INT8 codes, 2: 16-bit
// values), K row of D elements at pos * D, V element d of token pos at
// 16 * D + (pos / 4) * 4 * D + 4 * d + pos % 4 (in elements), and for
// per-token INT8 the K and V scales (fp16) after the codes.
template <int D, int E, bool Scales>
struct TokenLayout {
  static constexpr int kHeadBytes = 32 * D * E + (Scales ? 64 : 0);
  static constexpr int kRowBytes = D * E;
  static __device__ __forceinline__ int k_off(int pos) { return pos * D * E; }
  static __device__ __forceinline__ int v_off(int pos, int d) {
    return (16 * D + (pos >> 2) * 4 * D + 4 * d + (pos & 3)) * E;
  }
  static __device__ __forceinline__ int ks_off(int pos) { return 32 * D + 2 * pos; }
  static __device__ __forceinline__ int vs_off(int pos) { return 32 * D + 32 + 2 * pos; }
};

template <int E>
struct Elem;
template <>
struct Elem<1> {
  using T = uint8_t;
};
template <>
struct Elem<2> {
  using T = uint16_t;
};

template <int D, int E, bool Scales>
__global__ __launch_bounds__(kTrimThreads) void trim_keep_sink_kernel(TrimArgs a) {
  using Lay = TokenLayout<D, E, Scales>;
  using T = typename Elem<E>::T;
  constexpr int KV = Lay::kRowBytes / 16;  // 16-byte vectors per K row
  __shared__ u4_t s_k[kTrimChunk][KV];
  __shared__ T s_v[kTrimChunk][D];
  __shared__ uint32_t s_sc[kTrimChunk];  // K scale | V scale << 16
  __shared__ int s_src[kTrimChunk], s_dst[kTrimChunk];  // head block byte offsets, -1: skip

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

  // byte offset of the head block holding position p, or -1 (flagged)
  auto head_at = [&](int p) -> int64_t {
    const int32_t blk = row[p / kBlockSize];
    if (blk < 0 || blk >= a.num_blocks) {
      raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
      return -1;
    }
    return static_cast<int64_t>(blk) * a.page_bytes + static_cast<int64_t>(g) * Lay::kHeadBytes;
  };

  for (int c0 = 0; c0 < count; c0 += kTrimChunk) {
    const int m = min(kTrimChunk, count - c0);
    // head blocks of the chunk's sources and destinations (-1: a missing
    // page on either side; that token is not moved)
    if (tid < m) {
      const int64_t hs = head_at(a.keep + n + c0 + tid);
      const int64_t hd = head_at(a.keep + c0 + tid);
      const bool ok = hs >= 0 && hd >= 0;
      // the offsets fit in int32 after dividing out the head block (pool
      // sizes are checked on the host); keep them as head-block indexes
      s_src[tid] = ok ? static_cast<int>(hs / Lay::kHeadBytes) : -1;
      s_dst[tid] = ok ? static_cast<int>(hd / Lay::kHeadBytes) : -1;
    }
    __syncthreads();
    // read the chunk
    for (int e = tid; e < m * KV; e += kTrimThreads) {
      const int i = e / KV, c = e % KV;
      if (s_src[i] < 0) continue;
      const int pos = (a.keep + n + c0 + i) % kBlockSize;
      const uint8_t* h = a.pool + static_cast<int64_t>(s_src[i]) * Lay::kHeadBytes;
      s_k[i][c] = reinterpret_cast<const u4_t*>(h + Lay::k_off(pos))[c];
    }
    for (int e = tid; e < m * D; e += kTrimThreads) {
      const int i = e / D, d = e % D;
      if (s_src[i] < 0) continue;
      const int pos = (a.keep + n + c0 + i) % kBlockSize;
      const uint8_t* h = a.pool + static_cast<int64_t>(s_src[i]) * Lay::kHeadBytes;
      s_v[i][d] = *reinterpret_cast<const T*>(h + Lay::v_off(pos, d));
    }
    if constexpr (Scales) {
      if (tid < m && s_src[tid] >= 0) {
        const int pos = (a.keep + n + c0 + tid) % kBlockSize;
        const uint8_t* h = a.pool + static_cast<int64_t>(s_src[tid]) * Lay::kHeadBytes;
        s_sc[tid] = *reinterpret_cast<const uint16_t*>(h + Lay::ks_off(pos)) |
                    (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(h + Lay::vs_off(pos)))
                     << 16);
      }
    }
    __syncthreads();
    // write it n positions further to the front
    for (int e = tid; e < m * KV; e += kTrimThreads) {
      const int i = e / KV, c = e % KV;
      if (s_dst[i] < 0) continue;
      const int pos = (a.keep + c0 + i) % kBlockSize;
      uint8_t* h = a.pool + static_cast<int64_t>(s_dst[i]) * Lay::kHeadBytes;
      reinterpret_cast<u4_t*>(h + Lay::k_off(pos))[c] = s_k[i][c];
    }
    for (int e = tid; e < m * D; e += kTrimThreads) {
      const int i = e / D, d = e % D;
      if (s_dst[i] < 0) continue;
      const int pos = (a.keep + c0 + i) % kBlockSize;
      uint8_t* h = a.pool + static_cast<int64_t>(s_dst[i]) * Lay::kHeadBytes;
      *reinterpret_cast<T*>(h + Lay::v_off(pos, d)) = s_v[i][d];
    }
    if constexpr (Scales) {
      if (tid < m && s_dst[tid] >= 0) {
        const int pos = (a.keep + c0 + tid) % kBlockSize;
        uint8_t* h = a.pool + static_cast<int64_t>(s_dst[tid]) * Lay::kHeadBytes;
        *reinterpret_cast<uint16_t*>(h + Lay::ks_off(pos)) = static_cast<uint16_t>(s_sc[tid]);
        *reinterpret_cast<uint16_t*>(h + Lay::vs_off(pos)) =
            static_cast<uint16_t>(s_sc[tid] >> 16);
      }
    }
    __syncthreads();  // the next chunk reuses the LDS
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
