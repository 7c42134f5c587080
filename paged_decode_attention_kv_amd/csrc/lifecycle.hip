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
//   positions toward the front through the sequence's own block table.
//   Workgroups move rounds of up to 128 tokens, each round read completely
//   (K rows as 16-byte vectors, V as words holding a dimension of four
//   tokens) into LDS before any of it is written. A small trim is one chain
//   of rounds per (sequence, KV head); a trim of 128 or more splits into
//   windows of residues mod n that run in parallel (the ordering argument is
//   given above the kernel).
#include <algorithm>

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
// tokens moved per round (a multiple of 4); rounds of 256 measured slower
// (fewer workgroups per CU and fewer windows), 512 no faster
constexpr int kTrimRound = 128;
// workgroups a trim launch aims for (about sixteen per compute unit)
constexpr int64_t kTrimWorkgroups = 4096;

// Token layout of a KV head's part of a page. Code block (every head's code
// block comes first in a page, head g's at g * kCodeBytes): element size E
// (1: INT8 codes, 2: 16-bit values), K row of D elements at pos * D, V
// grouped four tokens at a time (element d of token pos at 16 * D +
// (pos / 4) * 4 * D + 4 * d + pos % 4, so one "V word" of 4 * E bytes holds
// dimension d of a whole group). Per-token INT8 pages then hold every head's
// fp16 scales (head g's 64 bytes at Hkv * kCodeBytes + 64 * g), a 16-byte
// record per four tokens: their K scales, then their V scales.
template <int D, int E, bool Scales>
struct TokenLayout {
  static constexpr int kCodeBytes = 32 * D * E;
  static constexpr int kRowBytes = D * E;
  static __device__ __forceinline__ int k_off(int pos) { return pos * D * E; }
  static __device__ __forceinline__ int vword_off(int group, int d) {  // group of the page
    return (16 * D + group * 4 * D + 4 * d) * E;
  }
  // from the head's scale records
  static __device__ __forceinline__ int ks_off(int pos) { return 16 * (pos / 4) + 2 * (pos % 4); }
  static __device__ __forceinline__ int vs_off(int pos) { return ks_off(pos) + 8; }
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

// Destination word of a group whose four tokens come from source groups lo
// and hi (consecutive), the first of them `shift` tokens into lo.
__device__ __forceinline__ uint32_t shift_word(uint32_t lo, uint32_t hi, int shift) {
  return shift == 0 ? lo : __builtin_amdgcn_alignbyte(hi, lo, shift);
}
__device__ __forceinline__ uint64_t shift_word(uint64_t lo, uint64_t hi, int shift) {
  return shift == 0 ? lo : (lo >> (16 * shift)) | (hi << (64 - 16 * shift));
}

// Moved tokens are numbered t = 0 .. count-1 (source keep + n + t,
// destination keep + t), so token t's destination is token (t - n)'s
// source. Every round reads all of its sources before writing any
// destination, and a workgroup runs its rounds in increasing t:
// * n >= C: window w owns the tokens whose t mod n lies in [w*C, w*C + C);
//   its round k moves t in w*C + k*n + [0, C). Round k writes exactly what
//   round k-1 of the same window read, and no other window touches these
//   positions, so windows run in parallel.
// * n < C: one window moves t in k*C + [0, C); round k writes into round
//   k-1's sources (at most), never into a later round's.
template <int D, int E, bool Scales>
__global__ __launch_bounds__(kTrimThreads) void trim_keep_sink_kernel(TrimArgs a) {
  using Lay = TokenLayout<D, E, Scales>;
  using T = typename Elem<E>::T;
  using W = typename Elem<E>::W;
  constexpr int C = kTrimRound;
  constexpr int KV = Lay::kRowBytes / 16;  // 16-byte vectors per K row
  static_assert(C * KV % kTrimThreads == 0, "K vectors split evenly over the threads");
  constexpr int KPT = C * KV / kTrimThreads;  // K vectors per thread
  // groups of four tokens a round touches on either side (C / 4 + 1), rounded
  // up so that the V words split evenly over the threads
  constexpr int VPT = ((C / 4 + 1) * D + kTrimThreads - 1) / kTrimThreads;
  constexpr int VG = VPT * kTrimThreads / D;
  static_assert(VG * D == VPT * kTrimThreads, "V words split evenly over the threads");
  constexpr int TPT = (C + kTrimThreads - 1) / kTrimThreads;  // tokens per thread
  __shared__ u4_t s_k[C][KV];
  __shared__ W s_vw[VG][D];     // the round's source V words
  __shared__ uint32_t s_sc[C];  // K scale | V scale << 16
  // block id of each token's source page (-1: missing) and of its
  // destination page (-1: missing, or the token is not moved)
  __shared__ int s_src[C], s_dst[C];
  __shared__ int s_whole[VG];  // destination group: all four tokens move in this round

  // window-major: the first windows of all pairs come first, so that the
  // busy workgroups of a small trim (window 0 only) spread over the XCDs
  const int units = a.num_seqs * a.num_kv_heads;
  const int w0 = blockIdx.x / units, unit = blockIdx.x % units;
  const int b = unit / a.num_kv_heads, g = unit % a.num_kv_heads;
  const int tid = threadIdx.x;
  const bool leader = g == 0 && w0 == 0 && tid == 0;
  int L = a.ctx[b];
  const int64_t cap = a.bt_stride * kBlockSize;
  if (L < 0 || L > cap) {
    if (leader) raise_flag(a.err, PDAKV_EFLAG_CONTEXT_RANGE);
    L = L < 0 ? 0 : static_cast<int>(cap);
  }
  const int room = L > a.keep ? L - a.keep : 0;
  int n = a.trim[b];
  n = n < 0 ? 0 : (n > room ? room : n);
  if (leader) a.new_ctx[b] = L - n;
  const int count = L - a.keep - n;  // tokens that move
  if (n == 0 || count <= 0) return;
  if (a.num_blocks < 1) {  // every page is missing; page 0 is not there to read
    if (w0 == 0 && tid == 0) raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
    return;
  }
  const int32_t* row = a.bt + static_cast<int64_t>(b) * a.bt_stride;
  // KV head g's code block and scale records in page blk
  auto head = [&](int blk) {
    return a.pool + static_cast<int64_t>(blk) * a.page_bytes + g * Lay::kCodeBytes;
  };
  auto scales = [&](int blk) {
    return a.pool + static_cast<int64_t>(blk) * a.page_bytes +
           a.num_kv_heads * Lay::kCodeBytes + 64 * g;
  };
  const int shift = n & 3;  // tokens between a destination group's start and its source group's
  const bool wide = n >= C;
  const int nwin = wide ? (min(n, count) + C - 1) / C : 1;
  const int step = wide ? n : C;

  for (int w = w0; w < nwin; w += a.windows) {
    const int width = wide ? min(C, n - w * C) : C;
    for (int t0 = wide ? w * C : 0; t0 < count; t0 += step) {
      const int m = min(width, count - t0);
      const int s0 = a.keep + n + t0;  // first source position of the round
      const int q0 = a.keep + t0;      // its destination
      for (int i = tid; i < m; i += kTrimThreads) {
        const int32_t bs = row[(s0 + i) / kBlockSize], bd = row[(q0 + i) / kBlockSize];
        const bool src_ok = bs >= 0 && bs < a.num_blocks;
        const bool dst_ok = bd >= 0 && bd < a.num_blocks;
        if (!src_ok || !dst_ok) raise_flag(a.err, PDAKV_EFLAG_BLOCK_RANGE);
        // the four tokens of a source group share its page, so they share
        // src_ok: a group's V word is read whenever one of them is moved
        s_src[i] = src_ok ? bs : -1;
        s_dst[i] = src_ok && dst_ok ? bd : -1;
      }
      __syncthreads();

      // read the round. Every load is issued unconditionally, before any is
      // used, and every loaded value is staged in LDS: an item past the
      // round's end is clamped to its last token, and an item whose source
      // page is missing reads page 0 instead (neither value is written out).
      u4_t kreg[KPT];
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int e = tid + r * kTrimThreads;
        const int i = min(e / KV, m - 1), c = e % KV;
        const int hs = s_src[i];
        const uint8_t* h = hs >= 0 ? head(hs) + Lay::k_off((s0 + i) % kBlockSize) : a.pool;
        kreg[r] = reinterpret_cast<const u4_t*>(h)[hs >= 0 ? c : 0];
      }
      const int gfirst = s0 / 4, ngroups = (s0 + m - 1) / 4 - gfirst + 1;
      W vreg[VPT];
#pragma unroll
      for (int r = 0; r < VPT; ++r) {
        const int e = tid + r * kTrimThreads;
        const int gi = min(e / D, ngroups - 1), d = e % D;
        const int p = max(4 * (gfirst + gi), s0);  // an in-round token of the group
        const int hs = s_src[p - s0];
        vreg[r] = *reinterpret_cast<const W*>(
            hs >= 0 ? head(hs) + Lay::vword_off((p % kBlockSize) / 4, d) : a.pool);
      }
      uint32_t sc[TPT];
      if constexpr (Scales) {
#pragma unroll
        for (int r = 0; r < TPT; ++r) {
          const int i = min(tid + r * kTrimThreads, m - 1);
          const int pos = (s0 + i) % kBlockSize, hs = s_src[i];
          const uint8_t* h = hs >= 0 ? scales(hs) : a.pool;
          sc[r] = *reinterpret_cast<const uint16_t*>(h + (hs >= 0 ? Lay::ks_off(pos) : 0)) |
                  (static_cast<uint32_t>(
                       *reinterpret_cast<const uint16_t*>(h + (hs >= 0 ? Lay::vs_off(pos) : 0)))
                   << 16);
        }
      }
      // destination groups of the round: whole when all four tokens move now
      const int hfirst = q0 / 4, nhead = (q0 + m - 1) / 4 - hfirst + 1;
      for (int gi = tid; gi < nhead; gi += kTrimThreads) {
        const int p0 = 4 * (hfirst + gi);
        bool whole = p0 >= q0 && p0 + 3 < q0 + m;
        for (int j = 0; whole && j < 4; ++j) whole = s_dst[p0 + j - q0] >= 0;
        s_whole[gi] = whole;
      }
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int e = tid + r * kTrimThreads;
        s_k[e / KV][e % KV] = kreg[r];
      }
#pragma unroll
      for (int r = 0; r < VPT; ++r) {
        const int e = tid + r * kTrimThreads;
        s_vw[e / D][e % D] = vreg[r];
      }
      if constexpr (Scales) {
#pragma unroll
        for (int r = 0; r < TPT; ++r) s_sc[min(tid + r * kTrimThreads, C - 1)] = sc[r];
      }
      __syncthreads();

      // write the round n positions further to the front: LDS first, then
      // the stores that apply
      u4_t kval[KPT];
      int kdst[KPT];
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int e = tid + r * kTrimThreads;
        kval[r] = s_k[e / KV][e % KV];
        kdst[r] = e < m * KV ? s_dst[e / KV] : -1;
      }
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int e = tid + r * kTrimThreads;
        const int i = e / KV, c = e % KV;
        if (kdst[r] >= 0)
          reinterpret_cast<u4_t*>(head(kdst[r]) + Lay::k_off((q0 + i) % kBlockSize))[c] = kval[r];
      }
      // V: a whole destination group takes its four tokens from positions
      // p0 + n .. p0 + n + 3, i.e. source groups gs and gs + 1 starting
      // `shift` tokens into gs; an edge group moves single elements
      W vval[VPT];
      int vdst[VPT];
#pragma unroll
      for (int r = 0; r < VPT; ++r) {
        const int e = tid + r * kTrimThreads;
        const int gi = e / D, d = e % D;
        const int p0 = 4 * (hfirst + gi);
        // (clamped into the array: only a whole group's value is stored)
        const int gs = max(0, min((p0 + n) / 4 - gfirst, VG - 2));
        vval[r] = shift_word(s_vw[gs][d], s_vw[gs + 1][d], shift);
        const bool whole = e < nhead * D && s_whole[gi];
        vdst[r] = whole ? s_dst[p0 - q0] : (e < nhead * D ? -2 : -1);
      }
#pragma unroll
      for (int r = 0; r < VPT; ++r) {
        const int e = tid + r * kTrimThreads;
        const int gi = e / D, d = e % D;
        const int p0 = 4 * (hfirst + gi);
        if (vdst[r] >= 0) {
          *reinterpret_cast<W*>(head(vdst[r]) + Lay::vword_off((p0 % kBlockSize) / 4, d)) = vval[r];
        } else if (vdst[r] == -2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int p = p0 + j;
            if (p < q0 || p >= q0 + m || s_dst[p - q0] < 0) continue;
            const int ps = p + n;  // its source position
            const T v = static_cast<T>(s_vw[ps / 4 - gfirst][d] >> (8 * E * (ps & 3)));
            *reinterpret_cast<T*>(head(s_dst[p - q0]) +
                                  Lay::vword_off((p % kBlockSize) / 4, d) + j * E) = v;
          }
        }
      }
      if constexpr (Scales) {
        for (int i = tid; i < m; i += kTrimThreads) {
          if (s_dst[i] < 0) continue;
          const int pos = (q0 + i) % kBlockSize;
          uint8_t* h = scales(s_dst[i]);
          *reinterpret_cast<uint16_t*>(h + Lay::ks_off(pos)) = static_cast<uint16_t>(s_sc[i]);
          *reinterpret_cast<uint16_t*>(h + Lay::vs_off(pos)) =
              static_cast<uint16_t>(s_sc[i] >> 16);
        }
      }
      __syncthreads();  // the next round reuses the LDS
    }
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
  // windows per (sequence, KV head): enough workgroups to fill the chip, and
  // no more than a context of the block table's capacity can use
  TrimArgs b = a;
  const int64_t units = static_cast<int64_t>(a.num_seqs) * a.num_kv_heads;
  const int64_t most = (a.bt_stride * kBlockSize + kTrimRound - 1) / kTrimRound;
  int64_t win = (kTrimWorkgroups + units - 1) / units;
  win = std::max<int64_t>(1, std::min(win, most));
  if (units * win > INT32_MAX) win = 1;
  b.windows = static_cast<int>(win);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(units * win)), dim3(kTrimThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace pdakv
