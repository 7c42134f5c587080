// Quantize-on-write and 16-bit write into paged KV pools (gfx950).
//
// One wave (64 lanes) owns one (token, KV head) pair and handles its K row and
// its V row; a workgroup holds four waves. Three pool formats: per-token INT8
// (codes + FP16 scales), static-scale INT8 (codes only) and 16-bit. The row
// quantizer (quant_row.h) follows MoE-Infinity PR #183 "feat: opt-in INT8
// KV-cache quantization" ("What landed", format-contract bullet; "Precision &
// memory") and the zero-token rule of mlxcel PR #717 ("The Int8 bug and fix").
#include "device_util.h"
#include "launch.h"
#include "quant_row.h"

namespace pdakv {

namespace {

constexpr int kWriteWaves = 4;

template <int D>
struct Int8Head {
  static constexpr int kBytes = 2 * kBlockSize * D + 4 * kBlockSize;
  static constexpr int kV = kBlockSize * D;          // V codes
  static constexpr int kKs = 2 * kBlockSize * D;     // K scales
  static constexpr int kVs = 2 * kBlockSize * D + 2 * kBlockSize;
};

template <typename T>
__device__ __forceinline__ uint16_t load_bits(const void* base, int64_t idx) {
  return static_cast<const uint16_t*>(base)[idx];
}

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kWriteWaves) void quant_write_int8_kernel(WriteArgs a) {
  constexpr int EPL = D / 64;  // elements per lane
  using H = Int8Head<D>;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWriteWaves + (threadIdx.x >> 6);
  if (row >= a.num_tokens * a.num_kv_heads) return;
  const int64_t t = row / a.num_kv_heads;
  const int h = static_cast<int>(row - t * a.num_kv_heads);
  const int32_t slot = a.slots[t];
  if (slot < 0) return;  // padding token
  if (slot >= a.num_blocks * kBlockSize) {
    if (lane == 0) raise_flag(a.err, PDAKV_EFLAG_SLOT_RANGE);
    return;
  }
  const int64_t blk = slot / kBlockSize;
  const int pos = slot % kBlockSize;
  uint8_t* head = a.pool + blk * a.page_bytes + static_cast<int64_t>(h) * H::kBytes;

  float xk[EPL], xv[EPL];
  float ak = 0.f, av = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int64_t d = lane * EPL + e;
    xk[e] = bits16_to_f32<BF16>(load_bits<uint16_t>(a.k, t * a.k_st + h * a.k_sh + d * a.k_sd));
    xv[e] = bits16_to_f32<BF16>(load_bits<uint16_t>(a.v, t * a.v_st + h * a.v_sh + d * a.v_sd));
    ak = fmaxf(ak, fabsf(xk[e]));
    av = fmaxf(av, fabsf(xv[e]));
  }
  ak = wave_max(ak);
  av = wave_max(av);

  uint16_t skb, svb;
  const bool okk = row_scale(ak, skb), okv = row_scale(av, svb);
  if (!okk || !okv) {
    if (lane == 0) raise_flag(a.err, PDAKV_EFLAG_SCALE_RANGE);
    return;
  }
  const float sk = f16_bits_to_f32(skb);
  const float sv = f16_bits_to_f32(svb);

  uint8_t ck[EPL], cv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    ck[e] = row_code(xk[e], sk);
    cv[e] = row_code(xv[e], sv);
  }
  // K: token-major row; V: dimension d of tokens grouped by four.
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int d = lane * EPL + e;
    head[pos * D + d] = ck[e];
    head[H::kV + (pos >> 2) * 4 * D + d * 4 + (pos & 3)] = cv[e];
  }
  if (lane == 0) {
    *reinterpret_cast<uint16_t*>(head + H::kKs + 2 * pos) = skb;
    *reinterpret_cast<uint16_t*>(head + H::kVs + 2 * pos) = svb;
  }
}

// Static scales (InfiniLM PR #553 "Summary"; TensorRT-LLM PR #18953
// "Summary"): the layer's K scale and V scale are given, so a row needs no
// reduction: code = clamp(rint(fl32(x / scale)), -127, 127), stored into a
// codes-only head block (K codes, then V codes grouped by four tokens).
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kWriteWaves) void quant_write_static_kernel(WriteArgs a) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWriteWaves + (threadIdx.x >> 6);
  if (row >= a.num_tokens * a.num_kv_heads) return;
  const int64_t t = row / a.num_kv_heads;
  const int h = static_cast<int>(row - t * a.num_kv_heads);
  const int32_t slot = a.slots[t];
  if (slot < 0) return;
  if (slot >= a.num_blocks * kBlockSize) {
    if (lane == 0) raise_flag(a.err, PDAKV_EFLAG_SLOT_RANGE);
    return;
  }
  const int64_t blk = slot / kBlockSize;
  const int pos = slot % kBlockSize;
  uint8_t* head = a.pool + blk * a.page_bytes + static_cast<int64_t>(h) * 2 * kBlockSize * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int d = lane * EPL + e;
    const float xk =
        bits16_to_f32<BF16>(load_bits<uint16_t>(a.k, t * a.k_st + h * a.k_sh + d * a.k_sd));
    const float xv =
        bits16_to_f32<BF16>(load_bits<uint16_t>(a.v, t * a.v_st + h * a.v_sh + d * a.v_sd));
    head[pos * D + d] = row_code(xk, a.k_scale);
    head[kBlockSize * D + (pos >> 2) * 4 * D + d * 4 + (pos & 3)] = row_code(xv, a.v_scale);
  }
}

template <int D>
__global__ __launch_bounds__(64 * kWriteWaves) void write_16bit_kernel(WriteArgs a) {
  constexpr int EPL = D / 64;
  constexpr int kHeadElems = 2 * kBlockSize * D;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kWriteWaves + (threadIdx.x >> 6);
  if (row >= a.num_tokens * a.num_kv_heads) return;
  const int64_t t = row / a.num_kv_heads;
  const int h = static_cast<int>(row - t * a.num_kv_heads);
  const int32_t slot = a.slots[t];
  if (slot < 0) return;
  if (slot >= a.num_blocks * kBlockSize) {
    if (lane == 0) raise_flag(a.err, PDAKV_EFLAG_SLOT_RANGE);
    return;
  }
  const int64_t blk = slot / kBlockSize;
  const int pos = slot % kBlockSize;
  uint16_t* head = reinterpret_cast<uint16_t*>(a.pool + blk * a.page_bytes) +
                   static_cast<int64_t>(h) * kHeadElems;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int d = lane * EPL + e;
    head[pos * D + d] = load_bits<uint16_t>(a.k, t * a.k_st + h * a.k_sh + d * a.k_sd);
    head[kBlockSize * D + (pos >> 2) * 4 * D + d * 4 + (pos & 3)] =
        load_bits<uint16_t>(a.v, t * a.v_st + h * a.v_sh + d * a.v_sd);
  }
}

unsigned write_grid(const WriteArgs& a) {
  const int64_t rows = a.num_tokens * a.num_kv_heads;
  return static_cast<unsigned>((rows + kWriteWaves - 1) / kWriteWaves);
}

}  // namespace

hipError_t launch_quant_write_int8(const WriteArgs& a, int head_dim, bool src_bf16,
                                   hipStream_t s) {
  const dim3 grid(write_grid(a)), block(64 * kWriteWaves);
  if (head_dim == 128) {
    if (src_bf16)
      hipLaunchKernelGGL((quant_write_int8_kernel<128, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((quant_write_int8_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (src_bf16)
      hipLaunchKernelGGL((quant_write_int8_kernel<64, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((quant_write_int8_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_quant_write_static(const WriteArgs& a, int head_dim, bool src_bf16,
                                     hipStream_t s) {
  const dim3 grid(write_grid(a)), block(64 * kWriteWaves);
  if (head_dim == 128) {
    if (src_bf16)
      hipLaunchKernelGGL((quant_write_static_kernel<128, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((quant_write_static_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (src_bf16)
      hipLaunchKernelGGL((quant_write_static_kernel<64, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((quant_write_static_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_write_16bit(const WriteArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(write_grid(a)), block(64 * kWriteWaves);
  if (head_dim == 128)
    hipLaunchKernelGGL((write_16bit_kernel<128>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((write_16bit_kernel<64>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace pdakv
