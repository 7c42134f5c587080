// Device helpers shared by the gfx950 kernels: vector types, 16-bit
// conversions, wave reductions, output stores.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/pdakv.h"

namespace pdakv {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <bool BF16>
__device__ __forceinline__ float bits16_to_f32(uint16_t b) {
  return BF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Four two's-complement int8 codes (one 32-bit word, byte i = element i)
// -> four fp16 values, exactly. Each byte is biased to c + 128, placed in the
// low mantissa bits of the fp16 constant 1024 (0x6400), and the bias
// 1024 + 128 is subtracted with one packed fp16 op per pair.
__device__ __forceinline__ u2_t i8x4_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = (u & 0xFFu) | ((u & 0xFF00u) << 8) | 0x64006400u;
  const uint32_t hi = ((u >> 16) & 0xFFu) | ((u >> 8) & 0xFF0000u) | 0x64006400u;
  const h2_t bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  const h2_t a = __builtin_bit_cast(h2_t, lo) - bias;
  const h2_t b = __builtin_bit_cast(h2_t, hi) - bias;
  u2_t r;
  r.x = __builtin_bit_cast(uint32_t, a);
  r.y = __builtin_bit_cast(uint32_t, b);
  return r;
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  h2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Maximum over the 64 lanes, in every lane, on the VALU alone: rotations by
// 8, 4, 2 and 1 lanes inside each row of 16 (DPP), then the row-swap
// instructions across rows and across the two halves (a lane shuffle would
// take six round trips through LDS).
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), Ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0x128>(x));  // row_ror:8
  x = max(x, dpp_u32<0x124>(x));  // row_ror:4
  x = max(x, dpp_u32<0x122>(x));  // row_ror:2
  x = max(x, dpp_u32<0x121>(x));  // row_ror:1
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(r[0], r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(h[0], h[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float max_nc(float a, float b) { return a > b ? a : b; }

// The larger of two values that are at most the largest finite float (-inf
// included), as one median-of-three against that bound. (Against +inf the
// compiler turns the median into a maximum and first quiets both operands,
// two more instructions, as the operands of a lane swap are not known to be
// canonical.)
constexpr float kMaxFinite = 3.40282347e38f;
__device__ __forceinline__ float max_fin(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, kMaxFinite);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (same column of a 16x16
// MFMA tile), with the gfx950 row-swap instructions (VALU only, no LDS round
// trip): swapping a value with itself across 32-lane halves, then across
// 16-lane rows, pairs every lane with its partner.
__device__ __forceinline__ float col_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = max_fin(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const uint32_t v = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max_fin(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const uint32_t v = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void store_out(void* out, int dtype, int64_t idx, float v) {
  if (dtype == PDAKV_DTYPE_F32) {
    static_cast<float*>(out)[idx] = v;
  } else if (dtype == PDAKV_DTYPE_F16) {
    static_cast<_Float16*>(out)[idx] = static_cast<_Float16>(v);
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  }
}

__device__ __forceinline__ void raise_flag(int32_t* err, int bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace pdakv
