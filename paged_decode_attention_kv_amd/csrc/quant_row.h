// Per-token symmetric INT8 quantizer of one row (D elements spread over the
// 64 lanes of a wave), as the decode kernel's append step uses it. The
// quantize-on-write kernel shares round_up_f16 (and row_code for static
// scales outside its division-free window) and computes the same scale and
// codes without a division, so both store bit-identical rows.
//
// MoE-Infinity PR #183 "feat: opt-in INT8 KV-cache quantization" ("What
// landed", format-contract bullet; "Precision & memory") and the zero-token
// rule of mlxcel PR #717 ("The Int8 bug and fix"):
//   a = max|x|; scale = 1.0 if a == 0 else the smallest FP16 >= fl32(a/127);
//   code = clamp(rint(fl32(x / scale)), -127, 127).
// The division is IEEE binary32 (the library is built with correctly rounded
// division and without denormal flushing), so codes are exact functions of
// the input and match any other IEEE implementation bit for bit.
#pragma once

#include "device_util.h"

namespace pdakv {

// Smallest fp16 >= s (s finite, 0 < s <= 65504), as raw bits.
__device__ __forceinline__ uint16_t round_up_f16(float s) {
  _Float16 h = static_cast<_Float16>(s);  // round to nearest even
  uint16_t bits = __builtin_bit_cast(uint16_t, h);
  if (static_cast<float>(h) < s) bits += 1;  // next fp16 above (s > 0)
  if (bits == 0) bits = 1;                     // s > 0 never rounds up to 0
  return bits;
}

// Scale of a row with absmax a (already reduced over the wave): false when
// a/127 exceeds the FP16 range or a is not finite (the row cannot be stored).
__device__ __forceinline__ bool row_scale(float a, uint16_t& bits) {
  const float s32 = a / 127.0f;
  if (!(s32 <= 65504.0f)) return false;
  bits = a == 0.f ? 0x3C00 : round_up_f16(s32);
  return true;
}

__device__ __forceinline__ uint8_t row_code(float x, float scale) {
  return static_cast<uint8_t>(static_cast<int8_t>(fminf(fmaxf(rintf(x / scale), -127.f), 127.f)));
}


}  // namespace pdakv
