// Internal interface between the C-ABI layer (abi.cpp) and the kernel
// translation units. Not installed; the public contract is include/pdakv.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/pdakv.h"

namespace pdakv {

constexpr int kBlockSize = 16;        // tokens per page
constexpr int kMaxGroup = 16;         // query heads per KV head (one MFMA N tile)
constexpr int kWaves = 4;             // waves per decode workgroup
constexpr int kMinPagesPerWave = 2;   // decode: fewest pages a busy wave gets (one pair)
constexpr int kInt8WavesPerSimd = 2;  // INT8 decode occupancy
constexpr int kInt8PageGroup = 2;     // pages per register buffer
constexpr int k16WavesPerSimd = 2;    // 16-bit decode occupancy
constexpr int k16PageGroup = 2;
constexpr int kOneWaveBlockBytes = 4096;  // one-token plans: one wave per SIMD from
                                          // this KV-head page-block size up
constexpr int kSimdsPerCU = 4;
constexpr int kDefaultCUs = 256;      // MI355X compute units (when no device answers)
constexpr int kMaxMergeWaves = 8;              // merge: waves per (sequence, q head)
constexpr int kLdsPerWave = 16384;             // decode: LDS staging budget per wave
constexpr int kMaxPagesPerWave = 128; // decode: block ids a wave holds (2 per lane)
// Calls with few units: one workgroup of kUnitWaves waves per (sequence, KV
// head), for one-token decodes of at most kUnitMaxUnits units whose pages
// split into at most kUnitMaxPagesPerWave per wave (measured: a 256-token
// context at batch 1, two pages per wave, 15.0 -> 9.4 us; at 2K, sixteen
// pages per wave, 16.8 -> 23.8 us, so longer contexts keep the even split
// over the grid).
constexpr int kUnitWaves = 8;
constexpr int kUnitMaxUnits = 64;
constexpr int kUnitMaxPagesPerWave = 4;

// Several-token decode: query tiles (16 columns each) per unit, at most
// kMaxUnitTiles, and the waves per SIMD of the kernel for a unit of `tiles`
// tiles (what the registers of that many tiles' states allow).
constexpr int kMaxUnitTiles = 4;
constexpr int wide_waves_per_simd(int kv_format, int tiles) {
  return tiles == 1 ? 2 : (tiles == 2 && kv_format != PDAKV_KV_16BIT) ? 2 : 1;
}

struct WriteArgs {
  const void* k;
  const void* v;
  int64_t num_tokens;
  int num_kv_heads;
  int64_t k_st, k_sh, k_sd;  // element strides
  int64_t v_st, v_sh, v_sd;
  const int32_t* slots;
  uint8_t* pool;
  int64_t num_blocks;
  int64_t page_bytes;
  float k_scale, v_scale;  // static-scale format: the layer's K and V scales
  float k_rcp, v_rcp;      // and their reciprocals fl(1 / scale)
  int32_t* err;
};

struct DecodeArgs {
  void* out;
  int out_dtype;
  int64_t out_ss, out_st, out_sh;  // element strides: sequence, query token, head
  const void* q;
  int64_t q_ss, q_st, q_sh;
  int q_vec16;  // q pointer and strides allow 16-byte loads of 8 elements
  uint8_t* pool;  // written only by the fused append
  int64_t num_blocks;
  int64_t page_bytes;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* ctx;
  int num_seqs, num_q_heads, num_kv_heads, group, max_ctx;
  // query tokens per sequence (the last qtok positions, causal among them);
  // their cols = qtok * group (token, head) columns per KV head are split
  // into tiles of up to 16 MFMA columns, unit_tiles consecutive tiles of a
  // KV head form a unit (streamed once for all its tiles), so a KV head has
  // units_per_head units: vheads = num_kv_heads * units_per_head per sequence
  int qtok, cols, unit_tiles, units_per_head, vheads;
  int slot_cols;  // columns per workspace slot: min(cols, 16 * unit_tiles)
  float scale_log2;  // sm_scale * log2(e) (times the K scale for static
                     // scales): logits are kept in base 2
  float out_mul;     // output factor: the V scale for static scales, else 1
  float k_scale, v_scale;  // static scales (quantizer of the fused append)
  float* ws;         // partials [num_waves + B * Hkv][G][D + 2]
  int2* desc;        // per (sequence, KV head): first covering wave, wave count
  int num_waves;     // waves of the decode grid (a multiple of kWaves)
  int merge_waves;   // waves per merge workgroup (1 .. kMaxMergeWaves)
  int unit_path;     // decode: one workgroup per unit (a call with few units)
  int seg_cap;       // decode: segments staged in LDS per pass
  int lds_wave_bytes;  // decode: LDS per wave (q rows, results, appended tokens)
  int lds_q_off;       // decode: offsets of the q rows, results and appended
  int lds_res_off;     // tokens in a wave's LDS
  int lds_nt_off;
  // append (fused write of each sequence's newest token, at position L - 1):
  // 16-bit K and V rows [B][Hkv][D] in q's dtype, element strides
  int append;
  const void* k_new;
  const void* v_new;
  int64_t kn_st, kn_sh, kn_sd, vn_st, vn_sh, vn_sd;
  int32_t* err;
};

// Whole-page copies between a pool and a packed page array.
struct PageCopyArgs {
  uint8_t* pool;
  int64_t num_blocks;
  int64_t page_bytes;  // a multiple of 16
  uint8_t* packed;     // [num_pages][page_bytes]
  const int32_t* ids;  // [num_pages] pool block of packed page i
  int64_t num_pages;
  int gather;          // 1: pool -> packed (swap-out), 0: packed -> pool (swap-in)
  int32_t* err;
};

// Front trim keeping `keep` sink tokens of every sequence.
struct TrimArgs {
  uint8_t* pool;
  int64_t num_blocks;
  int64_t page_bytes;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* ctx;
  const int32_t* trim;  // tokens to drop after the sink, per sequence
  int32_t* new_ctx;
  int num_seqs, num_kv_heads, keep;
  int windows;  // workgroups per (sequence, KV head); set by the launcher
  int32_t* err;
};

// Each returns hipSuccess or the launch error. Arguments are validated by the
// caller; the launchers only pick the template instance.
hipError_t launch_quant_write_int8(const WriteArgs& a, int head_dim, bool src_bf16,
                                   hipStream_t s);
hipError_t launch_write_16bit(const WriteArgs& a, int head_dim, hipStream_t s);
hipError_t launch_decode_int8(const DecodeArgs& a, int head_dim, bool q_bf16, hipStream_t s);
// several query tokens per sequence (a.qtok >= 1)
hipError_t launch_decode_int8_multi(const DecodeArgs& a, int head_dim, bool q_bf16,
                                    hipStream_t s);
hipError_t launch_decode_16bit_multi(const DecodeArgs& a, int head_dim, bool kv_bf16,
                                     hipStream_t s);

hipError_t launch_decode_16bit(const DecodeArgs& a, int head_dim, bool kv_bf16,
                               hipStream_t s);
hipError_t launch_quant_write_static(const WriteArgs& a, int head_dim, bool src_bf16,
                                     hipStream_t s);
hipError_t launch_page_copy(const PageCopyArgs& a, hipStream_t s);
hipError_t launch_trim_keep_sink(const TrimArgs& a, int kv_format, int head_dim, hipStream_t s);
hipError_t launch_decode_int8_static(const DecodeArgs& a, int head_dim, bool q_bf16,
                                     hipStream_t s);

}  // namespace pdakv
