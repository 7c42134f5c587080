// C-ABI entry points of libpdakv.so: argument validation, work planning,
// and dispatch to the gfx950 kernels. See include/pdakv.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/pdakv.h"
#include "launch.h"

namespace {

using pdakv::DecodeArgs;
using pdakv::WriteArgs;

// Compute units of the current device (asked once; MI355X's 256 when no
// device answers, e.g. for the host-only size queries on a machine without
// a GPU).
int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
      return n;
    (void)hipGetLastError();
    return pdakv::kDefaultCUs;
  }();
  return cus;
}

// Decode waves resident at once: CUs x 4 SIMDs x the waves per SIMD the
// kernel's register budget allows.
int64_t resident_waves(int waves_per_simd) {
  return int64_t{device_cus()} * pdakv::kSimdsPerCU * waves_per_simd;
}
// Waves per SIMD the one-token kernel of a format can hold (its registers).
int kernel_waves_per_simd(int kv_format) {
  return kv_format == PDAKV_KV_16BIT ? pdakv::k16WavesPerSimd : pdakv::kInt8WavesPerSimd;
}
// Waves per SIMD a one-token plan of `items` items fills. Each wave keeps
// two page groups in flight; where one KV head's block of a page holds at
// least kOneWaveBlockBytes (INT8 pages at head size 128, 16-bit pages) and
// one wave per SIMD can hold every item (<= kMaxPagesPerWave each), that
// round keeps enough bytes in flight and streams twice the pages per start
// and per partial, which measured faster at 8K and 32K contexts than two;
// smaller blocks (INT8 at head size 64) and larger calls take the kernel's
// occupancy (a full round, never a mix of SIMDs with one and two waves).
int format_waves_per_simd(int kv_format, int head_dim, int64_t items) {
  const int elem_bytes = kv_format == PDAKV_KV_16BIT ? 2 : 1;
  if (pdakv::kBlockSize * 2 * head_dim * elem_bytes >= pdakv::kOneWaveBlockBytes &&
      items <= resident_waves(1) * pdakv::kMaxPagesPerWave)
    return 1;
  return kernel_waves_per_simd(kv_format);
}

bool known_format(int f) {
  return f == PDAKV_KV_INT8_SYM || f == PDAKV_KV_16BIT || f == PDAKV_KV_INT8_STATIC;
}

// A static scale must be finite and positive.
bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Largest item count (sequence x KV head x page) a launch may hold, so that
// item indexes and wave * pages products stay in int32 on the device.
constexpr int64_t kMaxItems = int64_t{1} << 30;

bool supported_head_dim(int d) { return d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound of the items of a launch: every sequence at max_context_len.
int64_t item_bound(int num_seqs, int num_kv_heads, int max_context_len) {
  return static_cast<int64_t>(num_seqs) * num_kv_heads *
         ceil_div(max_context_len, pdakv::kBlockSize);
}

// Waves of the decode grid. The device splits the actual items evenly over
// them (at least kMinPagesPerWave each), so one resident round of waves is
// used whenever that keeps every wave at <= kMaxPagesPerWave items; small
// launches get fewer waves so that each still has a few pages to pipeline.
int64_t plan_waves(int waves_per_simd, int num_seqs, int num_kv_heads, int max_context_len) {
  const int64_t items = item_bound(num_seqs, num_kv_heads, max_context_len);
  int64_t v = std::max(resident_waves(waves_per_simd), ceil_div(items, pdakv::kMaxPagesPerWave));
  v = std::min(v, ceil_div(items, pdakv::kMinPagesPerWave));
  v = std::max<int64_t>(v, 1);
  return ceil_div(v, pdakv::kWaves) * pdakv::kWaves;
}

// Waves per merge workgroup: about one per kMergeBatch partials of the
// longest unit, estimated with every sequence at max_context_len (the
// device's split of the actual items gives at most a few more).
int merge_waves(int num_seqs, int num_kv_heads, int max_context_len, int64_t waves) {
  const int64_t items = item_bound(num_seqs, num_kv_heads, max_context_len);
  const int64_t ppw = std::max<int64_t>(pdakv::kMinPagesPerWave, ceil_div(items, waves));
  const int64_t parts = ceil_div(ceil_div(max_context_len, pdakv::kBlockSize), ppw) + 1;
  int w = 1;
  while (w < pdakv::kMaxMergeWaves && w * 8 < parts) w *= 2;
  return w;
}

// Waves per SIMD of the kernel a decode call launches, which its plan fills:
// the one-token kernels' occupancy per format, or that of the several-token
// kernel for units of unit_tiles tiles.
int launch_waves_per_simd(int kv_format, bool multi, int unit_tiles, int head_dim,
                          int64_t items) {
  return multi ? pdakv::wide_waves_per_simd(kv_format, unit_tiles)
               : format_waves_per_simd(kv_format, head_dim, items);
}

// Query columns of a call: T query tokens x G query heads per KV head, in
// tiles of at most 16 (one MFMA operand). A unit is one KV head's run of up
// to unit_tiles tiles, whose pages are streamed once for all of them: all
// the tiles of a KV head up to kMaxUnitTiles, else units of that many.
// waves_per_simd: the most that any decode kernel these columns can run in
// holds (every format; for one query token the one-token and the
// several-token kernels), an upper bound of every launch plan, so that a
// workspace sized with it holds the partial slots of every plan.
struct Columns {
  int cols, unit_tiles, units_per_head, slot_cols, waves_per_simd;
};
Columns columns(int num_q_heads, int num_kv_heads, int num_query_tokens) {
  Columns c;
  c.cols = num_query_tokens * (num_q_heads / num_kv_heads);
  const int tiles = (c.cols + 15) / 16;
  c.unit_tiles = std::min(tiles, pdakv::kMaxUnitTiles);
  c.units_per_head = (tiles + c.unit_tiles - 1) / c.unit_tiles;
  c.slot_cols = std::min(c.cols, 16 * c.unit_tiles);
  c.waves_per_simd = 0;
  for (int f : {PDAKV_KV_INT8_SYM, PDAKV_KV_INT8_STATIC, PDAKV_KV_16BIT}) {
    c.waves_per_simd =
        std::max(c.waves_per_simd, pdakv::wide_waves_per_simd(f, c.unit_tiles));
    if (num_query_tokens == 1)
      c.waves_per_simd = std::max(c.waves_per_simd, kernel_waves_per_simd(f));
  }
  return c;
}

// Partial results region of the decode workspace (a multiple of 16 bytes):
// [waves + units][C][D + 2] floats, C = columns per unit, with the waves of
// a plan at the most waves per SIMD any kernel for these columns holds (no
// launch plans more), so one workspace serves every format and head size.
size_t partials_bytes(int num_seqs, int num_query_tokens, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_context_len) {
  const Columns c = columns(num_q_heads, num_kv_heads, num_query_tokens);
  const int vheads = num_kv_heads * c.units_per_head;
  const int64_t v = plan_waves(c.waves_per_simd, num_seqs, vheads, max_context_len);
  const int64_t slots = v + static_cast<int64_t>(num_seqs) * vheads;
  const size_t bytes = static_cast<size_t>(slots) * c.slot_cols * (head_dim + 2) * sizeof(float);
  return (bytes + 15) / 16 * 16;
}

size_t decode_ws_bytes(int num_seqs, int num_query_tokens, int num_q_heads, int num_kv_heads,
                       int head_dim, int max_context_len) {
  if (num_seqs <= 0 || num_query_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_context_len <= 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const Columns c = columns(num_q_heads, num_kv_heads, num_query_tokens);
  const int vheads = num_kv_heads * c.units_per_head;
  if (item_bound(num_seqs, vheads, max_context_len) > kMaxItems) return 0;
  return partials_bytes(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim,
                        max_context_len) +
         static_cast<size_t>(num_seqs) * vheads * 2 * sizeof(int32_t);
}

int check_write(const void* k_src, const void* v_src, int src_dtype, int64_t num_tokens,
                int num_kv_heads, int head_dim, int64_t kst, int64_t ksh, int64_t ksd,
                int64_t vst, int64_t vsh, int64_t vsd, const int32_t* slot_mapping,
                void* kv_pool, int64_t num_blocks, int block_size) {
  if (src_dtype != PDAKV_DTYPE_F16 && src_dtype != PDAKV_DTYPE_BF16) return PDAKV_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PDAKV_ERR_INVALID_ARG;
  if (kst < 0 || ksh < 0 || ksd < 0 || vst < 0 || vsh < 0 || vsd < 0)
    return PDAKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim) || block_size != pdakv::kBlockSize)
    return PDAKV_ERR_UNSUPPORTED;
  if (num_blocks * block_size > INT32_MAX) return PDAKV_ERR_UNSUPPORTED;  // int32 slots
  if (num_tokens == 0) return PDAKV_OK;
  if (!k_src || !v_src || !slot_mapping || !kv_pool) return PDAKV_ERR_INVALID_ARG;
  if (!aligned16(kv_pool)) return PDAKV_ERR_INVALID_ARG;
  return PDAKV_OK;
}

int check_decode(void* out, int out_dtype, int64_t out_ss, int64_t out_st, int64_t out_sh,
                 const void* q, int q_dtype, int64_t q_ss, int64_t q_st, int64_t q_sh, int qtok,
                 const void* kv_pool,
                 int64_t num_blocks, int block_size, const int32_t* block_tables,
                 int64_t bt_stride, const int32_t* context_lens, int num_seqs, int num_q_heads,
                 int num_kv_heads, int head_dim, int max_context_len, float sm_scale,
                 const void* workspace, size_t workspace_bytes) {
  if (q_dtype != PDAKV_DTYPE_F16 && q_dtype != PDAKV_DTYPE_BF16) return PDAKV_ERR_DTYPE;
  if (out_dtype != PDAKV_DTYPE_F32 && out_dtype != PDAKV_DTYPE_F16 &&
      out_dtype != PDAKV_DTYPE_BF16)
    return PDAKV_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      num_blocks < 0 || bt_stride < 0 || out_ss < 0 || out_st < 0 || out_sh < 0 || q_ss < 0 ||
      q_st < 0 || q_sh < 0 || qtok <= 0)
    return PDAKV_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return PDAKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PDAKV_ERR_UNSUPPORTED;
  if (num_q_heads / num_kv_heads > pdakv::kMaxGroup) return PDAKV_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || block_size != pdakv::kBlockSize)
    return PDAKV_ERR_UNSUPPORTED;
  if (bt_stride < ceil_div(max_context_len, block_size)) return PDAKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PDAKV_OK;
  if (!out || !q || !block_tables || !context_lens) return PDAKV_ERR_INVALID_ARG;
  // a non-empty context needs a pool with at least one page (the kernels read
  // page 0 in place of a missing page)
  if (max_context_len > 0 && (!kv_pool || num_blocks < 1)) return PDAKV_ERR_INVALID_ARG;
  // head blocks are indexed as block * num_kv_heads + head in int32
  if (num_blocks * num_kv_heads > INT32_MAX) return PDAKV_ERR_UNSUPPORTED;
  if (kv_pool && !aligned16(kv_pool)) return PDAKV_ERR_INVALID_ARG;
  // device indexes are int32: items, (sequence, query token, query head) rows
  // of the merge grid
  const Columns c = columns(num_q_heads, num_kv_heads, qtok);
  if (item_bound(num_seqs, num_kv_heads * c.units_per_head, max_context_len) > kMaxItems)
    return PDAKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_seqs) * qtok * num_q_heads > INT32_MAX)
    return PDAKV_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(num_seqs, qtok, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PDAKV_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15u)) return PDAKV_ERR_INVALID_ARG;
  return PDAKV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PDAKV_OK : PDAKV_ERR_HIP; }

// The newest token of every sequence for the fused append (absent: plain decode).
struct AppendRows {
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t kst = 0, ksh = 0, ksd = 0, vst = 0, vsh = 0, vsd = 0;
};

// The layer's K and V scales of the static-scale format (1, 1 otherwise).
struct Scales {
  float k = 1.f, v = 1.f;
};

// Output and query views: [num_seqs][tokens][num_q_heads][head_dim] through
// element strides (one token: the token stride is unused).
struct Rows {
  void* out;
  int out_dtype;
  int64_t out_ss, out_st, out_sh;
  const void* q;
  int q_dtype;
  int64_t q_ss, q_st, q_sh;
  int tokens;
  bool multi;  // launch the several-token kernels
};

Rows one_token(void* out, int out_dtype, int64_t out_ss, int64_t out_sh, const void* q,
               int q_dtype, int64_t q_ss, int64_t q_sh) {
  return Rows{out, out_dtype, out_ss, 0, out_sh, q, q_dtype, q_ss, 0, q_sh, 1, false};
}

int decode_common(int fmt, Scales sc, const Rows& r, const AppendRows* app,
                  const void* kv_pool, int64_t num_blocks, int block_size,
                  const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                  int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
                  int32_t* err_flag, void* stream) {
  int st = check_decode(r.out, r.out_dtype, r.out_ss, r.out_st, r.out_sh, r.q, r.q_dtype, r.q_ss,
                        r.q_st, r.q_sh, r.tokens, kv_pool, num_blocks, block_size,
                        block_tables, bt_stride, context_lens, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, max_context_len, sm_scale, workspace,
                        workspace_bytes);
  if (st != PDAKV_OK) return st;
  const double scale_log2 = static_cast<double>(sm_scale) * sc.k * 1.4426950408889634;
  if (!valid_scale(sc.k) || !valid_scale(sc.v) || !std::isfinite(static_cast<float>(scale_log2)))
    return PDAKV_ERR_INVALID_ARG;
  if (app) {
    if (app->kst < 0 || app->ksh < 0 || app->ksd < 0 || app->vst < 0 || app->vsh < 0 ||
        app->vsd < 0)
      return PDAKV_ERR_INVALID_ARG;
    if (num_seqs > 0 && max_context_len > 0 && (!app->k || !app->v)) return PDAKV_ERR_INVALID_ARG;
  }
  if (num_seqs == 0) return st;
  // one query token through a several-token entry point is a one-token
  // decode (the same columns, limits and layout): it runs the one-token
  // kernels, so its results equal the one-token calls' bit for bit
  const bool multi = r.multi && r.tokens > 1;
  DecodeArgs a{};
  a.out = r.out;
  a.out_dtype = r.out_dtype;
  a.out_ss = r.out_ss;
  a.out_st = r.out_st;
  a.out_sh = r.out_sh;
  a.q = r.q;
  a.q_ss = r.q_ss;
  a.q_st = r.q_st;
  a.q_sh = r.q_sh;
  a.q_vec16 = aligned16(r.q) && r.q_ss % 8 == 0 && r.q_st % 8 == 0 && r.q_sh % 8 == 0;
  a.pool = static_cast<uint8_t*>(const_cast<void*>(kv_pool));
  a.num_blocks = num_blocks;
  a.page_bytes =
      static_cast<int64_t>(pdakv_page_bytes(fmt, block_size, num_kv_heads, head_dim));
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.ctx = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  const Columns cols = columns(num_q_heads, num_kv_heads, r.tokens);
  a.qtok = r.tokens;
  a.cols = cols.cols;
  a.unit_tiles = cols.unit_tiles;
  a.units_per_head = cols.units_per_head;
  a.vheads = num_kv_heads * cols.units_per_head;
  a.slot_cols = cols.slot_cols;
  a.max_ctx = max_context_len;
  a.scale_log2 = static_cast<float>(scale_log2);
  a.out_mul = fmt == PDAKV_KV_INT8_STATIC ? sc.v : 1.f;
  a.k_scale = sc.k;
  a.v_scale = sc.v;
  const int wps = launch_waves_per_simd(fmt, multi, cols.unit_tiles, head_dim,
                                        item_bound(num_seqs, a.vheads, max_context_len));
  a.num_waves = static_cast<int>(plan_waves(wps, num_seqs, a.vheads, max_context_len));
  a.merge_waves = merge_waves(num_seqs, a.vheads, max_context_len, a.num_waves);
  {
    // LDS staging of a decode pass of n segments: each segment's q rows
    // (16-bit), each segment's result (accumulator, max, sum per column)
    // and, with the fused append, each segment's new token (4 * head_dim
    // bytes). One-token kernels keep three separate regions. The
    // several-token kernels (16-column segments) let a segment's result,
    // stashed at the switch to the next segment before that segment's q
    // rows are read, cover q slots already read: q slots at the top of the
    // area, result slots from the bottom, the last result stashed in slot 0
    // once the others are written out; the area then needs
    // max(n * qb, (n - 1) * rb + qb, rb) bytes (rb > qb).
    const int qb = a.slot_cols * head_dim * 2, rb = a.slot_cols * (head_dim + 2) * 4;
    const int nb = app ? 4 * head_dim : 0;
    auto up16 = [](int x) { return (x + 15) / 16 * 16; };
    auto area = [&](int n) {
      return multi ? up16(std::max({n * qb, (n - 1) * rb + qb, rb})) : up16(n * (qb + rb));
    };
    int n = 1;
    while (n < 64 && area(n + 1) + (n + 1) * nb <= pdakv::kLdsPerWave) ++n;
    a.seg_cap = n;
    a.lds_q_off = multi ? area(n) - n * qb : 0;
    a.lds_res_off = multi ? 0 : n * qb;
    a.lds_nt_off = area(n);
    a.lds_wave_bytes = area(n) + n * nb;
    if (cols.unit_tiles > 1) {
      // several tiles per unit: passes of one segment, whose q rows are the
      // only LDS staging (results are written from registers)
      a.seg_cap = 1;
      a.lds_q_off = a.lds_res_off = a.lds_nt_off = 0;
      a.lds_wave_bytes = up16(qb);
    }
  }
  // the plan's partial slots (wave + unit) must lie inside the workspace's
  // partials region, which the unit records follow
  const size_t pbytes =
      partials_bytes(num_seqs, r.tokens, num_q_heads, num_kv_heads, head_dim, max_context_len);
  const size_t used = static_cast<size_t>(a.num_waves + static_cast<int64_t>(num_seqs) * a.vheads) *
                      a.slot_cols * (head_dim + 2) * sizeof(float);
  if (used > pbytes) return PDAKV_ERR_WORKSPACE;
  a.ws = static_cast<float*>(workspace);
  a.desc = reinterpret_cast<int2*>(static_cast<uint8_t*>(workspace) + pbytes);
  a.err = err_flag;
  if (app) {
    a.append = 1;
    a.k_new = app->k;
    a.v_new = app->v;
    a.kn_st = app->kst;
    a.kn_sh = app->ksh;
    a.kn_sd = app->ksd;
    a.vn_st = app->vst;
    a.vn_sh = app->vsh;
    a.vn_sd = app->vsd;
  }
  // few units with short contexts: one workgroup per unit, no merge launch
  a.unit_path = !multi &&
                static_cast<int64_t>(num_seqs) * num_kv_heads <= pdakv::kUnitMaxUnits &&
                ceil_div(ceil_div(max_context_len, pdakv::kBlockSize), pdakv::kUnitWaves) <=
                    pdakv::kUnitMaxPagesPerWave;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = r.q_dtype == PDAKV_DTYPE_BF16;
  if (multi)
    return hip_status(fmt == PDAKV_KV_INT8_SYM
                          ? pdakv::launch_decode_int8_multi(a, head_dim, bf16, s)
                          : pdakv::launch_decode_16bit_multi(a, head_dim, bf16, s));
  switch (fmt) {
    case PDAKV_KV_INT8_SYM: return hip_status(pdakv::launch_decode_int8(a, head_dim, bf16, s));
    case PDAKV_KV_INT8_STATIC:
      return hip_status(pdakv::launch_decode_int8_static(a, head_dim, bf16, s));
    default: return hip_status(pdakv::launch_decode_16bit(a, head_dim, bf16, s));
  }
}

int write_common(int fmt, Scales sc, const void* k_src, const void* v_src, int src_dtype,
                 int64_t num_tokens, int num_kv_heads, int head_dim, int64_t kst, int64_t ksh,
                 int64_t ksd, int64_t vst, int64_t vsh, int64_t vsd,
                 const int32_t* slot_mapping, void* kv_pool, int64_t num_blocks, int block_size,
                 int32_t* err_flag, void* stream) {
  int st = check_write(k_src, v_src, src_dtype, num_tokens, num_kv_heads, head_dim, kst, ksh,
                       ksd, vst, vsh, vsd, slot_mapping, kv_pool, num_blocks, block_size);
  if (st != PDAKV_OK) return st;
  if (!valid_scale(sc.k) || !valid_scale(sc.v)) return PDAKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return st;
  if (num_tokens * num_kv_heads / 4 >= INT32_MAX) return PDAKV_ERR_UNSUPPORTED;
  WriteArgs a{};
  a.k = k_src;
  a.v = v_src;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.k_st = kst;
  a.k_sh = ksh;
  a.k_sd = ksd;
  a.v_st = vst;
  a.v_sh = vsh;
  a.v_sd = vsd;
  a.slots = slot_mapping;
  a.pool = static_cast<uint8_t*>(kv_pool);
  a.num_blocks = num_blocks;
  a.page_bytes =
      static_cast<int64_t>(pdakv_page_bytes(fmt, block_size, num_kv_heads, head_dim));
  a.k_scale = sc.k;
  a.v_scale = sc.v;
  a.k_rcp = 1.0f / sc.k;  // IEEE binary32 division, correctly rounded
  a.v_rcp = 1.0f / sc.v;
  a.err = err_flag;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = src_dtype == PDAKV_DTYPE_BF16;
  switch (fmt) {
    case PDAKV_KV_INT8_SYM: return hip_status(pdakv::launch_quant_write_int8(a, head_dim, bf16, s));
    case PDAKV_KV_INT8_STATIC:
      return hip_status(pdakv::launch_quant_write_static(a, head_dim, bf16, s));
    default: return hip_status(pdakv::launch_write_16bit(a, head_dim, s));
  }
}

// The address under which the GPU reaches `p`: p itself for device memory,
// the mapped device address for pinned host memory, nullptr for memory the
// GPU cannot reach (pageable host memory) or an unknown pointer.
void* gpu_address(void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error state the query left
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return p;
  if (at.type == hipMemoryTypeHost) return at.devicePointer;
  return nullptr;
}

int page_copy(void* pool, int64_t num_blocks, int64_t page_bytes, const int32_t* ids,
              int64_t num_pages, void* packed, bool gather, int32_t* err_flag, void* stream) {
  if (num_blocks < 0 || num_pages < 0 || page_bytes <= 0 || page_bytes % 16 != 0)
    return PDAKV_ERR_INVALID_ARG;
  if (num_pages > INT32_MAX) return PDAKV_ERR_UNSUPPORTED;  // one workgroup per page
  if (num_pages == 0) return PDAKV_OK;
  if (!pool || !ids || !packed || !aligned16(pool) || !aligned16(packed))
    return PDAKV_ERR_INVALID_ARG;
  void* far = gpu_address(packed);
  if (!far || !aligned16(far)) return PDAKV_ERR_INVALID_ARG;
  pdakv::PageCopyArgs a{};
  a.pool = static_cast<uint8_t*>(pool);
  a.num_blocks = num_blocks;
  a.page_bytes = page_bytes;
  a.packed = static_cast<uint8_t*>(far);
  a.ids = ids;
  a.num_pages = num_pages;
  a.gather = gather ? 1 : 0;
  a.err = err_flag;
  return hip_status(pdakv::launch_page_copy(a, static_cast<hipStream_t>(stream)));
}

// Scratch of paged_attn_decode_int8_noalloc: the decode workspace (partial
// results and merge records) as a file-scope device array, so that the call
// allocates nothing. Every GPU the library runs on holds its own copy until
// the process ends; in host code `scratch` only names the symbol, its device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[PDAKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (looked up on the device's
// first call, with that device current).
int scratch_address(void** addr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PDAKV_ERR_NO_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) return PDAKV_ERR_NO_DEVICE;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return PDAKV_ERR_HIP;
      }
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return PDAKV_OK;
}

}  // namespace

extern "C" {

int pdakv_version(void) { return 100; /* 0.1.0 */ }

const char* pdakv_status_string(int status) {
  switch (status) {
    case PDAKV_OK: return "ok";
    case PDAKV_ERR_INVALID_ARG: return "invalid argument";
    case PDAKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PDAKV_ERR_DTYPE: return "unsupported dtype";
    case PDAKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PDAKV_ERR_HIP: return "HIP runtime or launch error";
    case PDAKV_ERR_NO_DEVICE: return "no usable HIP device";
    default: return "unknown status";
  }
}

size_t pdakv_page_bytes(int kv_format, int block_size, int num_kv_heads, int head_dim) {
  if (block_size <= 0 || block_size % 4 != 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  const size_t bs = static_cast<size_t>(block_size), d = static_cast<size_t>(head_dim);
  const size_t h = static_cast<size_t>(num_kv_heads);
  if (kv_format == PDAKV_KV_INT8_SYM) return h * (2 * bs * d + 4 * bs);
  if (kv_format == PDAKV_KV_16BIT) return h * 4 * bs * d;
  if (kv_format == PDAKV_KV_INT8_STATIC) return h * 2 * bs * d;
  return 0;
}

int pdakv_capabilities(uint32_t* flags_out) {
  if (!flags_out) return PDAKV_ERR_INVALID_ARG;
  *flags_out = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PDAKV_ERR_NO_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PDAKV_ERR_NO_DEVICE;
  uint32_t f = PDAKV_CAP_HEAD_DIM_64 | PDAKV_CAP_HEAD_DIM_128 | PDAKV_CAP_BLOCK_16 |
               PDAKV_CAP_F16 | PDAKV_CAP_BF16;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) f |= PDAKV_CAP_GFX950;
  *flags_out = f;
  return PDAKV_OK;
}

int pdakv_decode_plan(int kv_format, int num_seqs, int num_kv_heads, int head_dim,
                      int max_context_len, int* num_waves, int* max_pages_per_wave) {
  if (!known_format(kv_format)) return PDAKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0) return PDAKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PDAKV_ERR_UNSUPPORTED;
  if (item_bound(num_seqs, num_kv_heads, max_context_len) > kMaxItems)
    return PDAKV_ERR_UNSUPPORTED;
  const int64_t v = plan_waves(
      format_waves_per_simd(kv_format, head_dim,
                            item_bound(num_seqs, num_kv_heads, max_context_len)),
      num_seqs, num_kv_heads, max_context_len);
  const int64_t p = std::max<int64_t>(
      pdakv::kMinPagesPerWave, ceil_div(item_bound(num_seqs, num_kv_heads, max_context_len), v));
  if (num_waves) *num_waves = static_cast<int>(v);
  if (max_pages_per_wave) *max_pages_per_wave = static_cast<int>(p);
  return PDAKV_OK;
}

size_t pdakv_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                    int head_dim, int max_context_len) {
  return decode_ws_bytes(num_seqs, 1, num_q_heads, num_kv_heads, head_dim, max_context_len);
}

size_t paged_attn_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                         int max_context_len) {
  // the largest workspace over every KV-head count this query-head count
  // allows (num_kv_heads divides num_q_heads, at most 16 query heads each)
  if (num_q_heads <= 0) return 0;
  size_t need = 0;
  for (int hkv = 1; hkv <= num_q_heads; ++hkv) {
    if (num_q_heads % hkv != 0 || num_q_heads / hkv > pdakv::kMaxGroup) continue;
    need = std::max(need, decode_ws_bytes(num_seqs, 1, num_q_heads, hkv, head_dim,
                                          max_context_len));
  }
  return need;
}

size_t pdakv_decode_multi_workspace_bytes(int num_seqs, int num_query_tokens, int num_q_heads,
                                          int num_kv_heads, int head_dim,
                                          int max_context_len) {
  return decode_ws_bytes(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim,
                         max_context_len);
}

int kv_quant_int8_sym_write(const void* k_src, const void* v_src, int src_dtype,
                            int64_t num_tokens, int num_kv_heads, int head_dim,
                            int64_t k_stride_tok, int64_t k_stride_head, int64_t k_stride_dim,
                            int64_t v_stride_tok, int64_t v_stride_head, int64_t v_stride_dim,
                            const int32_t* slot_mapping, void* kv_pool, int64_t num_blocks,
                            int block_size, int32_t* err_flag, void* stream) {
  return write_common(PDAKV_KV_INT8_SYM, Scales{},
                      k_src, v_src, src_dtype, num_tokens, num_kv_heads, head_dim,
                      k_stride_tok, k_stride_head, k_stride_dim, v_stride_tok,
                      v_stride_head, v_stride_dim, slot_mapping, kv_pool, num_blocks,
                      block_size, err_flag, stream);
}

int kv_write_16bit(const void* k_src, const void* v_src, int src_dtype, int64_t num_tokens,
                   int num_kv_heads, int head_dim, int64_t k_stride_tok, int64_t k_stride_head,
                   int64_t k_stride_dim, int64_t v_stride_tok, int64_t v_stride_head,
                   int64_t v_stride_dim, const int32_t* slot_mapping, void* kv_pool,
                   int64_t num_blocks, int block_size, int32_t* err_flag, void* stream) {
  return write_common(PDAKV_KV_16BIT, Scales{},
                      k_src, v_src, src_dtype, num_tokens, num_kv_heads, head_dim,
                      k_stride_tok, k_stride_head, k_stride_dim, v_stride_tok,
                      v_stride_head, v_stride_dim, slot_mapping, kv_pool, num_blocks,
                      block_size, err_flag, stream);
}

int paged_attn_decode_int8(void* out, int out_dtype, int64_t out_stride_seq,
                           int64_t out_stride_head, const void* q, int q_dtype,
                           int64_t q_stride_seq, int64_t q_stride_head, const void* kv_pool,
                           int64_t num_blocks, int block_size, const int32_t* block_tables,
                           int64_t block_table_stride, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_context_len, float sm_scale, void* workspace,
                           size_t workspace_bytes, int32_t* err_flag, void* stream) {
  return decode_common(PDAKV_KV_INT8_SYM, Scales{},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       nullptr, kv_pool, num_blocks, block_size,
                       block_tables, block_table_stride, context_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, max_context_len, sm_scale,
                       workspace, workspace_bytes, err_flag, stream);
}

int paged_attn_decode_int8_noalloc(void* out, int out_dtype, int64_t out_stride_seq,
                                   int64_t out_stride_head, const void* q, int q_dtype,
                                   int64_t q_stride_seq, int64_t q_stride_head,
                                   const void* kv_pool, int64_t num_blocks, int block_size,
                                   const int32_t* block_tables, int64_t block_table_stride,
                                   const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int max_context_len,
                                   float sm_scale, int32_t* err_flag, void* stream) {
  // every host check first, with a stand-in for the scratch (aligned, of the
  // scratch's size): a call whose workspace would exceed the scratch returns
  // PDAKV_ERR_WORKSPACE before anything touches the device
  void* const stand_in = reinterpret_cast<void*>(uintptr_t{256});
  int st = check_decode(out, out_dtype, out_stride_seq, 0, out_stride_head, q, q_dtype,
                        q_stride_seq, 0, q_stride_head, 1, kv_pool, num_blocks, block_size,
                        block_tables, block_table_stride, context_lens, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, max_context_len, sm_scale, stand_in,
                        PDAKV_NOALLOC_SCRATCH_BYTES);
  if (st != PDAKV_OK || num_seqs == 0) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PDAKV_OK) return st;
  return decode_common(PDAKV_KV_INT8_SYM, Scales{},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       nullptr, kv_pool, num_blocks, block_size, block_tables,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, max_context_len, sm_scale, ws, PDAKV_NOALLOC_SCRATCH_BYTES,
                       err_flag, stream);
}

int paged_attn_decode_fp16(void* out, int out_dtype, int64_t out_stride_seq,
                           int64_t out_stride_head, const void* q, int q_dtype,
                           int64_t q_stride_seq, int64_t q_stride_head, const void* kv_pool,
                           int64_t num_blocks, int block_size, const int32_t* block_tables,
                           int64_t block_table_stride, const int32_t* context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int max_context_len, float sm_scale, void* workspace,
                           size_t workspace_bytes, int32_t* err_flag, void* stream) {
  return decode_common(PDAKV_KV_16BIT, Scales{},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       nullptr, kv_pool, num_blocks, block_size,
                       block_tables, block_table_stride, context_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, max_context_len, sm_scale,
                       workspace, workspace_bytes, err_flag, stream);
}

int paged_attn_decode_int8_append(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_head, const void* q,
    int q_dtype, int64_t q_stride_seq, int64_t q_stride_head, const void* k_new,
    const void* v_new, int64_t k_stride_seq, int64_t k_stride_head, int64_t k_stride_dim,
    int64_t v_stride_seq, int64_t v_stride_head, int64_t v_stride_dim, void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream) {
  AppendRows app;
  app.k = k_new;
  app.v = v_new;
  app.kst = k_stride_seq;
  app.ksh = k_stride_head;
  app.ksd = k_stride_dim;
  app.vst = v_stride_seq;
  app.vsh = v_stride_head;
  app.vsd = v_stride_dim;
  return decode_common(PDAKV_KV_INT8_SYM, Scales{},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       &app, kv_pool, num_blocks, block_size,
                       block_tables, block_table_stride, context_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, max_context_len, sm_scale,
                       workspace, workspace_bytes, err_flag, stream);
}

int paged_attn_decode_fp16_append(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_head, const void* q,
    int q_dtype, int64_t q_stride_seq, int64_t q_stride_head, const void* k_new,
    const void* v_new, int64_t k_stride_seq, int64_t k_stride_head, int64_t k_stride_dim,
    int64_t v_stride_seq, int64_t v_stride_head, int64_t v_stride_dim, void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream) {
  AppendRows app;
  app.k = k_new;
  app.v = v_new;
  app.kst = k_stride_seq;
  app.ksh = k_stride_head;
  app.ksd = k_stride_dim;
  app.vst = v_stride_seq;
  app.vsh = v_stride_head;
  app.vsd = v_stride_dim;
  return decode_common(PDAKV_KV_16BIT, Scales{},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       &app, kv_pool, num_blocks,
                       block_size, block_tables, block_table_stride, context_lens,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                       sm_scale, workspace, workspace_bytes, err_flag, stream);
}

int kv_quant_int8_static_write(const void* k_src, const void* v_src, int src_dtype,
                               int64_t num_tokens, int num_kv_heads, int head_dim,
                               int64_t k_stride_tok, int64_t k_stride_head, int64_t k_stride_dim,
                               int64_t v_stride_tok, int64_t v_stride_head, int64_t v_stride_dim,
                               float k_scale, float v_scale, const int32_t* slot_mapping,
                               void* kv_pool, int64_t num_blocks, int block_size,
                               int32_t* err_flag, void* stream) {
  return write_common(PDAKV_KV_INT8_STATIC, Scales{k_scale, v_scale}, k_src, v_src, src_dtype,
                      num_tokens, num_kv_heads, head_dim, k_stride_tok, k_stride_head,
                      k_stride_dim, v_stride_tok, v_stride_head, v_stride_dim, slot_mapping,
                      kv_pool, num_blocks, block_size, err_flag, stream);
}

int paged_attn_decode_int8_static(void* out, int out_dtype, int64_t out_stride_seq,
                                  int64_t out_stride_head, const void* q, int q_dtype,
                                  int64_t q_stride_seq, int64_t q_stride_head,
                                  const void* kv_pool, int64_t num_blocks, int block_size,
                                  const int32_t* block_tables, int64_t block_table_stride,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int max_context_len,
                                  float sm_scale, float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, int32_t* err_flag, void* stream) {
  return decode_common(PDAKV_KV_INT8_STATIC, Scales{k_scale, v_scale},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       nullptr, kv_pool, num_blocks, block_size, block_tables,
                       block_table_stride, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, max_context_len, sm_scale, workspace, workspace_bytes, err_flag,
                       stream);
}

int paged_attn_decode_int8_static_append(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_head, const void* q,
    int q_dtype, int64_t q_stride_seq, int64_t q_stride_head, const void* k_new,
    const void* v_new, int64_t k_stride_seq, int64_t k_stride_head, int64_t k_stride_dim,
    int64_t v_stride_seq, int64_t v_stride_head, int64_t v_stride_dim, void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, float k_scale, float v_scale, void* workspace,
    size_t workspace_bytes, int32_t* err_flag, void* stream) {
  AppendRows app;
  app.k = k_new;
  app.v = v_new;
  app.kst = k_stride_seq;
  app.ksh = k_stride_head;
  app.ksd = k_stride_dim;
  app.vst = v_stride_seq;
  app.vsh = v_stride_head;
  app.vsd = v_stride_dim;
  return decode_common(PDAKV_KV_INT8_STATIC, Scales{k_scale, v_scale},
                       one_token(out, out_dtype, out_stride_seq, out_stride_head, q, q_dtype,
                                 q_stride_seq, q_stride_head),
                       &app, kv_pool, num_blocks, block_size, block_tables, block_table_stride,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       max_context_len, sm_scale, workspace, workspace_bytes, err_flag, stream);
}

int paged_attn_decode_int8_multi(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_tok,
    int64_t out_stride_head, const void* q, int q_dtype, int64_t q_stride_seq,
    int64_t q_stride_tok, int64_t q_stride_head, int num_query_tokens, const void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream) {
  const Rows r{out, out_dtype, out_stride_seq, out_stride_tok, out_stride_head, q,
               q_dtype, q_stride_seq, q_stride_tok, q_stride_head, num_query_tokens, true};
  return decode_common(PDAKV_KV_INT8_SYM, Scales{}, r, nullptr, kv_pool, num_blocks, block_size,
                       block_tables, block_table_stride, context_lens, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, max_context_len, sm_scale, workspace,
                       workspace_bytes, err_flag, stream);
}

int paged_attn_decode_fp16_multi(
    void* out, int out_dtype, int64_t out_stride_seq, int64_t out_stride_tok,
    int64_t out_stride_head, const void* q, int q_dtype, int64_t q_stride_seq,
    int64_t q_stride_tok, int64_t q_stride_head, int num_query_tokens, const void* kv_pool,
    int64_t num_blocks, int block_size, const int32_t* block_tables, int64_t block_table_stride,
    const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
    int max_context_len, float sm_scale, void* workspace, size_t workspace_bytes,
    int32_t* err_flag, void* stream) {
  const Rows r{out, out_dtype, out_stride_seq, out_stride_tok, out_stride_head, q,
               q_dtype, q_stride_seq, q_stride_tok, q_stride_head, num_query_tokens, true};
  return decode_common(PDAKV_KV_16BIT, Scales{}, r, nullptr, kv_pool, num_blocks, block_size,
                       block_tables, block_table_stride, context_lens, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, max_context_len, sm_scale, workspace,
                       workspace_bytes, err_flag, stream);
}

int kv_pages_swap_out(const void* kv_pool, int64_t num_blocks, int64_t page_bytes,
                      const int32_t* block_ids, int64_t num_pages, void* dst, int32_t* err_flag,
                      void* stream) {
  return page_copy(const_cast<void*>(kv_pool), num_blocks, page_bytes, block_ids, num_pages, dst,
                   true, err_flag, stream);
}

int kv_pages_swap_in(const void* src, int64_t num_pages, const int32_t* block_ids, void* kv_pool,
                     int64_t num_blocks, int64_t page_bytes, int32_t* err_flag, void* stream) {
  return page_copy(kv_pool, num_blocks, page_bytes, block_ids, num_pages, const_cast<void*>(src),
                   false, err_flag, stream);
}

int kv_trim_keep_sink(int kv_format, void* kv_pool, int64_t num_blocks, int block_size,
                      int num_kv_heads, int head_dim, const int32_t* block_tables,
                      int64_t block_table_stride, const int32_t* context_lens,
                      const int32_t* trim_lens, int num_seqs, int keep,
                      int32_t* new_context_lens, int32_t* err_flag, void* stream) {
  if (!known_format(kv_format)) return PDAKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_kv_heads <= 0 || num_blocks < 0 || block_table_stride < 0 || keep < 0)
    return PDAKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim) || block_size != pdakv::kBlockSize)
    return PDAKV_ERR_UNSUPPORTED;
  // device indexes: head blocks (block * heads + head) and the grid in int32
  if (num_blocks * num_kv_heads > INT32_MAX) return PDAKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_seqs) * num_kv_heads > INT32_MAX) return PDAKV_ERR_UNSUPPORTED;
  if (block_table_stride * block_size > INT32_MAX) return PDAKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PDAKV_OK;
  if (!kv_pool || !block_tables || !context_lens || !trim_lens || !new_context_lens)
    return PDAKV_ERR_INVALID_ARG;
  if (!aligned16(kv_pool)) return PDAKV_ERR_INVALID_ARG;
  pdakv::TrimArgs a{};
  a.pool = static_cast<uint8_t*>(kv_pool);
  a.num_blocks = num_blocks;
  a.page_bytes =
      static_cast<int64_t>(pdakv_page_bytes(kv_format, block_size, num_kv_heads, head_dim));
  a.bt = block_tables;
  a.bt_stride = block_table_stride;
  a.ctx = context_lens;
  a.trim = trim_lens;
  a.new_ctx = new_context_lens;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.keep = keep;
  a.err = err_flag;
  return hip_status(pdakv::launch_trim_keep_sink(a, kv_format, head_dim,
                                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
