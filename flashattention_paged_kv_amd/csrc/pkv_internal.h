// Internal declarations shared by the libpkv translation units: workspace
// layout, kernel argument blocks and device helpers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// ---------------------------------------------------------------- constants
constexpr int kDecodeTile = 32;       // decode tokens per inner step (two 16-token MFMA blocks)
// Resident decode waves assumed when no device can be queried (256 CUs x 16).
constexpr int kFallbackResidentWaves = 4096;
constexpr int64_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;  // static decode scratch per device
constexpr int kExtendRows = 256;      // (head, token) rows per extend work item (8 waves x 32)
constexpr int kExtendTileN = 64;      // keys per extend inner step
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsSortMax = 4096; // extend items sorted in LDS (32 KiB) up to this count

// Workspace header words (int32).
enum : int {
  WS_MODE = 0,
  WS_BATCH = 1,
  WS_NUM_ITEMS = 2,
  WS_CAPACITY = 3,
  WS_CHUNK = 4,  // decode: chunk tiles; extend: block tokens
  WS_TARGET = 5, // decode: the item count the chunk was sized for
  WS_NCHUNKS = 6,    // decode: chunks (workgroups) of request segments
  WS_CHUNK_TAB = 7,  // decode: word offset of the chunk -> first segment table [NCHUNKS+1], 0 = one segment each
  WS_HEADER_INTS = 16
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Layout of the plan workspace, in int32 words from its start.
struct WsLayout {
  int64_t req_off = WS_HEADER_INTS;  // [B+1] split / tile offsets
  int64_t items_off = 0;             // [cap][4] work items
  int64_t tmp_off = 0;               // extend: unsorted items [cap][4]
  int64_t keys_off = 0;              // u64 sort keys [pow2(cap)] (8-byte aligned)
  int64_t total_ints = 0;
  int64_t capacity = 0;
};

inline int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

// New tokens per request in a decode call (1 unless several are verified at once).
inline int decode_q_len(const pkv_params& p) { return p.decode_q_len > 1 ? p.decode_q_len : 1; }

// Decode work units per split: one per (kv head, group of up to 16 of its
// (new token, query head) columns).
inline int64_t decode_units(const pkv_params& p) {
  return (int64_t)p.num_kv_heads * ceil_div((int64_t)decode_q_len(p) * (p.num_q_heads / p.num_kv_heads), 16);
}

// Split items the automatic chunk is sized for: by default the number of
// items whose waves the device holds at once (`resident_items`, from the
// decode kernel's occupancy), so a launch runs in one pass with no tail of
// late waves; a positive split_target asks for ceil(split_target / units).
inline int64_t decode_target_items(const pkv_params& p, int64_t resident_items) {
  const int64_t t = p.split_target > 0 ? ceil_div(p.split_target, decode_units(p)) : resident_items;
  return t > 1 ? t : 1;
}

// Granularity of the automatic decode chunks: the decode kernel's tile (32
// tokens for bf16 K/V, 64 for 8-bit), so segment bounds inside a request fall
// on tile bounds and no tile is cut short except at a request's end.
inline bool is_8bit(const pkv_params& p) { return p.kv_dtype == PKV_FP8_E4M3 || p.kv_dtype == PKV_SAGE_INT8; }
inline int decode_plan_tile(const pkv_params& p) { return is_8bit(p) ? 64 : kDecodeTile; }

inline int64_t decode_capacity(const pkv_params& p, int64_t batch, int64_t target_items) {
  const int64_t tile = decode_plan_tile(p);
  const int64_t max_tiles = ceil_div(p.max_kv_len, tile) > 0 ? ceil_div(p.max_kv_len, tile) : 1;
  if (p.kv_chunk > 0) {
    int64_t per = ceil_div(p.max_kv_len, p.kv_chunk);
    return batch * (per > 0 ? per : 1);
  }
  // balanced chunks: at most target_items chunks, and every chunk boundary
  // inside a request adds one segment; a request never has more segments
  // than tiles
  const int64_t a = target_items + batch, b = batch * max_tiles;
  return a < b ? a : b;
}

inline int extend_block_tokens(const pkv_params& p) {
  int group = p.num_q_heads / p.num_kv_heads;
  int bt = kExtendRows / group;
  return bt > 0 ? bt : 1;
}

inline int64_t extend_capacity(const pkv_params& p, int64_t batch, int64_t total_q) {
  return ceil_div(total_q, extend_block_tokens(p)) + batch;
}

inline WsLayout ws_layout(const pkv_params& p, int mode, int64_t batch, int64_t total_q, int64_t target_items) {
  WsLayout w;
  w.req_off = WS_HEADER_INTS;
  w.items_off = align_up(w.req_off + batch + 1, 4);
  w.capacity = mode == PKV_DECODE ? decode_capacity(p, batch, target_items) : extend_capacity(p, batch, total_q);
  w.tmp_off = w.items_off + 4 * w.capacity;
  w.keys_off = align_up(w.tmp_off + 4 * w.capacity, 2);
  w.total_ints = w.keys_off + 2 * next_pow2(w.capacity > 0 ? w.capacity : 1);
  return w;
}

// Decode scratch: split partials, fp32.
struct DecodeScratch {
  int64_t part_o_bytes = 0;
  int64_t part_lse_off = 0;
  int64_t total_bytes = 0;
};

inline DecodeScratch decode_scratch(const pkv_params& p, int64_t batch, int64_t target_items) {
  DecodeScratch s;
  const int64_t cap = decode_capacity(p, batch, target_items);
  const int64_t rows = (int64_t)decode_q_len(p) * p.num_q_heads;  // partial rows per split
  s.part_o_bytes = align_up(cap * rows * p.head_dim * (int64_t)sizeof(float), 256);
  s.part_lse_off = s.part_o_bytes;
  s.total_bytes = s.part_o_bytes + align_up(cap * rows * (int64_t)sizeof(float), 256);
  return s;
}

// ---------------------------------------------------------------- kernel args
struct PlanArgs {
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  int32_t* ws;
  int64_t req_off, items_off, tmp_off, keys_off;
  int64_t capacity;
  int64_t total_q;
  int32_t batch;
  int32_t mode;
  int32_t max_kv_len;
  int32_t kv_chunk;
  int32_t target_items;
  int32_t block_tokens;
  int32_t tile;  // decode, automatic chunks: tokens per tile
};

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* rtt;
  const int32_t* rpi;
  const int32_t* ws;
  void* out;
  float* lse;
  float* part_o;
  float* part_lse;
  const float* sfq;
  const float* sfk;
  const float* sfv;
  const float* v_mean;
  int64_t rtt_stride;
  int64_t pool_slots;
  int64_t items_off;
  int64_t req_off;
  const int32_t* seq_lens;
  int32_t max_kv_len;
  int32_t q_len;  // new tokens per request (1 for ordinary decode)
  int32_t hq, hkv, group, head_groups;  // head_groups: 16-column groups of q_len * group per kv head
  int32_t k_block, sfk_stride;
  float scale_log2;  // sm_scale * log2(e)
};

struct ExtendArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* rtt;
  const int32_t* rpi;
  const int32_t* seq_lens;
  const int32_t* cu_seqlens_q;
  const int32_t* ws;
  void* out;
  float* lse;
  int64_t rtt_stride;
  int64_t pool_slots;
  int64_t items_off;
  int64_t total_q;
  int32_t hq, hkv, group, block_tokens;
  int32_t max_kv_len;
  float scale_log2;
  // 8-bit path only
  const float* sfq;
  const float* sfk;
  const float* sfv;
  const float* v_mean;
  int32_t k_block, sfk_stride;
};

// Block-sparse decode: compacted page table of the listed KV blocks.
constexpr int kSparseSplit = 16;  // workgroups per request
struct SparseTableArgs {
  const int32_t* seq_lens;
  const int32_t* rtt;
  const int32_t* rpi;
  const int32_t* indptr;   // [batch + 1]
  const int32_t* indices;  // [num_indices], ascending per request
  const float* sfk;        // 8-bit: [batch, hkv, sfk_stride]; else NULL
  int32_t* out_rtt;        // [batch, max_kv_len]
  int32_t* out_lens;       // [batch]
  float* out_sfk;          // 8-bit: [batch, hkv, sfk_stride]; else NULL
  int64_t rtt_stride, num_indices;
  int32_t block_shift, max_kv_len, hkv, k_block, sfk_stride;
};

// ---------------------------------------------------------------- launchers
hipError_t launch_block_sparse_table(const SparseTableArgs& a, int32_t batch, hipStream_t s);
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// Device address of the static decode scratch on the current device (looked
// up on the first call per device).
hipError_t static_scratch_address(void** ptr);
hipError_t launch_extend_fp8(const ExtendArgs& a, int64_t capacity, hipStream_t s);
hipError_t launch_kv_store(void* k_pool, void* v_pool, int64_t pool_slots, const void* k_new,
                           const void* v_new, const int32_t* slots, int64_t num_tokens,
                           int64_t row_bytes, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, int head_dim, int64_t capacity, int32_t batch,
                              hipStream_t s);
// qk_int8: Q and K hold int8 codes (PKV_SAGE_INT8), else E4M3 bytes.
hipError_t launch_decode_fp8(const DecodeArgs& a, bool qk_int8, int64_t capacity, int32_t batch, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, int64_t capacity, int32_t batch,
                               hipStream_t s);
// Work items (all their waves) of a decode launch that the current device
// holds at once, from the kernel's occupancy and the CU count.
hipError_t decode_bf16_resident_items(int head_dim, int units, int64_t* items);
hipError_t decode_fp8_resident_items(int units, bool qk_int8, int64_t* items);
hipError_t resident_items_of(const void* kernel, int wpb, int units, int64_t* items);
// Waves per workgroup the decode launchers use for `units` waves per item.
inline int decode_waves_per_block(int units) { return units >= 8 ? 8 : (units >= 4 ? 4 : (units >= 2 ? 2 : 1)); }
// The decode kernels read K/V with non-temporal loads when at most two
// workgroups cover the kv heads of a token (up to 16 (kv head, head group)
// units).  Measured on MI355X: 7-12% faster split kernels for 8 and 16 kv
// heads; with 40 kv heads (five workgroups per token) the same loads gained
// nothing on the dense decode and lost 5% on the 8-bit block-sparse one.
inline bool decode_streams(int units) { return units <= 2 * decode_waves_per_block(units); }
hipError_t launch_extend_bf16(const ExtendArgs& a, int head_dim, int64_t capacity, hipStream_t s);

}  // namespace pkv
