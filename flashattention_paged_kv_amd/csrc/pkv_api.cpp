// C ABI of libpkv: host-side validation, workspace layout and kernel
// launches.  Every entry point validates all host arguments before touching
// HIP, so argument errors are reported without a device; then it enqueues
// its kernels on the caller's stream and returns without synchronising.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PKV_OK;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validation of the plan-time description shared by every entry point.
int check_params(const pkv_params* p, int mode) {
  if (!p) return fail(PKV_EINVAL, "params is NULL");
  if (mode != PKV_DECODE && mode != PKV_EXTEND) return fail(PKV_EINVAL, "mode=%d is not PKV_DECODE or PKV_EXTEND", mode);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(PKV_EINVAL, "num_q_heads=%d and num_kv_heads=%d must be >= 1", p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_q_heads=%d is not a multiple of num_kv_heads=%d", p->num_q_heads, p->num_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim=%d is unsupported (64 or 128)", p->head_dim);
  if (!is_pow2(p->page_size) || p->page_size > 256)
    return fail(PKV_EINVAL, "page_size=%d must be a power of two in [1, 256]", p->page_size);
  if (p->max_kv_len < 1) return fail(PKV_EINVAL, "max_kv_len=%d must be >= 1", p->max_kv_len);
  if (p->max_kv_len > (1 << 30)) return fail(PKV_EUNSUPPORTED, "max_kv_len=%d exceeds 2^30", p->max_kv_len);
  if (p->kv_chunk < 0 || p->kv_chunk % pkv::kDecodeTile != 0)
    return fail(PKV_EINVAL, "kv_chunk=%d must be 0 or a positive multiple of %d", p->kv_chunk, pkv::kDecodeTile);
  if (p->split_target < 0) return fail(PKV_EINVAL, "split_target=%d must be >= 0", p->split_target);
  if (p->decode_q_len < 0 || p->decode_q_len > 64)
    return fail(PKV_EINVAL, "decode_q_len=%d must be in [0, 64]", p->decode_q_len);
  if (p->decode_q_len > 1 && mode != PKV_DECODE)
    return fail(PKV_EINVAL, "decode_q_len applies to DECODE plans only (EXTEND takes cu_seqlens_q)");
  if (p->kv_dtype == PKV_BF16) {
    // block sizes only exist for the 8-bit recipe: reject them like an
    // inapplicable plan input (FlashInfer Sage page, code §2)
    if (p->q_block != 0) return fail(PKV_EINVAL, "q_block is unsupported by a bf16 plan");
    if (p->k_block != 0) return fail(PKV_EINVAL, "k_block is unsupported by a bf16 plan");
  } else if (pkv::is_8bit(*p)) {
    const char* name = p->kv_dtype == PKV_FP8_E4M3 ? "fp8_e4m3" : "sage_int8";
    if (p->head_dim != 128) return fail(PKV_EUNSUPPORTED, "kv_dtype=%s requires head_dim=128", name);
    if (p->kv_dtype == PKV_SAGE_INT8 && mode != PKV_DECODE)
      return fail(PKV_EUNSUPPORTED, "kv_dtype=sage_int8 is a DECODE path (INT8 Q/K decode of the Sage page)");
    if (p->k_block < 16 || p->k_block % 16 != 0)
      return fail(PKV_EINVAL, "k_block=%d must be a positive multiple of 16", p->k_block);
    if (p->q_block < 1) return fail(PKV_EINVAL, "q_block=%d must be >= 1", p->q_block);
    if (mode == PKV_EXTEND && p->q_block != 1)
      return fail(PKV_EUNSUPPORTED, "an fp8_e4m3 extend plan takes one sfQ per row (q_block=1), not q_block=%d",
                  p->q_block);
  } else {
    return fail(PKV_EUNSUPPORTED, "kv_dtype=%d is unsupported", p->kv_dtype);
  }
  if (mode == PKV_EXTEND && p->num_q_heads / p->num_kv_heads > pkv::kExtendRows)
    return fail(PKV_EUNSUPPORTED, "extend supports at most %d query heads per kv head", pkv::kExtendRows);
  return PKV_OK;
}

int64_t elem_bytes(const pkv_params* p) { return pkv::is_8bit(*p) ? 1 : 2; }

// Decode items the current device holds at once for these params (cached per
// device and kernel variant).  Without a device (host-only sizing) the
// library assumes 256 CUs x 16 resident waves.
int64_t resident_items(const pkv_params& p) {
  const int units = (int)pkv::decode_units(p);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    const int wpb = pkv::decode_waves_per_block(units);
    const int64_t blocks = pkv::kFallbackResidentWaves / wpb;
    const int64_t r = blocks / pkv::ceil_div(units, wpb);
    return r > 1 ? r : 1;
  }
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int>, int64_t> cache;
  const auto key = std::make_tuple(dev, (int)p.kv_dtype, p.head_dim, units);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int64_t items = 0;
  hipError_t e = pkv::is_8bit(p) ? pkv::decode_fp8_resident_items(units, p.kv_dtype == PKV_SAGE_INT8, &items)
                                             : pkv::decode_bf16_resident_items(p.head_dim, units, &items);
  if (e != hipSuccess || items < 1) {
    (void)hipGetLastError();
    items = 1;
  }
  std::lock_guard<std::mutex> g(mu);
  cache[key] = items;
  return items;
}

int64_t target_items(const pkv_params& p, int mode) {
  return mode == PKV_DECODE ? pkv::decode_target_items(p, p.split_target > 0 ? 1 : resident_items(p)) : 0;
}

int check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int pkv_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_workspace_size(const pkv_params* params, int32_t mode, int32_t max_batch, int64_t max_total_q,
                       size_t* workspace_bytes, size_t* scratch_bytes) {
  if (int rc = check_params(params, mode)) return rc;
  if (max_batch < 0) return fail(PKV_EINVAL, "max_batch=%d must be >= 0", max_batch);
  if (max_total_q < 0) return fail(PKV_EINVAL, "max_total_q=%lld must be >= 0", (long long)max_total_q);
  if (!workspace_bytes || !scratch_bytes) return fail(PKV_EINVAL, "output pointers must not be NULL");
  const int64_t tgt = target_items(*params, mode);
  const pkv::WsLayout w = pkv::ws_layout(*params, mode, max_batch, max_total_q, tgt);
  *workspace_bytes = (size_t)(w.total_ints * 4);
  *scratch_bytes = mode == PKV_DECODE ? (size_t)pkv::decode_scratch(*params, max_batch, tgt).total_bytes : 0;
  return ok();
}

int pkv_plan_metadata(const pkv_params* params, int32_t mode, int32_t batch, int64_t total_q,
                      const int32_t* seq_lens, const int32_t* cu_seqlens_q, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (int rc = check_params(params, mode)) return rc;
  if (batch < 0) return fail(PKV_EINVAL, "batch=%d must be >= 0", batch);
  if (mode == PKV_EXTEND && total_q < 0) return fail(PKV_EINVAL, "total_q=%lld must be >= 0", (long long)total_q);
  if (!workspace) return fail(PKV_EINVAL, "workspace is NULL");
  if (batch > 0 && !seq_lens) return fail(PKV_EINVAL, "seq_lens is NULL");
  if (mode == PKV_EXTEND && batch > 0 && !cu_seqlens_q) return fail(PKV_EINVAL, "cu_seqlens_q is NULL for an extend plan");
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return fail(PKV_EINVAL, "workspace must be 16-byte aligned");
  const int64_t tq = mode == PKV_EXTEND ? total_q : 0;
  const int64_t tgt = target_items(*params, mode);
  const pkv::WsLayout w = pkv::ws_layout(*params, mode, batch, tq, tgt);
  if ((int64_t)workspace_bytes < w.total_ints * 4)
    return fail(PKV_EWORKSPACE, "workspace_bytes=%zu is smaller than the %lld bytes required", workspace_bytes,
                (long long)(w.total_ints * 4));
  if (w.capacity > INT32_MAX) return fail(PKV_EUNSUPPORTED, "work-item capacity %lld exceeds int32", (long long)w.capacity);
  if (mode == PKV_DECODE && (int64_t)batch * pkv::ceil_div(params->max_kv_len, pkv::decode_plan_tile(*params)) > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "batch=%d x max_kv_len=%d exceeds the plan's int32 tile offsets", batch,
                params->max_kv_len);
  pkv::PlanArgs a{};
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.ws = static_cast<int32_t*>(workspace);
  a.req_off = w.req_off;
  a.items_off = w.items_off;
  a.tmp_off = w.tmp_off;
  a.keys_off = w.keys_off;
  a.capacity = w.capacity;
  a.total_q = tq;
  a.batch = batch;
  a.mode = mode;
  a.max_kv_len = params->max_kv_len;
  a.kv_chunk = params->kv_chunk;
  if (tgt > INT32_MAX) return fail(PKV_EUNSUPPORTED, "split target %lld exceeds int32", (long long)tgt);
  a.target_items = (int32_t)tgt;
  a.block_tokens = pkv::extend_block_tokens(*params);
  a.tile = pkv::decode_plan_tile(*params);
  return check_launch(pkv::launch_plan(a, static_cast<hipStream_t>(stream)), "plan_metadata launch");
}

int pkv_block_sparse_table(const pkv_params* params, int32_t batch, const int32_t* seq_lens,
                           const int32_t* req_to_token, int64_t rtt_stride, const int32_t* req_pool_indices,
                           const int32_t* blk_indptr, const int32_t* blk_indices, int64_t num_indices,
                           int32_t block_size, const float* sfk, int32_t* sparse_req_to_token,
                           int32_t* sparse_seq_lens, float* sparse_sfk, void* stream) {
  if (int rc = check_params(params, PKV_DECODE)) return rc;
  if (batch < 0) return fail(PKV_EINVAL, "batch=%d must be >= 0", batch);
  if (params->decode_q_len > 1)
    return fail(PKV_EUNSUPPORTED, "block-sparse decode takes one new token per request (decode_q_len=%d)",
                params->decode_q_len);
  if (!is_pow2(block_size) || block_size > (1 << 20))
    return fail(PKV_EINVAL, "block_size=%d must be a power of two in [1, 2^20]", block_size);
  if (num_indices < 0 || num_indices > INT32_MAX)
    return fail(PKV_EINVAL, "num_indices=%lld must be in [0, 2^31)", (long long)num_indices);
  if (rtt_stride < params->max_kv_len)
    return fail(PKV_EINVAL, "rtt_stride=%lld is smaller than max_kv_len=%d", (long long)rtt_stride, params->max_kv_len);
  const bool fp8 = pkv::is_8bit(*params);
  if (fp8) {
    if (block_size % params->k_block != 0)
      return fail(PKV_EINVAL, "block_size=%d must be a multiple of k_block=%d", block_size, params->k_block);
    if (batch > 0 && (!sfk || !sparse_sfk)) return fail(PKV_EINVAL, "the 8-bit path needs sfk and sparse_sfk");
  } else if (sfk || sparse_sfk) {
    return fail(PKV_EINVAL, "sfk and sparse_sfk are unsupported by a bf16 plan");
  }
  if (batch == 0) return ok();
  if (!seq_lens || !req_to_token || !blk_indptr || !sparse_req_to_token || !sparse_seq_lens)
    return fail(PKV_EINVAL, "a required pointer (seq_lens, req_to_token, blk_indptr, sparse outputs) is NULL");
  if (num_indices > 0 && !blk_indices) return fail(PKV_EINVAL, "blk_indices is NULL");
  pkv::SparseTableArgs a{};
  a.seq_lens = seq_lens;
  a.rtt = req_to_token;
  a.rpi = req_pool_indices;
  a.indptr = blk_indptr;
  a.indices = blk_indices;
  a.sfk = fp8 ? sfk : nullptr;
  a.out_rtt = sparse_req_to_token;
  a.out_lens = sparse_seq_lens;
  a.out_sfk = fp8 ? sparse_sfk : nullptr;
  a.rtt_stride = rtt_stride;
  a.num_indices = num_indices;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  a.block_shift = shift;
  a.max_kv_len = params->max_kv_len;
  a.hkv = params->num_kv_heads;
  a.k_block = fp8 ? params->k_block : 1;
  a.sfk_stride = fp8 ? (int32_t)pkv::ceil_div(params->max_kv_len, params->k_block) : 0;
  return check_launch(pkv::launch_block_sparse_table(a, batch, static_cast<hipStream_t>(stream)),
                      "block_sparse_table launch");
}

int pkv_kv_store(const pkv_params* params, void* k_pool, void* v_pool, int64_t pool_slots, const void* k_new,
                 const void* v_new, const int32_t* slots, int64_t num_tokens, void* stream) {
  // a plain row copy: the dtype rules of a decode plan cover both pool types
  if (int rc = check_params(params, PKV_DECODE)) return rc;
  if (num_tokens < 0 || num_tokens > INT32_MAX)
    return fail(PKV_EINVAL, "num_tokens=%lld must be in [0, 2^31)", (long long)num_tokens);
  if (pool_slots < 1) return fail(PKV_EINVAL, "pool_slots=%lld must be >= 1", (long long)pool_slots);
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !slots) return fail(PKV_EINVAL, "a pool, new-row or slots pointer is NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_EINVAL, "pools and new rows must be 16-byte aligned");
  const int64_t row_bytes = (int64_t)params->num_kv_heads * params->head_dim * elem_bytes(params);
  return check_launch(pkv::launch_kv_store(k_pool, v_pool, pool_slots, k_new, v_new, slots, num_tokens, row_bytes,
                                           static_cast<hipStream_t>(stream)),
                      "kv_store launch");
}

}  // extern "C"

namespace {

// Shared by pkv_attn_decode (caller's scratch) and pkv_attn_decode_noalloc
// (the static scratch): with static_scratch set, `scratch` is ignored and the
// static array serves if it is large enough.
int attn_decode_impl(const pkv_params* params, void* out, float* lse, const void* q, const void* k_pool,
                     const void* v_pool, int64_t pool_slots, const int32_t* req_to_token, int64_t rtt_stride,
                     const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch, float sm_scale,
                     const float* sfq, const float* sfk, const float* sfv, const float* v_mean,
                     const void* workspace, size_t workspace_bytes, void* scratch, size_t scratch_bytes,
                     bool static_scratch, void* stream) {
  if (int rc = check_params(params, PKV_DECODE)) return rc;
  if (batch < 0) return fail(PKV_EINVAL, "batch=%d must be >= 0", batch);
  if (pool_slots < 1 || pool_slots > ((int64_t)1 << 31))
    return fail(PKV_EINVAL, "pool_slots=%lld must be in [1, 2^31] (slots are int32)", (long long)pool_slots);
  if (rtt_stride < params->max_kv_len)
    return fail(PKV_EINVAL, "rtt_stride=%lld is smaller than max_kv_len=%d", (long long)rtt_stride, params->max_kv_len);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f)) return fail(PKV_EINVAL, "sm_scale must be finite and > 0");
  const bool fp8 = pkv::is_8bit(*params);
  if (!fp8) {
    if (sfq) return fail(PKV_EINVAL, "sfq is unsupported by a bf16 plan");
    if (sfk) return fail(PKV_EINVAL, "sfk is unsupported by a bf16 plan");
    if (sfv) return fail(PKV_EINVAL, "sfv is unsupported by a bf16 plan");
    if (v_mean) return fail(PKV_EINVAL, "v_mean is unsupported by a bf16 plan");
  } else if (batch > 0 && (!sfq || !sfk || !sfv)) {
    return fail(PKV_EINVAL, "the 8-bit decode needs sfq, sfk and sfv");
  }
  if (batch == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !req_to_token || !seq_lens || !workspace)
    return fail(PKV_EINVAL, "a required pointer (out, q, pools, req_to_token, seq_lens, workspace) is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_EINVAL, "out, q and the pools must be 16-byte aligned");
  const int64_t tgt = target_items(*params, PKV_DECODE);
  const pkv::WsLayout w = pkv::ws_layout(*params, PKV_DECODE, batch, 0, tgt);
  if ((int64_t)workspace_bytes < w.total_ints * 4)
    return fail(PKV_EWORKSPACE, "workspace_bytes=%zu is smaller than the %lld bytes required", workspace_bytes,
                (long long)(w.total_ints * 4));
  const pkv::DecodeScratch sc = pkv::decode_scratch(*params, batch, tgt);
  if (static_scratch) {
    if (sc.total_bytes > pkv::kStaticScratchBytes)
      return fail(PKV_EWORKSPACE,
                  "this decode needs %lld bytes of split scratch; the static scratch holds %lld "
                  "(use pkv_attn_decode with a caller buffer)",
                  (long long)sc.total_bytes, (long long)pkv::kStaticScratchBytes);
    void* p = nullptr;
    const hipError_t e = pkv::static_scratch_address(&p);
    if (e != hipSuccess) return fail(PKV_EHIP, "static scratch address: %s", hipGetErrorString(e));
    scratch = p;
    scratch_bytes = (size_t)pkv::kStaticScratchBytes;
  }
  if (!scratch || (int64_t)scratch_bytes < sc.total_bytes)
    return fail(PKV_EWORKSPACE, "scratch_bytes=%zu is smaller than the %lld bytes required", scratch ? scratch_bytes : 0,
                (long long)sc.total_bytes);
  if (!aligned16(scratch)) return fail(PKV_EINVAL, "scratch must be 16-byte aligned");
  const int group = params->num_q_heads / params->num_kv_heads;
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.rtt = req_to_token;
  a.rpi = req_pool_indices;
  a.ws = static_cast<const int32_t*>(workspace);
  a.out = out;
  a.lse = lse;
  a.part_o = static_cast<float*>(scratch);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(scratch) + sc.part_lse_off);
  a.sfq = sfq;
  a.sfk = sfk;
  a.sfv = sfv;
  a.v_mean = v_mean;
  a.rtt_stride = rtt_stride;
  a.pool_slots = pool_slots;
  a.items_off = w.items_off;
  a.req_off = w.req_off;
  a.hq = params->num_q_heads;
  a.hkv = params->num_kv_heads;
  a.seq_lens = seq_lens;
  a.max_kv_len = params->max_kv_len;
  a.q_len = pkv::decode_q_len(*params);
  a.group = group;
  a.head_groups = (int32_t)pkv::ceil_div((int64_t)a.q_len * group, 16);
  a.k_block = params->k_block;
  a.sfk_stride = fp8 ? (int32_t)pkv::ceil_div(params->max_kv_len, params->k_block) : 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  const int64_t units = (int64_t)a.hkv * a.head_groups;
  if (w.capacity * pkv::ceil_div(units, pkv::decode_waves_per_block((int)units)) > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "decode grid of %lld work items x %lld kv-head units exceeds int32",
                (long long)w.capacity, (long long)units);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = fp8 ? pkv::launch_decode_fp8(a, params->kv_dtype == PKV_SAGE_INT8, w.capacity, batch, s)
                     : pkv::launch_decode_bf16(a, params->head_dim, w.capacity, batch, s);
  if (e != hipSuccess) return check_launch(e, "attn_decode launch");
  return check_launch(pkv::launch_decode_merge(a, params->head_dim, w.capacity, batch, s), "attn_decode merge launch");
}

}  // namespace

extern "C" {

int pkv_attn_decode(const pkv_params* params, void* out, float* lse, const void* q, const void* k_pool,
                    const void* v_pool, int64_t pool_slots, const int32_t* req_to_token, int64_t rtt_stride,
                    const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch, float sm_scale,
                    const float* sfq, const float* sfk, const float* sfv, const float* v_mean,
                    const void* workspace, size_t workspace_bytes, void* scratch, size_t scratch_bytes,
                    void* stream) {
  return attn_decode_impl(params, out, lse, q, k_pool, v_pool, pool_slots, req_to_token, rtt_stride,
                          req_pool_indices, seq_lens, batch, sm_scale, sfq, sfk, sfv, v_mean, workspace,
                          workspace_bytes, scratch, scratch_bytes, false, stream);
}

int pkv_attn_decode_noalloc(const pkv_params* params, void* out, float* lse, const void* q, const void* k_pool,
                            const void* v_pool, int64_t pool_slots, const int32_t* req_to_token,
                            int64_t rtt_stride, const int32_t* req_pool_indices, const int32_t* seq_lens,
                            int32_t batch, float sm_scale, const float* sfq, const float* sfk, const float* sfv,
                            const float* v_mean, const void* workspace, size_t workspace_bytes, void* stream) {
  return attn_decode_impl(params, out, lse, q, k_pool, v_pool, pool_slots, req_to_token, rtt_stride,
                          req_pool_indices, seq_lens, batch, sm_scale, sfq, sfk, sfv, v_mean, workspace,
                          workspace_bytes, nullptr, 0, true, stream);
}

int pkv_attn_extend(const pkv_params* params, void* out, float* lse, const void* q, const void* k_pool,
                    const void* v_pool, int64_t pool_slots, const int32_t* req_to_token, int64_t rtt_stride,
                    const int32_t* req_pool_indices, const int32_t* seq_lens, const int32_t* cu_seqlens_q,
                    int32_t batch, int64_t total_q, float sm_scale, const float* sfq, const float* sfk,
                    const float* sfv, const float* v_mean, const void* workspace, size_t workspace_bytes,
                    void* scratch, size_t scratch_bytes, void* stream) {
  (void)scratch;
  (void)scratch_bytes;
  if (int rc = check_params(params, PKV_EXTEND)) return rc;
  const bool fp8 = params->kv_dtype == PKV_FP8_E4M3;
  if (!fp8 && (sfq || sfk || sfv || v_mean))
    return fail(PKV_EINVAL, "sfq, sfk, sfv and v_mean are unsupported by a bf16 plan");
  if (fp8 && batch > 0 && total_q > 0 && (!sfq || !sfk || !sfv))
    return fail(PKV_EINVAL, "the fp8_e4m3 extend needs sfq, sfk and sfv");
  if (batch < 0) return fail(PKV_EINVAL, "batch=%d must be >= 0", batch);
  if (total_q < 0) return fail(PKV_EINVAL, "total_q=%lld must be >= 0", (long long)total_q);
  if (pool_slots < 1 || pool_slots > ((int64_t)1 << 31))
    return fail(PKV_EINVAL, "pool_slots=%lld must be in [1, 2^31] (slots are int32)", (long long)pool_slots);
  if (rtt_stride < params->max_kv_len)
    return fail(PKV_EINVAL, "rtt_stride=%lld is smaller than max_kv_len=%d", (long long)rtt_stride, params->max_kv_len);
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f)) return fail(PKV_EINVAL, "sm_scale must be finite and > 0");
  if (batch == 0 || total_q == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !req_to_token || !seq_lens || !cu_seqlens_q || !workspace)
    return fail(PKV_EINVAL, "a required pointer (out, q, pools, req_to_token, seq_lens, cu_seqlens_q, workspace) is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_EINVAL, "out, q and the pools must be 16-byte aligned");
  const pkv::WsLayout w = pkv::ws_layout(*params, PKV_EXTEND, batch, total_q, 0);
  if ((int64_t)workspace_bytes < w.total_ints * 4)
    return fail(PKV_EWORKSPACE, "workspace_bytes=%zu is smaller than the %lld bytes required", workspace_bytes,
                (long long)(w.total_ints * 4));
  if (w.capacity * params->num_kv_heads > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "extend work items x kv heads (%lld) exceed the grid limit",
                (long long)(w.capacity * params->num_kv_heads));
  pkv::ExtendArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.rtt = req_to_token;
  a.rpi = req_pool_indices;
  a.seq_lens = seq_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.ws = static_cast<const int32_t*>(workspace);
  a.out = out;
  a.lse = lse;
  a.rtt_stride = rtt_stride;
  a.pool_slots = pool_slots;
  a.items_off = w.items_off;
  a.total_q = total_q;
  a.hq = params->num_q_heads;
  a.hkv = params->num_kv_heads;
  a.group = params->num_q_heads / params->num_kv_heads;
  a.block_tokens = pkv::extend_block_tokens(*params);
  a.max_kv_len = params->max_kv_len;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.sfq = sfq;
  a.sfk = sfk;
  a.sfv = sfv;
  a.v_mean = v_mean;
  a.k_block = params->k_block;
  a.sfk_stride = fp8 ? (int32_t)pkv::ceil_div(params->max_kv_len, params->k_block) : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return check_launch(fp8 ? pkv::launch_extend_fp8(a, w.capacity, s)
                          : pkv::launch_extend_bf16(a, params->head_dim, w.capacity, s),
                      "attn_extend launch");
}

}  // extern "C"
