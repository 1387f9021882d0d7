/*
 * pkv.h — C ABI of libpkv: paged-KV FlashAttention (EXTEND and DECODE) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes softmax(S)·V with S = sm_scale·Q·Kᵀ, reading K and V
 * through a two-level paged KV cache, and never writes S to device memory:
 *
 *   - the attention definition and the reason for tiling it (the score
 *     matrix must not live in HBM) follow the FlashAttention part of the
 *     page "FlashAttention: 优化计算过程中的临时显存占用" (§1 and §2);
 *   - the two-level cache follows "Implement Flash Attention Back End in
 *     SGLang – Basics and KV Cache" (KV-cache part) and "Flash Attention
 *     Backend in SGLang: Grundlagen und KV Cache optimal nutzen" (KV-cache
 *     paragraph): req_to_token maps (request row, position) to a KV slot,
 *     and each layer's K pool and V pool map a slot to a row [Hkv, d];
 *   - EXTEND (new tokens appended to a cached prefix, causal) and DECODE
 *     (one new token per request) are the two forward modes of the same
 *     pages;
 *   - the scheduling metadata is computed once per batch and reused by every
 *     layer, as in "SGLang의 FA3 디코드 최적화: get_scheduler_metadata 도입"
 *     (intro and code §1-§3);
 *   - the optional 8-bit decode and extend follow the Sage formula of
 *     "FlashInfer PrimTS, Sage Attention 도입으로 8비트 양자화 및 성능 최적화
 *     달성" (code §1, §4, §5), and the block-sparse decode its block-sparse
 *     mode (README block and the measured cases).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   B          batch (requests in the call), Hq / Hkv query / KV heads,
 *              G = Hq / Hkv (query head h reads KV head h / G), d = head_dim.
 *   seq_lens   int32 [B] device: L_b, the KV length attended by request b,
 *              INCLUDING this step's new tokens (store them with
 *              pkv_kv_store first).
 *   cu_seqlens_q int32 [B+1] device (EXTEND): new-token rows of request b
 *              are q rows [cu[b], cu[b+1]); n_b = cu[b+1]-cu[b], the cached
 *              prefix is p_b = L_b - n_b and new token i sees keys 0..p_b+i.
 *   req_to_token int32 [rows, rtt_stride] device: slot of position j of
 *              request b is req_to_token[row(b) * rtt_stride + j], with
 *              row(b) = req_pool_indices[b] (or b when that pointer is NULL).
 *   pools      K and V pools of ONE layer, [pool_slots, Hkv, d] row-major,
 *              bf16 (or E4M3 bytes on the 8-bit paths; int8 K and E4M3 V
 *              with PKV_SAGE_INT8).
 *   q / out    [T, Hq, d] row-major (T = B in DECODE); out is bf16; lse is
 *              float [T, Hq], natural-log log-sum-exp of the scaled scores
 *              (-inf for a row with no keys), optional (NULL).
 *   stream     a hipStream_t passed as void* (NULL = default stream).
 *
 * Ownership and execution: the caller allocates and frees every buffer; the
 * library allocates no device memory (its code object carries one static
 * scratch array per device, used only by pkv_attn_decode_noalloc).  Its host-side state is the
 * thread-local error text and a mutex-guarded cache, per device and kernel
 * variant, of how many decode work items the device holds at once (an
 * occupancy query made on the first plan for that device and variant),
 * which sets how the decode work is cut: results move by rounding only.
 * Every call validates its host arguments, then enqueues kernels on
 * `stream` and returns without synchronising.  Grids depend only on host arguments, never on device
 * values, so calls can be captured in a HIP graph.
 *
 * Errors: a non-zero pkv_status means nothing was enqueued (PKV_EHIP: a
 * launch failed); pkv_last_error() describes the last failure of the calling
 * thread.  Device-side VALUES are not validated (as the Sage page states for
 * its scales): seq_lens are clamped to [0, max_kv_len], query row ranges to
 * [0, total_q], and slots outside [0, pool_slots) are clamped when read and
 * skipped when written, so bad values give wrong numbers but never an
 * out-of-bounds access.  The one exception is req_pool_indices: the ABI has
 * no row count for req_to_token, so its values must be valid rows.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* malformed argument (NULL, negative size, ...) */
  PKV_EUNSUPPORTED = 2,  /* well formed but not implemented (head_dim, dtype, ...) */
  PKV_EWORKSPACE = 3,    /* workspace or scratch smaller than required */
  PKV_EHIP = 4           /* a HIP launch failed */
} pkv_status;

typedef enum pkv_dtype {
  PKV_BF16 = 0,
  PKV_FP8_E4M3 = 1, /* OCP E4M3FN: 1-4-3, bias 7, largest finite 448 */
  PKV_SAGE_INT8 = 2 /* Sage with INT8 Q and K (two's complement) and E4M3 V: the
                       FlashInfer PrimTS Sage page, code §3 and §4.  DECODE only */
} pkv_dtype;

typedef enum pkv_mode { PKV_DECODE = 0, PKV_EXTEND = 1 } pkv_mode;

/* Plan-time description of the attention problem (cf. the Sage page, code
 * §5: block sizes are fixed when planning, scales are supplied per run). */
typedef struct pkv_params {
  int32_t num_q_heads;  /* Hq >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t page_size;    /* power of two in [1, 256]; informational (reads are per token) */
  int32_t kv_dtype;     /* pkv_dtype; the 8-bit types need head_dim 128 (PKV_FP8_E4M3: q_block 1
                           for EXTEND; PKV_SAGE_INT8: DECODE plans only) */
  int32_t q_block;      /* 8-bit: q rows per sfQ block (DECODE: one row per request; EXTEND: 1); else 0 */
  int32_t k_block;      /* 8-bit: key positions per sfK block, a multiple of 16; else 0 */
  int32_t max_kv_len;   /* upper bound of seq_lens (1 .. 2^30, <= rtt_stride of the run calls) */
  int32_t kv_chunk;     /* DECODE split size in tokens: 0 = automatic, else a multiple of 32 */
  int32_t split_target; /* DECODE automatic mode: waves per call to size splits for; 0 = as many
                           as the current device holds at once (from the kernel's occupancy;
                           256 CUs x 16 when no device is present) */
  int32_t decode_q_len; /* DECODE: new tokens per request, n in [1, 64] (0 means 1).  With n > 1
                           (e.g. verifying n drafted tokens) q and out are [B*n, Hq, d], rows
                           request-major, and new token i of request b attends to keys
                           0 .. L_b - n + i (bottom-right causal, as EXTEND); on the 8-bit path
                           sfq holds one scale per new-token row, [B*n, Hq] */
} pkv_params;

/* Sizes of the plan workspace (written by pkv_plan_metadata, read by the run
 * calls of every layer) and of the per-call scratch (split partials) for a
 * batch of at most `max_batch` requests and `max_total_q` new-token rows.
 * Neither grows with the square of the sequence length.  Host pointers out.
 * With split_target == 0 the DECODE sizes depend on the current device, so
 * size, plan and run on the same device. */
int pkv_workspace_size(const pkv_params* params, int32_t mode, int32_t max_batch,
                       int64_t max_total_q, size_t* workspace_bytes, size_t* scratch_bytes);

/* Once per batch (SGLang get_scheduler_metadata page, code §1-§3 and the
 * "why" part): from seq_lens (and cu_seqlens_q for EXTEND) compute the
 * split-KV / query-tile work list into `workspace` (device, >=
 * workspace_bytes).  One kernel launch; the result is reused unchanged by
 * every layer's pkv_attn_* call with the same batch.  DECODE ignores
 * cu_seqlens_q (may be NULL) and total_q.  DECODE splits are the smallest
 * that keep the work items within what the device runs at once, so a call
 * runs in a single pass. */
int pkv_plan_metadata(const pkv_params* params, int32_t mode, int32_t batch, int64_t total_q,
                      const int32_t* seq_lens, const int32_t* cu_seqlens_q, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Store this step's new K/V rows (KV-cache paragraph of the SGLang pages:
 * the cache is updated inside the forward pass):
 * k_pool[slots[t]] = k_new[t] and v_pool[slots[t]] = v_new[t] for
 * t < num_tokens, each row [Hkv, d] of the params' kv_dtype (bf16; one
 * byte per element on the 8-bit paths: E4M3, or int8 K and E4M3 V for
 * PKV_SAGE_INT8; rows are copied as bytes).  k_new/v_new
 * are [num_tokens, Hkv, d] device buffers; slots int32 [num_tokens] device,
 * distinct.  A slot outside [0, pool_slots) is skipped. */
int pkv_kv_store(const pkv_params* params, void* k_pool, void* v_pool, int64_t pool_slots,
                 const void* k_new, const void* v_new, const int32_t* slots, int64_t num_tokens,
                 void* stream);

/* Block-sparse DECODE, once per batch (block-sparse mode of the FlashInfer
 * PrimTS Sage page: README block and the measured cases at densities 0.125
 * and 0.10).  Request b attends exactly to the keys j < L_b whose block
 * j / block_size is listed in blk_indices[blk_indptr[b] .. blk_indptr[b+1]),
 * one list per request shared by all heads; each list must be strictly
 * ascending (a number outside [0, ceil(L_b / block_size)) selects no key).
 * This call lays the listed blocks end to end and writes, per request, the
 * slot of each of those keys in order (sparse_req_to_token, int32
 * [B, max_kv_len], device, row b = request b), their count V_b
 * (sparse_seq_lens, int32 [B]) and, on the 8-bit path, the sfK of each
 * k_block of them (sparse_sfk, float [B, Hkv, ceil(max_kv_len / k_block)];
 * block_size must be a multiple of k_block; sfk is the full-sequence sfK of
 * pkv_attn_decode).  One launch; the tables serve every layer.  Block-sparse
 * attention is then pkv_plan_metadata(PKV_DECODE, seq_lens =
 * sparse_seq_lens) and pkv_attn_decode(req_to_token = sparse_req_to_token,
 * rtt_stride = max_kv_len, req_pool_indices = NULL, seq_lens =
 * sparse_seq_lens, sfk = sparse_sfk): the softmax over a set of keys does
 * not depend on their order.  block_size: a power of two in [1, 2^20];
 * decode_q_len must be 1; bf16 plans pass sfk = sparse_sfk = NULL.  A list
 * that is not ascending gives unspecified numbers but no out-of-bounds
 * access; empty selections give O = 0 and lse = -inf (v_mean on the 8-bit
 * path). */
int pkv_block_sparse_table(const pkv_params* params, int32_t batch, const int32_t* seq_lens,
                           const int32_t* req_to_token, int64_t rtt_stride, const int32_t* req_pool_indices,
                           const int32_t* blk_indptr, const int32_t* blk_indices, int64_t num_indices,
                           int32_t block_size, const float* sfk, int32_t* sparse_req_to_token,
                           int32_t* sparse_seq_lens, float* sparse_sfk, void* stream);

/* DECODE: one query row per request (q, out: [B, Hq, d]; [B*n, Hq, d] with
 * params->decode_q_len = n).  bf16 path: q and
 * pools bf16, sfq/sfk/sfv/v_mean must be NULL.  8-bit path (kv_dtype ==
 * PKV_FP8_E4M3): q and pools hold E4M3 bytes; kv_dtype == PKV_SAGE_INT8: q
 * and the K pool hold int8 codes (q8·k8 is the exact integer dot product)
 * and the V pool E4M3 bytes.  Both apply the Sage formula:
 * S = sm_scale·sfq[b,h]·sfk[b,g,j/k_block]·(q8·k8), P stored as E4M3 of
 * 448·exp(S - m), O = sfv[b,g,:]·(Σ P8·v8)/(448·l) (+ v_mean[b,g,:]), where l
 * sums the unquantised exp(S - m).  sfq float [B*decode_q_len, Hq], sfk float
 * [B, Hkv, sfk_stride] with sfk_stride = ceil(max_kv_len / k_block), sfv and
 * v_mean float [B, Hkv, d]; v_mean may be NULL.  Scale values are not checked.
 * `workspace` comes from pkv_plan_metadata(PKV_DECODE) for this batch;
 * `scratch` (device, >= scratch_bytes) holds split partials and may be
 * reused by the next call on the same stream. */
int pkv_attn_decode(const pkv_params* params, void* out, float* lse, const void* q,
                    const void* k_pool, const void* v_pool, int64_t pool_slots,
                    const int32_t* req_to_token, int64_t rtt_stride, const int32_t* req_pool_indices,
                    const int32_t* seq_lens, int32_t batch, float sm_scale, const float* sfq,
                    const float* sfk, const float* sfv, const float* v_mean,
                    const void* workspace, size_t workspace_bytes, void* scratch,
                    size_t scratch_bytes, void* stream);

/* Largest split scratch pkv_attn_decode_noalloc can serve (32 MiB). */
#define PKV_STATIC_SCRATCH_BYTES (32ll << 20)

/* DECODE without a scratch buffer, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors are those of
 * pkv_attn_decode, whose kernels it runs; the split partials go to a static
 * device array of PKV_STATIC_SCRATCH_BYTES that the library's code object
 * holds on every GPU it runs on until the process ends (its address is
 * looked up once per device, on the first call with that device current).
 * A decode whose scratch_bytes (pkv_workspace_size) exceeds that size is
 * rejected with PKV_EWORKSPACE.  The call allocates and frees nothing.  Every
 * call on one GPU shares that GPU's array and no part of it needs clearing
 * (the split kernel writes every partial the merge reads), so calls that
 * overlap on one GPU (different streams, or host threads) race and give
 * wrong results: serialise them, e.g. on one stream. */
int pkv_attn_decode_noalloc(const pkv_params* params, void* out, float* lse, const void* q,
                            const void* k_pool, const void* v_pool, int64_t pool_slots,
                            const int32_t* req_to_token, int64_t rtt_stride,
                            const int32_t* req_pool_indices, const int32_t* seq_lens, int32_t batch,
                            float sm_scale, const float* sfq, const float* sfk, const float* sfv,
                            const float* v_mean, const void* workspace, size_t workspace_bytes,
                            void* stream);

/* EXTEND: causal attention of the total_q new-token rows (q: [total_q, Hq, d],
 * out: [total_q, Hq, d] bf16) over their request's cached prefix and
 * themselves.  bf16 path: q and pools bf16, sfq/sfk/sfv/v_mean NULL.  8-bit
 * path (kv_dtype == PKV_FP8_E4M3, q_block == 1): q and pools hold E4M3 bytes
 * and the Sage formula of pkv_attn_decode applies to every row, with sfq
 * float [total_q, Hq] (one scale per row), sfk [B, Hkv, ceil(max_kv_len /
 * k_block)], sfv and v_mean [B, Hkv, d] (v_mean may be NULL); sfq and sfk
 * must be positive (as quantisation scales are; values are not checked); the
 * reference maximum never falls below a score already seen, so no quantised
 * probability exceeds 448.  `workspace`
 * comes from pkv_plan_metadata(PKV_EXTEND) with the same batch and total_q.
 * `scratch` is not used (may be NULL). */
int pkv_attn_extend(const pkv_params* params, void* out, float* lse, const void* q,
                    const void* k_pool, const void* v_pool, int64_t pool_slots,
                    const int32_t* req_to_token, int64_t rtt_stride, const int32_t* req_pool_indices,
                    const int32_t* seq_lens, const int32_t* cu_seqlens_q, int32_t batch,
                    int64_t total_q, float sm_scale, const float* sfq, const float* sfk,
                    const float* sfv, const float* v_mean, const void* workspace,
                    size_t workspace_bytes, void* scratch, size_t scratch_bytes, void* stream);

/* Text of the calling thread's last error ("" if none).  Valid until the
 * thread's next pkv_* call. */
const char* pkv_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PKV_H_ */
