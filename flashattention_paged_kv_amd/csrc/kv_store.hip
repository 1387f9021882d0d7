// Store new tokens' K/V rows into their slots of one layer's pools (the
// cache update inside the forward pass of the SGLang KV-cache pages).  A row
// is Hkv*d elements of the pool's type, moved as 16-byte vectors; the slot
// index is read once per vector, writes to slots outside the pool are skipped.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_store_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                                                       int64_t pool_slots, const u32x4* __restrict__ k_new,
                                                       const u32x4* __restrict__ v_new,
                                                       const int32_t* __restrict__ slots, int64_t num_tokens,
                                                       int64_t row_vecs) {
  const int64_t per_pool = num_tokens * row_vecs;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * per_pool; i += stride) {
    const bool is_v = i >= per_pool;
    const int64_t k = is_v ? i - per_pool : i;
    const int64_t t = k / row_vecs;
    const int64_t c = k - t * row_vecs;
    const int s = slots[t];
    if ((uint32_t)s >= (uint64_t)pool_slots) continue;
    const u32x4 v = is_v ? v_new[k] : k_new[k];
    u32x4* dst = is_v ? v_pool : k_pool;
    dst[(int64_t)s * row_vecs + c] = v;
  }
}

hipError_t launch_kv_store(void* k_pool, void* v_pool, int64_t pool_slots, const void* k_new,
                           const void* v_new, const int32_t* slots, int64_t num_tokens,
                           int64_t row_bytes, hipStream_t s) {
  const int64_t row_vecs = row_bytes / 16;
  const int64_t work = 2 * num_tokens * row_vecs;
  int64_t blocks = ceil_div(work, 256);
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(k_pool), reinterpret_cast<u32x4*>(v_pool), pool_slots,
                     reinterpret_cast<const u32x4*>(k_new), reinterpret_cast<const u32x4*>(v_new), slots,
                     num_tokens, row_vecs);
  return hipGetLastError();
}

}  // namespace pkv
