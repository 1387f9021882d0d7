// Store new tokens' K/V rows into their slots of one layer's pools (the
// cache update inside the forward pass of the SGLang KV-cache pages).  A row
// is Hkv*d elements of the pool's type, moved as 16-byte vectors; writes to
// slots outside the pool are skipped.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// Workgroup (token t, pool): one slot read, uniform across the workgroup, then
// the row's 16-byte vectors; no per-element index arithmetic.
__global__ __launch_bounds__(256) void kv_store_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                                                       int64_t pool_slots, const u32x4* __restrict__ k_new,
                                                       const u32x4* __restrict__ v_new,
                                                       const int32_t* __restrict__ slots, int row_vecs) {
  const int64_t t = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const u32x4* src = (is_v ? v_new : k_new) + t * row_vecs;
  // the first vector is requested together with the slot, not after it
  const int c0 = threadIdx.x;
  const u32x4 first = c0 < row_vecs ? src[c0] : u32x4{0u, 0u, 0u, 0u};
  const int s = __builtin_amdgcn_readfirstlane(slots[t]);
  if ((uint32_t)s >= (uint64_t)pool_slots) return;
  u32x4* dst = (is_v ? v_pool : k_pool) + (int64_t)s * row_vecs;
  if (c0 < row_vecs) dst[c0] = first;
  for (int c = c0 + blockDim.x; c < row_vecs; c += blockDim.x) dst[c] = src[c];
}

hipError_t launch_kv_store(void* k_pool, void* v_pool, int64_t pool_slots, const void* k_new,
                           const void* v_new, const int32_t* slots, int64_t num_tokens,
                           int64_t row_bytes, hipStream_t s) {
  const int64_t row_vecs = row_bytes / 16;
  if (num_tokens < 1 || row_vecs < 1) return hipSuccess;
  const int threads = row_vecs >= 256 ? 256 : (int)((row_vecs + 63) / 64 * 64);
  hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)num_tokens, 2), dim3(threads), 0, s,
                     reinterpret_cast<u32x4*>(k_pool), reinterpret_cast<u32x4*>(v_pool), pool_slots,
                     reinterpret_cast<const u32x4*>(k_new), reinterpret_cast<const u32x4*>(v_new), slots,
                     (int)row_vecs);
  return hipGetLastError();
}

}  // namespace pkv
