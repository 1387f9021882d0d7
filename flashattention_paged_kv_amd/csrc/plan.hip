// Once-per-batch scheduling metadata (split-KV decode items, query-tile
// extend items).  The metadata depends only on seq_lens (and cu_seqlens_q),
// never on slot values, and is reused unchanged by every layer of the batch,
// as the sglang get_scheduler_metadata analysis describes (intro, code §1-3).
//
// One workgroup of 1024 threads: block reductions / scans over the requests,
// then an item table written in parallel.
//
// Decode: the automatic chunk is the smallest number of 32-token tiles for
// which the batch splits into at most target_items items (the items whose
// waves the device holds at once), found by bisection over the chunk size;
// the launch then runs in one pass.  Items stay in request order unless they
// exceed that count (many short requests, or a fixed kv_chunk), in which case
// they are ordered longest first so the short ones fill the tail.
// Extend: items are ordered by causal KV range, longest first.
// Ordering is a bitonic sort on (length, index) keys, in LDS up to
// kPlanLdsSortMax items and in the workspace's key area beyond that.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int64_t u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Exclusive scan of one value per thread across the block; returns the
// thread's exclusive prefix and writes the block total to *total.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* sh /*[16]*/, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  int64_t inc = wave_inclusive_scan(v);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t run = 0;
    for (int w = 0; w < nwaves; ++w) {
      int64_t t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[16] = run;
  }
  __syncthreads();
  int64_t ex = sh[wave] + inc - v;
  *total = sh[16];
  __syncthreads();
  return ex;
}

__device__ int64_t block_max(int64_t v, int64_t* sh /*[17]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    int64_t u = __shfl_xor(v, off, 64);
    v = u > v ? u : v;
  }
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t m = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = sh[w] > m ? sh[w] : m;
    sh[16] = m;
  }
  __syncthreads();
  const int64_t r = sh[16];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int clamp_len(int L, int max_kv_len) {
  return L < 0 ? 0 : (L > max_kv_len ? max_kv_len : L);
}

// Index b with req[b] <= i < req[b+1] (req non-decreasing, req[0] = 0).
__device__ __forceinline__ int find_request(const int32_t* req, int batch, int64_t i) {
  int lo = 0, hi = batch;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (req[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int sort_size(int64_t num) {
  return (int)(num <= 1 ? 1 : (1ll << (64 - __builtin_clzll((unsigned long long)(num - 1)))));
}

template <typename Ptr>
__device__ void bitonic_sort_u64(Ptr a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t x = a[i], y = a[ixj];
          bool up = (i & k) == 0;
          if ((x > y) == up) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int64_t sh[17];
  __shared__ uint64_t keys_lds[kPlanLdsSortMax];
  int32_t* ws = a.ws;
  int32_t* req = ws + a.req_off;
  int4* items = reinterpret_cast<int4*>(ws + a.items_off);
  const int B = a.batch;
  int64_t carry = 0;

  if (a.mode == PKV_DECODE) {
    // 1. total and largest tile counts
    int64_t my_tiles = 0, my_max = 0;
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      const int64_t t = (clamp_len(a.seq_lens[b], a.max_kv_len) + kDecodeTile - 1) / kDecodeTile;
      my_tiles += t;
      my_max = t > my_max ? t : my_max;
    }
    int64_t total_tiles;
    (void)block_exclusive_scan(my_tiles, sh, &total_tiles);
    const int64_t max_tiles = block_max(my_max, sh);
    // items the batch splits into for a chunk of c tiles (a request has >= 1)
    auto count_items = [&](int64_t c) {
      int64_t mine = 0;
      for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int64_t t = (clamp_len(a.seq_lens[b], a.max_kv_len) + kDecodeTile - 1) / kDecodeTile;
        const int64_t n = (t + c - 1) / c;
        mine += n < 1 ? 1 : n;
      }
      int64_t tot;
      (void)block_exclusive_scan(mine, sh, &tot);
      return tot;
    };
    int64_t chunk;
    if (a.kv_chunk > 0) {
      chunk = a.kv_chunk / kDecodeTile;
    } else {
      // smallest chunk with count_items(chunk) <= target (count is non-increasing
      // in the chunk; at max_tiles every request is one item)
      const int64_t T = a.target_items;
      int64_t hi = max_tiles > 0 ? max_tiles : 1;
      int64_t lo = (total_tiles + T - 1) / T;
      lo = lo < 1 ? 1 : (lo > hi ? hi : lo);
      if (count_items(hi) > T) {
        chunk = hi;
      } else {
        while (lo < hi) {  // block-uniform: every bound comes from a block total
          const int64_t mid = (lo + hi) >> 1;
          if (count_items(mid) <= T) hi = mid; else lo = mid + 1;
        }
        chunk = lo;
      }
    }
    // 2. splits per request, exclusive scan -> req[]
    for (int base = 0; base < B; base += blockDim.x) {
      int b = base + threadIdx.x;
      int64_t splits = 0;
      if (b < B) {
        int64_t tiles = (clamp_len(a.seq_lens[b], a.max_kv_len) + kDecodeTile - 1) / kDecodeTile;
        splits = (tiles + chunk - 1) / chunk;
        if (splits < 1) splits = 1;
      }
      int64_t tot;
      int64_t ex = block_exclusive_scan(splits, sh, &tot);
      if (b < B) req[b] = (int32_t)(carry + ex);
      carry += tot;
    }
    if (threadIdx.x == 0) req[B] = (int32_t)carry;
    const int64_t num = carry < a.capacity ? carry : a.capacity;
    __threadfence_block();
    __syncthreads();
    // 3. items (b, kv_begin, kv_end, partial index), created request-major;
    //    the partial index of split s of request b is req[b] + s.  Sorted
    //    (through tmp) only when they overflow the target.
    const bool sorted = num > a.target_items;
    int4* tmp = reinterpret_cast<int4*>(ws + (sorted ? a.tmp_off : a.items_off));
    const int n2 = sorted ? sort_size(num) : (int)num;
    const bool in_lds = n2 <= kPlanLdsSortMax;
    uint64_t* keys_g = reinterpret_cast<uint64_t*>(ws + a.keys_off);
    for (int64_t i = threadIdx.x; i < n2; i += blockDim.x) {
      uint64_t key = ~0ull;
      if (i < num) {
        int b = find_request(req, B, i);
        int s = (int)(i - req[b]);
        int n = req[b + 1] - req[b];
        int L = clamp_len(a.seq_lens[b], a.max_kv_len);
        int tiles = (L + kDecodeTile - 1) / kDecodeTile;
        int t0 = (int)(((int64_t)s * tiles) / n);
        int t1 = (int)(((int64_t)(s + 1) * tiles) / n);
        int kb = t0 * kDecodeTile;
        int ke = t1 * kDecodeTile < L ? t1 * kDecodeTile : L;
        tmp[i] = make_int4(b, kb, ke, n > 1 ? (int)i : -1);
        key = ((uint64_t)(uint32_t)(0x7fffffff - (ke - kb)) << 32) | (uint64_t)i;  // longest split first
      }
      if (!sorted) continue;
      if (in_lds) keys_lds[i] = key; else keys_g[i] = key;
    }
    if (sorted) {
      __threadfence_block();
      __syncthreads();
      if (in_lds) bitonic_sort_u64(keys_lds, n2);
      else bitonic_sort_u64(keys_g, n2);
      for (int64_t j = threadIdx.x; j < num; j += blockDim.x) {
        uint64_t key = in_lds ? keys_lds[j] : keys_g[j];
        items[j] = tmp[(uint32_t)(key & 0xffffffffu)];
      }
    }
    if (threadIdx.x == 0) {
      ws[WS_MODE] = PKV_DECODE;
      ws[WS_BATCH] = B;
      ws[WS_NUM_ITEMS] = (int32_t)num;
      ws[WS_CAPACITY] = (int32_t)a.capacity;
      ws[WS_CHUNK] = (int32_t)chunk;
      ws[WS_TARGET] = a.target_items;
    }
    return;
  }

  // ---------------------------------------------------------------- extend
  const int bt = a.block_tokens;
  for (int base = 0; base < B; base += blockDim.x) {
    int b = base + threadIdx.x;
    int64_t tiles = 0;
    if (b < B) {
      int64_t q0 = a.cu_seqlens_q[b], q1 = a.cu_seqlens_q[b + 1];
      q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
      q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
      tiles = (q1 - q0 + bt - 1) / bt;
    }
    int64_t tot;
    int64_t ex = block_exclusive_scan(tiles, sh, &tot);
    if (b < B) req[b] = (int32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) req[B] = (int32_t)carry;
  const int64_t num = carry < a.capacity ? carry : a.capacity;
  __threadfence_block();
  __syncthreads();
  int4* tmp = reinterpret_cast<int4*>(ws + a.tmp_off);
  const int n2 = sort_size(num);
  const bool in_lds = n2 <= kPlanLdsSortMax;
  uint64_t* keys_g = reinterpret_cast<uint64_t*>(ws + a.keys_off);
  for (int64_t i = threadIdx.x; i < n2; i += blockDim.x) {
    uint64_t key = ~0ull;
    if (i < num) {
      int b = find_request(req, B, i);
      int t = (int)(i - req[b]);
      int64_t q0 = a.cu_seqlens_q[b], q1 = a.cu_seqlens_q[b + 1];
      q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
      q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
      int n = (int)(q1 - q0);
      int L = clamp_len(a.seq_lens[b], a.max_kv_len);
      int p = L - n;
      int end_row = (t + 1) * bt < n ? (t + 1) * bt : n;
      int kv_end = p + end_row;
      kv_end = kv_end < 0 ? 0 : (kv_end > L ? L : kv_end);
      tmp[i] = make_int4(b, t, kv_end, (int)(q0 + (int64_t)t * bt));
      key = ((uint64_t)(uint32_t)(0x7fffffff - kv_end) << 32) | (uint64_t)i;
    }
    if (in_lds) keys_lds[i] = key; else keys_g[i] = key;
  }
  __threadfence_block();
  __syncthreads();
  if (in_lds) bitonic_sort_u64(keys_lds, n2);
  else bitonic_sort_u64(keys_g, n2);
  for (int64_t j = threadIdx.x; j < num; j += blockDim.x) {
    uint64_t key = in_lds ? keys_lds[j] : keys_g[j];
    items[j] = tmp[(uint32_t)(key & 0xffffffffu)];
  }
  if (threadIdx.x == 0) {
    ws[WS_MODE] = PKV_EXTEND;
    ws[WS_BATCH] = B;
    ws[WS_NUM_ITEMS] = (int32_t)num;
    ws[WS_CAPACITY] = (int32_t)a.capacity;
    ws[WS_CHUNK] = bt;
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
