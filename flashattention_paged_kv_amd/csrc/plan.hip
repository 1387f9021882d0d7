// Once-per-batch scheduling metadata (split-KV decode items, query-tile
// extend items).  The metadata depends only on seq_lens (and cu_seqlens_q),
// never on slot values, and is reused unchanged by every layer of the batch,
// as the sglang get_scheduler_metadata analysis describes (intro, code §1-3).
//
// One workgroup of 1024 threads: block reductions / scans over the requests,
// then an item table written in parallel.
//
// Decode, automatic: the requests' tiles, laid end to end, are cut
// into at most target_items equal chunks (target_items = the items whose
// waves the device holds at once), so the launch runs in one pass and every
// workgroup streams the same amount of KV.  A chunk is a short list of
// request segments; a request cut by chunk boundaries writes split partials
// that the merge combines.  Decode with a fixed kv_chunk: one item per split,
// ordered longest first when there are more than target_items.
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

__device__ __forceinline__ int clamp_len(int L, int max_kv_len) {
  return L < 0 ? 0 : (L > max_kv_len ? max_kv_len : L);
}

__device__ __forceinline__ int wave_inclusive_scan32(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// LDS words the one-wave decode plan keeps per batch ahead of its chunk table,
// and the most segments per request for which each lane writes its own
// request's segments (beyond it the segments are spread over the lanes).
constexpr int kOneWaveReqWords = 4 * 65;
constexpr int kOneWaveLaneSegs = 8;

// Whether the one-wave decode plan below applies (decided on the host too).
__host__ __device__ __forceinline__ bool plan_decode_by_one_wave(const PlanArgs& a) {
  return a.mode == PKV_DECODE && a.kv_chunk == 0 && a.batch <= 64 &&
         a.capacity + 1 + kOneWaveReqWords <= 2 * (int64_t)kPlanLdsSortMax;
}

// Balanced decode chunks for at most 64 requests, by one wave (one lane per
// request for the scans; the segments written by their request's lane, or
// spread over all lanes when a request has many; 32-bit arithmetic, no
// workgroup barrier): the same work list, offsets and chunk table as the
// workgroup path below.  LDS holds the requests' segment offsets, tile
// offsets, tile counts and lengths (4 x 65 words) and then the chunk table
// (nchunks + 1 <= capacity + 1 entries): every segment lowers its chunk's
// entry to its own index, so an entry ends as the chunk's first segment (num
// where no segment was kept).
__device__ void plan_decode_one_wave(const PlanArgs& a, int32_t* lds) {
  int32_t* const first_l = lds;
  int32_t* const o_l = lds + 65;
  int32_t* const t_l = lds + 130;
  int32_t* const len_l = lds + 195;
  int32_t* const tab_lds = lds + kOneWaveReqWords;
  int32_t* ws = a.ws;
  int32_t* req = ws + a.req_off;
  int4* items = reinterpret_cast<int4*>(ws + a.items_off);
  int32_t* goff = ws + a.tmp_off;  // [B+1] global tile offset of each request
  int32_t* tab = goff + a.batch + 1;
  const int B = a.batch, b = threadIdx.x;
  const bool on = b < B;
  const int L = on ? clamp_len(a.seq_lens[b], a.max_kv_len) : 0;
  const int t = on ? L / a.tile + (L % a.tile != 0) : 0;
  const int o = wave_inclusive_scan32(t) - t;  // the host keeps the batch's tiles below 2^31
  const int T = __shfl(o + t, 63, 64);
  const int C = T > a.target_items ? (int)(((int64_t)T + a.target_items - 1) / a.target_items) : 1;
  const int nchunks = T > C ? (int)(((int64_t)T + C - 1) / C) : 1;
  const int nseg = on ? (t == 0 ? 1 : (o + t - 1) / C - o / C + 1) : 0;
  const int first = wave_inclusive_scan32(nseg) - nseg;
  const int total = __shfl(first + nseg, 63, 64);
  const int num = total < a.capacity ? total : (int)a.capacity;
  if (on) {
    goff[b] = o;
    req[b] = first;
  }
  if (b == 0) {
    goff[B] = T;
    req[B] = total;
  }
  for (int cc = b; cc <= nchunks; cc += 64) tab_lds[cc] = num;
  // segment sgi of request r: the item and its chunk-table entry
  auto put = [&](int r, int ro, int rt, int rl, int rn, int sgi, int jseg) {
    if (rt == 0) {  // an empty request keeps one empty segment
      items[jseg] = make_int4(r, 0, 0, -1);
      atomicMin(&tab_lds[ro / C < nchunks ? ro / C : nchunks - 1], jseg);
      return;
    }
    const int cc = ro / C + sgi;
    const int64_t g0 = ro > (int64_t)cc * C ? ro : (int64_t)cc * C;
    const int64_t g1 = (int64_t)ro + rt < ((int64_t)cc + 1) * C ? (int64_t)ro + rt : ((int64_t)cc + 1) * C;
    const int kb = (int)((g0 - ro) * a.tile);
    const int ke = (int)((g1 - ro) * a.tile < rl ? (g1 - ro) * a.tile : rl);
    items[jseg] = make_int4(r, kb, ke, rn > 1 ? jseg : -1);
    atomicMin(&tab_lds[cc], jseg);
  };
  int most = nseg;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) most = max(most, __shfl_xor(most, off, 64));
  if (most <= kOneWaveLaneSegs) {
    // few segments per request: each lane writes its own request's
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int sgi = 0; sgi < nseg && first + sgi < num; ++sgi) put(b, o, t, L, nseg, sgi, first + sgi);
  } else {
    // many (a few long requests): the segments spread over all lanes; segment
    // j belongs to the request r with first_l[r] <= j < first_l[r + 1] (every
    // request has at least one segment, so the offsets increase)
    if (on) {
      first_l[b] = first;
      o_l[b] = o;
      t_l[b] = t;
      len_l[b] = L;
    }
    if (b == 0) first_l[B] = total;
    // other lanes read these entries: order the LDS writes before the reads
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int jseg = b; jseg < num; jseg += 64) {
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (first_l[mid] <= jseg) lo = mid; else hi = mid;
      }
      put(lo, o_l[lo], t_l[lo], len_l[lo], first_l[lo + 1] - first_l[lo], jseg - first_l[lo], jseg);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int cc = b; cc <= nchunks; cc += 64) tab[cc] = cc == nchunks ? num : tab_lds[cc];
  if (b == 0) {
    ws[WS_MODE] = PKV_DECODE;
    ws[WS_BATCH] = B;
    ws[WS_NUM_ITEMS] = num;
    ws[WS_CAPACITY] = (int32_t)a.capacity;
    ws[WS_CHUNK] = C;
    ws[WS_TARGET] = a.target_items;
    ws[WS_NCHUNKS] = nchunks;
    ws[WS_CHUNK_TAB] = (int32_t)(a.tmp_off + B + 1);
  }
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

  if (plan_decode_by_one_wave(a)) {  // launched as one wave
    if (threadIdx.x < 64) plan_decode_one_wave(a, reinterpret_cast<int32_t*>(keys_lds));
    return;
  }
  if (a.mode == PKV_DECODE && a.kv_chunk == 0) {
    // Balanced chunks: the requests' tiles (a.tile tokens) laid end to end (request
    // b at global tiles [o_b, o_b + t_b)) are cut into chunks of C tiles,
    // C = ceil(T / target); a chunk is one workgroup and holds the request
    // segments it overlaps, so every workgroup streams the same amount of KV.
    // The arrays below are written to the workspace and, when they fit, read
    // back from copies in LDS (the sort buffer is idle here): each read of
    // the workspace would be a round trip through L2, and the chunk table's
    // binary search is a chain of them.
    int32_t* const lds_i = reinterpret_cast<int32_t*>(keys_lds);
    const bool in_lds = 2 * ((int64_t)B + 1) + a.capacity <= 2 * (int64_t)kPlanLdsSortMax;
    int32_t* goff_ws = ws + a.tmp_off;  // [B+1] global tile offset of each request
    int32_t* goff = in_lds ? lds_i : goff_ws;
    int32_t* req_rd = in_lds ? lds_i + (B + 1) : req;
    for (int base = 0; base < B; base += blockDim.x) {
      const int b = base + threadIdx.x;
      const int64_t t = b < B ? ((int64_t)clamp_len(a.seq_lens[b], a.max_kv_len) + a.tile - 1) / a.tile : 0;
      int64_t tot;
      const int64_t ex = block_exclusive_scan(t, sh, &tot);
      if (b < B) goff[b] = goff_ws[b] = (int32_t)(carry + ex);
      carry += tot;
    }
    const int64_t T = carry;
    if (threadIdx.x == 0) goff[B] = goff_ws[B] = (int32_t)T;
    int64_t C = (T + a.target_items - 1) / a.target_items;
    C = C < 1 ? 1 : C;
    int64_t nchunks = (T + C - 1) / C;
    nchunks = nchunks < 1 ? 1 : nchunks;
    __threadfence_block();
    __syncthreads();
    // segments per request (an empty request keeps one empty segment)
    carry = 0;
    for (int base = 0; base < B; base += blockDim.x) {
      const int b = base + threadIdx.x;
      int64_t nseg = 0;
      if (b < B) {
        const int64_t o = goff[b], t = goff[b + 1] - o;
        nseg = t == 0 ? 1 : (o + t - 1) / C - o / C + 1;
      }
      int64_t tot;
      const int64_t ex = block_exclusive_scan(nseg, sh, &tot);
      if (b < B) req_rd[b] = req[b] = (int32_t)(carry + ex);
      carry += tot;
    }
    if (threadIdx.x == 0) req_rd[B] = req[B] = (int32_t)carry;
    const int64_t num = carry < a.capacity ? carry : a.capacity;
    __threadfence_block();
    __syncthreads();
    // segments (b, kv_begin, kv_end, partial index) in request order, and
    // the chunk of each (non-decreasing along the list)
    int32_t* seg_chunk_ws = ws + a.keys_off;
    int32_t* seg_chunk = in_lds ? lds_i + 2 * (B + 1) : seg_chunk_ws;
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      const int L = clamp_len(a.seq_lens[b], a.max_kv_len);
      const int64_t o = goff[b], t = goff[b + 1] - o;
      const int first = req_rd[b], n = req_rd[b + 1] - req_rd[b];
      if (t == 0) {
        if (first < num) {
          items[first] = make_int4(b, 0, 0, -1);
          const int64_t cc = o / C;
          seg_chunk[first] = seg_chunk_ws[first] = (int32_t)(cc < nchunks ? cc : nchunks - 1);
        }
        continue;
      }
      for (int sgi = 0; sgi < n && first + sgi < num; ++sgi) {
        const int64_t cc = o / C + sgi;
        const int64_t g0 = o > cc * C ? o : cc * C;
        const int64_t g1 = o + t < (cc + 1) * C ? o + t : (cc + 1) * C;
        const int kb = (int)((g0 - o) * a.tile);
        const int ke = (int)((g1 - o) * a.tile < L ? (g1 - o) * a.tile : L);
        items[first + sgi] = make_int4(b, kb, ke, n > 1 ? first + sgi : -1);
        seg_chunk[first + sgi] = seg_chunk_ws[first + sgi] = (int32_t)cc;
      }
    }
    __threadfence_block();
    __syncthreads();
    // chunk table: first segment of each chunk
    int32_t* tab = ws + a.tmp_off + B + 1;
    for (int64_t cc = threadIdx.x; cc <= nchunks; cc += blockDim.x) {
      int lo = 0, hi = (int)num;  // first segment with chunk >= cc
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (seg_chunk[mid] < cc) lo = mid + 1; else hi = mid;
      }
      tab[cc] = cc == nchunks ? (int32_t)num : lo;
    }
    if (threadIdx.x == 0) {
      ws[WS_MODE] = PKV_DECODE;
      ws[WS_BATCH] = B;
      ws[WS_NUM_ITEMS] = (int32_t)num;
      ws[WS_CAPACITY] = (int32_t)a.capacity;
      ws[WS_CHUNK] = (int32_t)C;
      ws[WS_TARGET] = a.target_items;
      ws[WS_NCHUNKS] = (int32_t)nchunks;
      ws[WS_CHUNK_TAB] = (int32_t)(a.tmp_off + B + 1);
    }
    return;
  }

  if (a.mode == PKV_DECODE) {
    // Fixed splits of kv_chunk tokens per request; each split is its own
    // chunk.  Ordered longest first when they overflow the target.
    const int64_t chunk = a.kv_chunk / kDecodeTile;
    for (int base = 0; base < B; base += blockDim.x) {
      int b = base + threadIdx.x;
      int64_t splits = 0;
      if (b < B) {
        int64_t tiles = ((int64_t)clamp_len(a.seq_lens[b], a.max_kv_len) + kDecodeTile - 1) / kDecodeTile;
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
    // items (b, kv_begin, kv_end, partial index), created request-major; the
    // partial index of split s of request b is req[b] + s
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
      ws[WS_NCHUNKS] = (int32_t)num;
      ws[WS_CHUNK_TAB] = 0;
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
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(plan_decode_by_one_wave(a) ? 64 : kPlanThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
