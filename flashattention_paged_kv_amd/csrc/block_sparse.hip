// Block-sparse DECODE, the once-per-batch step.  The block-sparse mode of the
// FlashInfer PrimTS Sage page (README block; measured at densities 0.125 and
// 0.10) attends exactly to the keys of the listed KV blocks: one ascending,
// duplicate-free list of block numbers per request, shared by all heads, a
// block being block_size consecutive logical positions.
//
// The listed blocks are laid end to end into "virtual" positions
// 0 .. V_b - 1 (block i of the list, if it holds keys, starts at virtual
// position (i - i0) · block_size, i0 = the list's first non-negative entry;
// only the last such block can be partial).  This kernel writes, per request,
// the slot of every virtual position (a compacted page table), V_b, and for
// the 8-bit path the sfK of every virtual k_block (block_size is a multiple
// of k_block, so a virtual k_block is one logical k_block).  The decode plan
// and kernels then run unchanged over the virtual positions: the softmax
// over a set of keys does not depend on their order, and the only
// position-dependent input, sfK, is carried over.
//
// Work: grid (batch, kSparseSplit) workgroups of 256 threads; workgroup
// (b, y) takes every kSparseSplit-th group of 256 (entry, token) pairs of
// request b.  Every read is clamped to its buffer and every write is bounded
// by max_kv_len (sfk_stride for sfK), so a malformed list gives wrong
// numbers, never an out-of-bounds access.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kSparseThreads = 256;

// first index in [lo, hi) whose entry is >= key (entries ascending)
__device__ __forceinline__ int lower_bound(const int32_t* __restrict__ v, int lo, int hi, int key) {
  while (lo < hi) {
    const int mid = lo + ((hi - lo) >> 1);
    if (v[mid] < key)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

}  // namespace

__global__ __launch_bounds__(kSparseThreads) void block_sparse_table_kernel(SparseTableArgs a) {
  const int b = blockIdx.x;
  const int y = blockIdx.y;
  const int tid = threadIdx.x;
  const int L = min(max(a.seq_lens[b], 0), a.max_kv_len);
  const int shift = a.block_shift;
  const int bs = 1 << shift;
  const int nblk = (L + bs - 1) >> shift;  // blocks that hold keys
  const int64_t nnz = a.num_indices;
  const int e0 = (int)min(max((int64_t)a.indptr[b], (int64_t)0), nnz);
  const int e1 = (int)min(max((int64_t)a.indptr[b + 1], (int64_t)e0), nnz);
  // entries [i0, i1) of the ascending list select keys: 0 <= k < nblk
  __shared__ int s_range[2];
  if (tid == 0) {
    s_range[0] = lower_bound(a.indices, e0, e1, 0);
    s_range[1] = lower_bound(a.indices, s_range[0], e1, nblk);
  }
  __syncthreads();
  const int i0 = s_range[0], i1 = s_range[1];
  const int32_t* rtt_row = a.rtt + (int64_t)(a.rpi ? a.rpi[b] : b) * a.rtt_stride;
  int32_t* out_row = a.out_rtt + (int64_t)b * a.max_kv_len;

  // slots: pair p = (entry i0 + (p >> shift), token p & (bs - 1))
  const int pairs = (i1 - i0) << shift;
  for (int p = y * kSparseThreads + tid; p < pairs; p += kSparseSplit * kSparseThreads) {
    const int j = p >> shift, t = p & (bs - 1);
    const int k = a.indices[i0 + j];
    // a list that is not ascending can carry k outside [0, nblk) here
    if (k < 0 || k >= nblk) continue;
    const int pos = (k << shift) + t;  // logical position
    const int v = p;                   // virtual position (j · bs + t)
    if (pos < L && v < a.max_kv_len) out_row[v] = rtt_row[pos];
  }
  if (a.out_sfk) {
    // sfK of the virtual k_blocks: triple (kv head g, entry, k_block u in the entry)
    const int kpb = bs / a.k_block;
    const int per_g = (i1 - i0) * kpb;
    for (int p = y * kSparseThreads + tid; p < per_g * a.hkv; p += kSparseSplit * kSparseThreads) {
      const int g = p / per_g;
      const int r = p - g * per_g;
      const int j = r / kpb, u = r - j * kpb;
      const int k = a.indices[i0 + j];
      if (k < 0 || k >= nblk) continue;
      const int pos = (k << shift) + u * a.k_block;
      const int vb = r;  // virtual k_block: (j · bs + u · k_block) / k_block
      if (pos < L && vb < a.sfk_stride) {
        const int64_t base = ((int64_t)b * a.hkv + g) * a.sfk_stride;
        a.out_sfk[base + vb] = a.sfk[base + pos / a.k_block];
      }
    }
  }
  if (y == 0 && tid == 0) {
    // V_b: full blocks, then the last listed block cut at L
    int vlen = 0;
    if (i1 > i0) {
      const int k_last = min(max(a.indices[i1 - 1], 0), nblk - 1);  // in range for an ascending list
      vlen = ((i1 - i0 - 1) << shift) + min(bs, L - (k_last << shift));
    }
    a.out_lens[b] = min(max(vlen, 0), a.max_kv_len);
  }
}

hipError_t launch_block_sparse_table(const SparseTableArgs& a, int32_t batch, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_sparse_table_kernel, dim3((unsigned)batch, (unsigned)kSparseSplit),
                     dim3(kSparseThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
