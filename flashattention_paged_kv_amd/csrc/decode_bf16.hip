// Split-KV paged decode, bf16 K/V, fp32 accumulation (one query row per
// request).  HBM-bound: every K/V byte of a request is read exactly once.
//
// One wave64 per work item (request b, one split of its KV range, kv head g,
// group of up to 16 query heads of g).  The wave walks its range in 32-token
// tiles; every tile is gathered straight from the pools into registers
// through req_to_token (a slot lookup per token, so any page size works):
//
//  * scores use the MFMA 16x16x32 bf16 product Sᵀ = K·Qᵀ: K rows are the A
//    operand (one 16-byte load per lane and 32-wide d chunk), the query
//    heads of the group are the B operand, kept in registers for the item;
//  * the Sᵀ output leaves every lane with 4+4 scores of ONE head, so the
//    online softmax (running max m, sum l, rescale of the accumulator) is
//    per-lane arithmetic plus two xor-shuffles for the tile max, and the
//    probabilities are already in the B-operand layout of the PV product;
//  * PV is Oᵀ = Vᵀ·Pᵀ with Vᵀ as the A operand: each lane loads 8 V rows
//    (16 bytes of each) and transposes them to operands with byte permutes,
//    so no LDS round trip is needed.
// K and V rows are read once; with few kv heads per token the loads carry
// the non-temporal hint (STREAM).
//
// Items with one split write bf16 O and lse directly; otherwise the split's
// normalised partial O and log2-sum-exp go to scratch and the merge kernel
// (decode_merge.h) combines them.
#include "decode_merge.h"
#include "decode_stream.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

template <int D>
struct KVTile {
  static constexpr int KB = D / 32;
  u32x4 k[2][KB];  // A operands of Sᵀ = K·Qᵀ: [token block][32-wide d chunk]
  u32x4 v[8];      // the lane's 8 V rows, elements d = 8*(lane%16) .. +8
};

// Lane l's token slot for position t0 + (l & 31) of the tile.  Positions past
// the item's range are clamped to its last token, so every load below is
// unconditional (straight-line code keeps the compiler's load counting exact)
// and re-reads a row already fetched; their scores are masked to -inf.
__device__ __forceinline__ uint32_t tile_slot(const int32_t* __restrict__ rtt_row, int t0, int kv_end,
                                              uint32_t last, int lane) {
  const int tok = min(t0 + (lane & 31), kv_end - 1);
  return clamp_slot_u32(rtt_row[tok], last);
}

template <int D, bool STREAM>
__device__ __forceinline__ void load_tile(KVTile<D>& t, uint32_t slot, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, uint32_t row_elems, int lane) {
  constexpr int KB = D / 32;
  const int l16 = lane & 15, j = lane >> 4;
  const uint32_t sk0 = __shfl(slot, l16), sk1 = __shfl(slot, 16 + l16);
  const uint16_t* k0 = kbase + row_offset(sk0, row_elems) + 8 * j;
  const uint16_t* k1 = kbase + row_offset(sk1, row_elems) + 8 * j;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    t.k[0][kb] = ldg16_once<STREAM>(k0 + 32 * kb);
    t.k[1][kb] = ldg16_once<STREAM>(k1 + 32 * kb);
  }
  // d = 64: lanes 8..15 re-read columns of their own row; they only feed
  // output rows d >= 64, which are never stored
  const int dcol = 8 * (l16 & (D / 8 - 1));
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int tau = r < 4 ? 4 * j + r : 16 + 4 * j + (r - 4);
    const uint32_t sv = __shfl(slot, tau);
    t.v[r] = ldg16_once<STREAM>(vbase + row_offset(sv, row_elems) + dcol);
  }
}

template <int D>
__device__ __forceinline__ void compute_tile(const KVTile<D>& t, const u32x4 (&qop)[D / 32], int t0, int kv_end,
                                             float scale_log2, float& m, float& lpart, floatx4 (&acc)[8],
                                             int lane) {
  constexpr int KB = D / 32;
  const int j = lane >> 4;
  floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    s0 = mfma16x16x32(as_bf16x8(t.k[0][kb]), as_bf16x8(qop[kb]), s0);
    s1 = mfma16x16x32(as_bf16x8(t.k[1][kb]), as_bf16x8(qop[kb]), s1);
  }
  float sc[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = (t0 + 4 * j + r < kv_end) ? s0[r] * scale_log2 : kNegInf;
    sc[4 + r] = (t0 + 16 + 4 * j + r < kv_end) ? s1[r] * scale_log2 : kNegInf;
  }
  float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
  mx = max_xor32(max_xor16(mx));
  // -inf only for a column that has seen no key yet (a new token whose causal
  // limit lies below this tile); it then keeps zero weight
  const float m_new = fmaxf(m, mx);
  const float alpha = m_new == kNegInf ? 1.f : exp2_fast(m - m_new);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  m = m_new;
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = exp2_fast(sc[i] - m_use);
    ps += p[i];
  }
  lpart = lpart * alpha + ps;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= alpha;
  u32x4 pop;
  pop[0] = pack_bf16x2(p[0], p[1]);
  pop[1] = pack_bf16x2(p[2], p[3]);
  pop[2] = pack_bf16x2(p[4], p[5]);
  pop[3] = pack_bf16x2(p[6], p[7]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    u32x4 vop;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      vop[k] = (e & 1) ? pack_hi16(t.v[2 * k][w], t.v[2 * k + 1][w]) : pack_lo16(t.v[2 * k][w], t.v[2 * k + 1][w]);
    acc[e] = mfma16x16x32(as_bf16x8(vop), as_bf16x8(pop), acc[e]);
  }
}

}  // namespace

// Q of output row (request b, new token qi), query head h, as the B operand.
template <int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, u32x4 (&qop)[D / 32], int b, int qi, int h, bool head_ok,
                                       int j) {
  qi = opaque(qi);
  h = opaque(h);
  j = opaque(j);
  const uint16_t* qrow =
      static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.q_len + (head_ok ? qi : 0)) * a.hq + (head_ok ? h : 0)) * D;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) qop[kb] = head_ok ? ldg16(qrow + 32 * kb + 8 * j) : z;
}

// Normalises one segment's accumulator and writes it: bf16 O and lse for a
// request covered by one segment, else the fp32 partial and its log2-sum-exp.
template <int D>
__device__ __forceinline__ void finish_segment(const DecodeArgs& a, int b, int part, float m, float lpart,
                                               const floatx4 (&acc)[8], int qi, int h, bool head_ok, int j) {
  qi = opaque(qi);
  h = opaque(h);
  j = opaque(j);
  float l = lpart + __shfl_xor(lpart, 16);
  l += __shfl_xor(l, 32);
  const bool rows_ok = (D == 128) || (j < 2);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse2 = l > 0.f ? m + __log2f(l) : kNegInf;
  if (part < 0) {
    if (head_ok && rows_ok) {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + (((int64_t)b * a.q_len + qi) * a.hq + h) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(acc[2 * k][r] * inv, acc[2 * k + 1][r] * inv);
        stg16(orow + 32 * j + 8 * r, w);
      }
    }
    if (head_ok && j == 0 && a.lse) a.lse[((int64_t)b * a.q_len + qi) * a.hq + h] = lse2 * kLn2;
    return;
  }
  if (head_ok && rows_ok) {
    float* po = a.part_o + (((int64_t)part * a.q_len + qi) * a.hq + h) * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      floatx4 w0 = {acc[0][r] * inv, acc[1][r] * inv, acc[2][r] * inv, acc[3][r] * inv};
      floatx4 w1 = {acc[4][r] * inv, acc[5][r] * inv, acc[6][r] * inv, acc[7][r] * inv};
      *reinterpret_cast<floatx4*>(po + 32 * j + 8 * r) = w0;
      *reinterpret_cast<floatx4*>(po + 32 * j + 8 * r + 4) = w1;
    }
  }
  if (head_ok && j == 0) a.part_lse[((int64_t)part * a.q_len + qi) * a.hq + h] = lse2;
}

// One chunk (the request segments [s0, s1)) for one unit (kv head g,
// 16-head group).  The chunk's tiles form one stream, so the software
// pipeline runs across segment boundaries: while tile i is computed, the K/V
// rows of tile i+1 are in flight and the slots of tile i+2 were requested
// before them, whichever segments the three tiles belong to.  Two register
// buffers are used in turn.  When the computed tile enters a new segment the
// previous one is written out and the online-softmax state restarts.
template <int D, bool STREAM>
__device__ __forceinline__ void decode_chunk(const DecodeArgs& a, int s0, int s1, int unit, int4* win_rec,
                                             int2* win_req) {
  const int g = unit / a.head_groups, hg = unit - g * a.head_groups;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, j = lane >> 4;
  // MFMA column l16 of this unit = (new token qi, query head hl of kv head g)
  const int col = hg * 16 + l16;
  const int qi = col / a.group, hl = col - qi * a.group;
  const bool head_ok = qi < a.q_len;
  const int h = g * a.group + hl;
  const uint32_t row_elems = (uint32_t)a.hkv * D;
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(a.k_pool) + (int64_t)g * D;
  const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(a.v_pool) + (int64_t)g * D;
  const uint32_t last = (uint32_t)(a.pool_slots - 1);

  SegWindow w;
  w.rec = win_rec;
  w.req = win_req;
  load_window(a, w, s0, s1, lane);
  // first non-empty segment
  TileCursor C = seg_at(a, w, s0, s1, lane);
  C.t0 -= kDecodeTile;
  C = next_tile<kDecodeTile>(a, w, C, s1, lane);
  finish_empty<D>(a, w, s0, C.seg, s1, qi, h, head_ok, j, lane);
  if (C.seg >= s1) return;

  u32x4 qop[D / 32];
  load_q<D>(a, qop, C.b, qi, h, head_ok, j);
  float m = kNegInf, lpart = 0.f;
  floatx4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto rtt_of = [&](const TileCursor& c) { return a.rtt + (int64_t)c.row * a.rtt_stride; };
  KVTile<D> ta, tb;
  load_tile<D, STREAM>(ta, tile_slot(rtt_of(C), C.t0, C.kv_end, last, lane), kbase, vbase, row_elems, lane);
  TileCursor L = next_tile<kDecodeTile>(a, w, C, s1, lane);
  uint32_t s_odd = tile_slot(rtt_of(L), L.t0, L.kv_end, last, lane), s_even;
  TileCursor S = next_tile<kDecodeTile>(a, w, L, s1, lane);

  // after tile C is computed: shift the cursors and, on entering a new
  // segment, write the finished one out and restart the softmax state
  auto advance = [&]() -> bool {
    const TileCursor prev = C;
    C = L;
    L = S;
    S = next_tile<kDecodeTile>(a, w, S, s1, lane);
    if (C.seg == prev.seg) return true;
    finish_segment<D>(a, prev.b, prev.part, m, lpart, acc, qi, h, head_ok, j);
    finish_empty<D>(a, w, prev.seg + 1, C.seg, s1, qi, h, head_ok, j, lane);
    if (C.seg >= s1) return false;
    load_q<D>(a, qop, C.b, qi, h, head_ok, j);
    m = kNegInf;
    lpart = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    return true;
  };

  for (;;) {
    s_even = tile_slot(rtt_of(S), S.t0, S.kv_end, last, lane);
    load_tile<D, STREAM>(tb, s_odd, kbase, vbase, row_elems, lane);
    __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of this tile's math
    compute_tile<D>(ta, qop, C.t0, min(C.kv_end, C.lim + qi + 1), a.scale_log2, m, lpart, acc, lane);
    if (!advance()) break;
    s_odd = tile_slot(rtt_of(S), S.t0, S.kv_end, last, lane);
    load_tile<D, STREAM>(ta, s_even, kbase, vbase, row_elems, lane);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile<D>(tb, qop, C.t0, min(C.kv_end, C.lim + qi + 1), a.scale_log2, m, lpart, acc, lane);
    if (!advance()) break;
  }
}

// WPB waves per workgroup take WPB consecutive (kv head, head group) units of
// the same chunk, so the rows of one token are requested together.  The plan
// lays the requests' tiles end to end and cuts them into chunks of equal
// length; a chunk is a list of request segments.
template <int D, int WPB, bool STREAM>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(2))) void decode_bf16_kernel(DecodeArgs a) {
  const int32_t* __restrict__ ws = a.ws;
  // 1-D grid, unit group fastest: the workgroups of one chunk are
  // dispatched back to back and the unused tail of the capacity comes last
  const int ngroups = (a.hkv * a.head_groups + WPB - 1) / WPB;
  const int c = __builtin_amdgcn_readfirstlane((int)blockIdx.x / ngroups);  // uniform
  if (c >= ws[WS_NCHUNKS]) return;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform
  const int unit = __builtin_amdgcn_readfirstlane(((int)blockIdx.x - c * ngroups) * WPB + wv);
  if (unit >= a.hkv * a.head_groups) return;
  const int tab = ws[WS_CHUNK_TAB];
  const int s0 = tab ? ws[tab + c] : c, s1 = tab ? ws[tab + c + 1] : c + 1;
  __shared__ int4 win_rec[WPB][64];
  __shared__ int2 win_req[WPB][64];
  decode_chunk<D, STREAM>(a, s0, s1, unit, win_rec[wv], win_req[wv]);
}

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, int64_t capacity, int32_t batch,
                               hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  dim3 grid((unsigned)batch, (unsigned)(a.q_len * a.hq));
  const int nw = merge_waves(capacity, batch);
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(64 * nw), 0, s, a); };
  if (head_dim == 128) {
    if (nw == 8) go(decode_merge_many_kernel<128, 8>);
    else if (nw == 4) go(decode_merge_many_kernel<128, 4>);
    else go(decode_merge_few_kernel<128>);
  } else {
    if (nw == 8) go(decode_merge_many_kernel<64, 8>);
    else if (nw == 4) go(decode_merge_many_kernel<64, 4>);
    else go(decode_merge_few_kernel<64>);
  }
  return hipGetLastError();
}

// Kernel instance for head_dim D, wpb waves per workgroup and the load
// form; fewer than 8 units always stream (decode_streams).
template <int D>
const void* decode_bf16_kernel_for(int wpb, bool stream) {
  if (wpb == 8) return stream ? (const void*)decode_bf16_kernel<D, 8, true> : (const void*)decode_bf16_kernel<D, 8, false>;
  return wpb == 4 ? (const void*)decode_bf16_kernel<D, 4, true> : wpb == 2 ? (const void*)decode_bf16_kernel<D, 2, true>
                                                                            : (const void*)decode_bf16_kernel<D, 1, true>;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int head_dim, int64_t capacity, int32_t batch,
                              hipStream_t s) {
  if (capacity <= 0 || batch <= 0) return hipSuccess;
  // up to 8 waves per workgroup: the kv heads of one split run side by side
  const int units = a.hkv * a.head_groups;
  const int wpb = decode_waves_per_block(units);
  const bool stream = decode_streams(units);
  const void* k = head_dim == 128 ? decode_bf16_kernel_for<128>(wpb, stream) : decode_bf16_kernel_for<64>(wpb, stream);
  DecodeArgs args = a;
  void* kargs[] = {&args};
  const hipError_t e = hipLaunchKernel(k, dim3((unsigned)(capacity * ceil_div(units, wpb))), dim3(64 * wpb), kargs, 0, s);
  const hipError_t last = hipGetLastError();  // also clears what the launch left
  return e != hipSuccess ? e : last;
}

hipError_t resident_items_of(const void* kernel, int wpb, int units, int64_t* items) {
  int dev = 0, cus = 0, blocks = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 64 * wpb, 0);
  if (e != hipSuccess) return e;
  const int64_t per_item = ceil_div(units, wpb);  // workgroups of one item
  *items = (int64_t)cus * blocks / per_item;
  return hipSuccess;
}

hipError_t decode_bf16_resident_items(int head_dim, int units, int64_t* items) {
  const int wpb = decode_waves_per_block(units);
  const bool stream = decode_streams(units);
  const void* k = head_dim == 128 ? decode_bf16_kernel_for<128>(wpb, stream) : decode_bf16_kernel_for<64>(wpb, stream);
  return resident_items_of(k, wpb, units, items);
}

}  // namespace pkv
