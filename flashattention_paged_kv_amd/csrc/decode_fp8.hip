// 8-bit (OCP E4M3) split-KV decode following the Sage formula of the
// FlashInfer PrimTS Sage page (code §1, §4):
//
//   S = sm_scale · sfQ[b,h] · sfK[b,g,⌊j/k_block⌋] · (q8 · k8_j)
//   P8 = E4M3(448 · exp(S - m)),  l = Σ exp(S - m)  (unquantised)
//   O = sfV[b,g,:] · (Σ_j P8_j · v8_j) / (448 · l)  (+ v_mean[b,g,:])
//
// Q and K scales enter before the row max and the exponential; the V scale
// is per channel and applied once at the end.  This kernel keeps a running
// max m (online softmax), so P8 is quantised against the running max and
// the accumulator is rescaled in fp32 when the max grows.
//
// Same decomposition as the bf16 decode (one wave per (request, split, kv
// head, group of 16 (new token, head) columns); a request with several
// splits is merged by the kernels of decode_merge.h; with several new tokens per
// request each column has its own causal limit and sfQ row), with 64-token
// tiles and the gfx950 fp8 MFMA
// 16x16x128 (f8f6f4, unit block scales):
//  * Sᵀ = K8·Q8ᵀ: one MFMA per 16 keys covers all 128 channels (each lane
//    holds 32 bytes of one key row);
//  * Oᵀ += V8ᵀ·P8ᵀ: each lane gathers 16 keys x 8 channels of V8 and
//    transposes the bytes with permutes into 8 A operands; 64 of the 128
//    k slots carry the tile's keys, the rest are zero.
// With INT8 Q and K (the page's code §3 and §4) Sᵀ is two int8 MFMAs
// 16x16x64 per 16 keys, one per 16-byte half of the lanes' 32 bytes; A and
// B take the same bytes of the same lanes, so their products pair channel
// with channel whatever order the instruction sums them in.  The int32 dot
// product (|q·k| <= 128·128·128 < 2^24) converts to fp32 exactly.
#include "decode_stream.h"
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kTile8 = 64;

__device__ __forceinline__ floatx4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, floatx4 c) {
  // fp8 E4M3 for both operands (format 0), block scales 2^0 (E8M0 127)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Scores of 16 keys x 16 columns over the 128 channels: E4M3 codes, or
// int8 codes (two int8 MFMAs over the lanes' two 16-byte halves).
template <bool I8>
__device__ __forceinline__ floatx4 qk_scores(i32x8 kop, i32x8 qop) {
  if constexpr (I8) {
    const i32x4 k0 = {kop[0], kop[1], kop[2], kop[3]}, k1 = {kop[4], kop[5], kop[6], kop[7]};
    const i32x4 q0 = {qop[0], qop[1], qop[2], qop[3]}, q1 = {qop[4], qop[5], qop[6], qop[7]};
    i32x4 s = {0, 0, 0, 0};
    s = __builtin_amdgcn_mfma_i32_16x16x64_i8(k0, q0, s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_i32_16x16x64_i8(k1, q1, s, 0, 0, 0);
    return floatx4{(float)s[0], (float)s[1], (float)s[2], (float)s[3]};
  } else {
    return mfma_fp8_16x16x128(kop, qop, floatx4{0.f, 0.f, 0.f, 0.f});
  }
}

struct Tile8 {
  u32x4 k[4][2];  // A operands of Sᵀ: 4 blocks of 16 keys, 32 bytes (channels 32j..32j+31)
  u32x2 v[16];    // the lane's 16 V rows, channels 8*(lane%16) .. +8
  float ks;       // sfK of 16-key block (lane & 3) of the tile
};

// token (within the tile) of element e (0..15) held by lane group j in the Pᵀ / Vᵀ operands
__device__ __forceinline__ int tok_of(int j, int e) { return 16 * (e >> 2) + 4 * j + (e & 3); }

// Slot of token t0 + (lane & 63), clamped to the item's last token: every
// load is unconditional and positions past the range re-read a fetched row
// (their scores are masked to -inf).
__device__ __forceinline__ uint32_t slot_at(const int32_t* __restrict__ rtt_row, int t0, int kv_end, uint32_t last,
                                            int lane) {
  return clamp_slot_u32(rtt_row[min(t0 + lane, kv_end - 1)], last);
}

template <bool STREAM>
__device__ __forceinline__ void load_tile8(Tile8& t, uint32_t slot, int t0, int kv_end,
                                           const float* __restrict__ sfk_row, int k_block,
                                           const uint8_t* __restrict__ kbase, const uint8_t* __restrict__ vbase,
                                           uint32_t row_bytes, int lane) {
  // `slot`: slot of token (lane & 63) of the tile
  const int l16 = lane & 15, j = lane >> 4;
  t.ks = sfk_row[min(t0 + 16 * (lane & 3), kv_end - 1) / k_block];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const uint32_t sk = __shfl(slot, 16 * blk + l16);
    const uint8_t* p = kbase + row_offset(sk, row_bytes) + 32 * j;
    t.k[blk][0] = ldg16_once<STREAM>(p);
    t.k[blk][1] = ldg16_once<STREAM>(p + 16);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t sv = __shfl(slot, tok_of(j, e));
    t.v[e] = ldg8_once<STREAM>(vbase + row_offset(sv, row_bytes) + 8 * l16);
  }
}

// 4x4 byte transpose: out[c] = {x0.byte c, x1.byte c, x2.byte c, x3.byte c}
__device__ __forceinline__ void transpose4x4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t (&o)[4]) {
  const uint32_t a_lo = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t a_hi = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t b_lo = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);  // x0.b0 x1.b0 x2.b0 x3.b0
  o[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0,1 (OCP E4M3, nearest even)
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);       // bytes 2,3
  return (uint32_t)w;
}

}  // namespace

// Q8 of new token qi of request b as the B operand (lane holds
// q8[row][h][32 j .. 32 j + 32], row = b·q_len + qi) and the score factor
// sm_scale·log2(e)·sfQ[row, h].
__device__ __forceinline__ void load_q8(const DecodeArgs& a, i32x8& qop, float& qscale, int b, int qi, int h,
                                        bool head_ok, int j) {
  constexpr int D = 128;
  h = opaque(h);
  j = opaque(j);
  const int64_t row = ((int64_t)b * a.q_len + (head_ok ? qi : 0)) * a.hq + h;
  const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + row * D + 32 * j;
  const u32x4 z = {0u, 0u, 0u, 0u};
  const u32x4 q0 = head_ok ? ldg16(qrow) : z, q1 = head_ok ? ldg16(qrow + 16) : z;
  qop = i32x8{(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3], (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
  qscale = head_ok ? a.sfq[row] * a.scale_log2 : 0.f;
}

// Applies the per-channel V scale (and mean) to one segment's accumulator and
// writes it: bf16 O and lse for a request covered by one segment, else the
// fp32 partial and its log2-sum-exp.
__device__ __forceinline__ void finish_segment8(const DecodeArgs& a, int b, int g, int part, float m, float lpart,
                                                const floatx4 (&acc)[8], int qi, int h, bool head_ok, int j) {
  constexpr int D = 128;
  h = opaque(h);
  j = opaque(j);
  float l = lpart + __shfl_xor(lpart, 16);
  l += __shfl_xor(l, 32);
  // Oᵀ block c, row 4 j + r  <->  channel d = 8 (4 j + r) + c = 32 j + 8 r + c
  const float inv = l > 0.f ? 1.f / (448.f * l) : 0.f;
  const float lse2 = l > 0.f ? m + __log2f(l) : kNegInf;
  const float* sfv = a.sfv + ((int64_t)b * a.hkv + g) * D;
  const float* vmean = a.v_mean ? a.v_mean + ((int64_t)b * a.hkv + g) * D : nullptr;
  float o[4][8];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d = 32 * j + 8 * r + c;
      o[r][c] = acc[c][r] * inv * sfv[d] + (vmean ? vmean[d] : 0.f);
    }
  if (part < 0) {
    if (head_ok) {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + (((int64_t)b * a.q_len + qi) * a.hq + h) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(o[r][2 * k], o[r][2 * k + 1]);
        stg16(orow + 32 * j + 8 * r, w);
      }
      if (j == 0 && a.lse) a.lse[((int64_t)b * a.q_len + qi) * a.hq + h] = lse2 * kLn2;
    }
    return;
  }
  if (head_ok) {
    float* po = a.part_o + (((int64_t)part * a.q_len + qi) * a.hq + h) * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<floatx4*>(po + 32 * j + 8 * r) = floatx4{o[r][0], o[r][1], o[r][2], o[r][3]};
      *reinterpret_cast<floatx4*>(po + 32 * j + 8 * r + 4) = floatx4{o[r][4], o[r][5], o[r][6], o[r][7]};
    }
    if (j == 0) a.part_lse[((int64_t)part * a.q_len + qi) * a.hq + h] = lse2;
  }
}

// Empty segments (requests with no KV) in [from, to): the epilogue of an
// empty sum, so O = v_mean (0 without it) and lse = -inf.
__device__ __forceinline__ void finish_empty8(const DecodeArgs& a, SegWindow& w, int from, int to, int s1, int g,
                                              int qi, int h, bool head_ok, int j, int lane) {
  floatx4 zero[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) zero[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int s = from; s < to; ++s) {
    const TileCursor e = seg_at(a, w, s, s1, lane);
    finish_segment8(a, e.b, g, e.part, kNegInf, 0.f, zero, qi, h, head_ok, j);
  }
}

// One chunk (the request segments [s0, s1)) for one unit (kv head g,
// 16-head group), its 64-token tiles walked as one stream as in the bf16
// decode: while tile i is computed the rows of tile i+1 are in flight and
// the slots of tile i+2 were requested before them, whichever segments the
// tiles belong to.
// MULTI: several new tokens per request (per-lane causal limits); the
// one-token instance keeps none of that state in the tile loop.
template <bool MULTI, bool I8, bool STREAM>
__device__ __forceinline__ void decode_fp8_chunk(const DecodeArgs& a, int s0, int s1, int unit, int4* win_rec,
                                                 int2* win_req) {
  constexpr int D = 128;
  const int g = unit / a.head_groups, hg = unit - g * a.head_groups;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, j = lane >> 4;
  // MFMA column = (new token qi, head hl of the group), token-major
  const int col = hg * 16 + l16;
  const int qi = MULTI ? col / a.group : 0;
  const int hl = MULTI ? col - qi * a.group : col;
  const bool head_ok = MULTI ? qi < a.q_len : hl < a.group;
  const int h = g * a.group + (head_ok ? hl : 0);
  const uint32_t row_bytes = (uint32_t)a.hkv * D;
  const uint8_t* __restrict__ kbase = static_cast<const uint8_t*>(a.k_pool) + (int64_t)g * D;
  const uint8_t* __restrict__ vbase = static_cast<const uint8_t*>(a.v_pool) + (int64_t)g * D;
  const uint32_t last = (uint32_t)(a.pool_slots - 1);

  SegWindow w;
  w.rec = win_rec;
  w.req = win_req;
  load_window(a, w, s0, s1, lane);
  // first non-empty segment
  TileCursor C = seg_at(a, w, s0, s1, lane);
  C.t0 -= kTile8;
  C = next_tile<kTile8>(a, w, C, s1, lane);
  finish_empty8(a, w, s0, C.seg, s1, g, qi, h, head_ok, j, lane);
  if (C.seg >= s1) return;

  i32x8 qop;
  float qscale;
  load_q8(a, qop, qscale, C.b, qi, h, head_ok, j);
  float m = kNegInf, lpart = 0.f;
  floatx4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Tile8& cur, int t0, int kv_end) {
    // ---- scores: 4 blocks of 16 keys; every 16-key block lies in one sfK block
    float sc[16];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const i32x8 kop = {(int)cur.k[blk][0][0], (int)cur.k[blk][0][1], (int)cur.k[blk][0][2], (int)cur.k[blk][0][3],
                         (int)cur.k[blk][1][0], (int)cur.k[blk][1][1], (int)cur.k[blk][1][2], (int)cur.k[blk][1][3]};
      const floatx4 s = qk_scores<I8>(kop, qop);
      const int tb = t0 + 16 * blk;
      const float ks = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.ks), blk)) * qscale;
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[4 * blk + r] = (tb + 4 * j + r < kv_end) ? s[r] * ks : kNegInf;
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = max_xor32(max_xor16(mx));
    // -inf only for a column that has seen no key yet (a new token whose
    // causal limit lies below this tile); it then keeps zero weight
    const float m_new = fmaxf(m, mx);  // one token per request: finite, key t0 is in range
    const float alpha = (MULTI && m_new == kNegInf) ? 1.f : exp2_fast(m - m_new);
    const float m_use = (MULTI && m_new == kNegInf) ? 0.f : m_new;
    m = m_new;
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = exp2_fast(sc[e] - m_use);
      ps += p[e];
    }
    lpart = lpart * alpha + ps;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= alpha;
    // P8ᵀ operand: element e (byte e) <-> key tok_of(j, e); bytes 16..31 are zero
    i32x8 pop;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      pop[q] = (int)pack_fp8x4(448.f * p[4 * q], 448.f * p[4 * q + 1], 448.f * p[4 * q + 2], 448.f * p[4 * q + 3]);
    pop[4] = pop[5] = pop[6] = pop[7] = 0;
    // V8ᵀ operands: block c holds channel 8*l16 + c of the lane's 16 keys
    uint32_t vt[8][4];  // [channel c][key group of 4]
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint32_t o_lo[4], o_hi[4];
      transpose4x4(cur.v[4 * q4][0], cur.v[4 * q4 + 1][0], cur.v[4 * q4 + 2][0], cur.v[4 * q4 + 3][0], o_lo);
      transpose4x4(cur.v[4 * q4][1], cur.v[4 * q4 + 1][1], cur.v[4 * q4 + 2][1], cur.v[4 * q4 + 3][1], o_hi);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vt[c][q4] = o_lo[c];
        vt[4 + c][q4] = o_hi[c];
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const i32x8 vop = {(int)vt[c][0], (int)vt[c][1], (int)vt[c][2], (int)vt[c][3], 0, 0, 0, 0};
      acc[c] = mfma_fp8_16x16x128(vop, pop, acc[c]);
    }
  };

  auto rtt_of = [&](const TileCursor& c) { return a.rtt + (int64_t)c.row * a.rtt_stride; };
  auto sfk_of = [&](const TileCursor& c) { return a.sfk + ((int64_t)c.b * a.hkv + g) * a.sfk_stride; };
  Tile8 ta, tb;
  load_tile8<STREAM>(ta, slot_at(rtt_of(C), C.t0, C.kv_end, last, lane), C.t0, C.kv_end, sfk_of(C), a.k_block, kbase, vbase,
             row_bytes, lane);
  TileCursor L = next_tile<kTile8>(a, w, C, s1, lane);
  uint32_t s_odd = slot_at(rtt_of(L), L.t0, L.kv_end, last, lane), s_even;
  TileCursor S = next_tile<kTile8>(a, w, L, s1, lane);

  // after tile C is computed: shift the cursors and, on entering a new
  // segment, write the finished one out and restart the softmax state
  auto advance = [&]() -> bool {
    const TileCursor prev = C;
    C = L;
    L = S;
    S = next_tile<kTile8>(a, w, S, s1, lane);
    if (C.seg == prev.seg) return true;
    finish_segment8(a, prev.b, g, prev.part, m, lpart, acc, qi, h, head_ok, j);
    finish_empty8(a, w, prev.seg + 1, C.seg, s1, g, qi, h, head_ok, j, lane);
    if (C.seg >= s1) return false;
    load_q8(a, qop, qscale, C.b, qi, h, head_ok, j);
    m = kNegInf;
    lpart = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    return true;
  };

  for (;;) {
    s_even = slot_at(rtt_of(S), S.t0, S.kv_end, last, lane);
    load_tile8<STREAM>(tb, s_odd, L.t0, L.kv_end, sfk_of(L), a.k_block, kbase, vbase, row_bytes, lane);
    __builtin_amdgcn_sched_barrier(0);  // the loads above stay ahead of this tile's math
    compute(ta, C.t0, MULTI ? min(C.kv_end, C.lim + qi + 1) : C.kv_end);
    if (!advance()) break;
    s_odd = slot_at(rtt_of(S), S.t0, S.kv_end, last, lane);
    load_tile8<STREAM>(ta, s_even, L.t0, L.kv_end, sfk_of(L), a.k_block, kbase, vbase, row_bytes, lane);
    __builtin_amdgcn_sched_barrier(0);
    compute(tb, C.t0, MULTI ? min(C.kv_end, C.lim + qi + 1) : C.kv_end);
    if (!advance()) break;
  }
}

// WPB units of one chunk per workgroup, as in the bf16 decode.
template <int WPB, bool MULTI, bool I8, bool STREAM>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(2))) void decode_fp8_kernel(DecodeArgs a) {
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
  decode_fp8_chunk<MULTI, I8, STREAM>(a, s0, s1, unit, win_rec[wv], win_req[wv]);
}

// Kernel instance for wpb waves per workgroup and the load form; fewer than
// 8 units always stream (decode_streams).
template <bool MULTI, bool I8>
const void* decode_fp8_kernel_for(int wpb, bool stream) {
  if (wpb == 8)
    return stream ? (const void*)decode_fp8_kernel<8, MULTI, I8, true> : (const void*)decode_fp8_kernel<8, MULTI, I8, false>;
  return wpb == 4 ? (const void*)decode_fp8_kernel<4, MULTI, I8, true>
       : wpb == 2 ? (const void*)decode_fp8_kernel<2, MULTI, I8, true> : (const void*)decode_fp8_kernel<1, MULTI, I8, true>;
}

static const void* decode_fp8_kernel_of(bool multi, bool qk_int8, int wpb, bool stream) {
  if (multi) return qk_int8 ? decode_fp8_kernel_for<true, true>(wpb, stream) : decode_fp8_kernel_for<true, false>(wpb, stream);
  return qk_int8 ? decode_fp8_kernel_for<false, true>(wpb, stream) : decode_fp8_kernel_for<false, false>(wpb, stream);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, bool qk_int8, int64_t capacity, int32_t batch, hipStream_t s) {
  // head_dim 128 only (validated by the host API)
  if (capacity <= 0 || batch <= 0) return hipSuccess;
  const int units = a.hkv * a.head_groups;
  const int wpb = decode_waves_per_block(units);
  const void* k = decode_fp8_kernel_of(a.q_len > 1, qk_int8, wpb, decode_streams(units));
  DecodeArgs args = a;
  void* kargs[] = {&args};
  const hipError_t e = hipLaunchKernel(k, dim3((unsigned)(capacity * ceil_div(units, wpb))), dim3(64 * wpb), kargs, 0, s);
  const hipError_t last = hipGetLastError();  // also clears what the launch left
  return e != hipSuccess ? e : last;
}

hipError_t decode_fp8_resident_items(int units, bool qk_int8, int64_t* items) {
  const int wpb = decode_waves_per_block(units);
  return resident_items_of(decode_fp8_kernel_of(false, qk_int8, wpb, decode_streams(units)), wpb, units, items);
}

}  // namespace pkv
