// Decode work as a stream of tiles.  The plan cuts the requests' KV into
// chunks of equal length, each a short list of request segments; a decode
// workgroup takes one chunk and every wave walks the chunk's tiles as one
// stream, so the loads of the next tiles are in flight across segment
// boundaries.  Shared by the bf16 and the 8-bit decode kernels.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// Position in a chunk's tile stream: segment index, its request and
// req_to_token row, the tile's first token, the segment's end and partial
// index.  seg == s1 once the stream is exhausted; t0 then runs past kv_end,
// so a slot lookup for it clamps to the last token of the last segment.
struct TileCursor {
  int seg, b, row, t0, kv_end, part;
  int lim;  // L_b - q_len: new token i of the request sees keys <= lim + i
};

// The chunk's segment records, staged in the wave's own LDS area (64 at a
// time: entry i is segment base + i).  They are read with one vector load
// before the tile stream starts, so the stream's own loads are never waited
// for behind a record lookup, and they cost no registers while the stream
// runs; a chunk of more than 64 segments reloads the window when a lookup
// falls outside it.
struct SegWindow {
  int base;
  int4* rec;  // [64] (b, kv_begin, kv_end, part)
  int2* req;  // [64] (req_to_token row of b, L_b - q_len)
};

__device__ __forceinline__ void load_window(const DecodeArgs& a, SegWindow& w, int base, int s1, int lane) {
  w.base = base;
  if (base + lane < s1) {
    const int4 it = reinterpret_cast<const int4*>(a.ws + a.items_off)[base + lane];
    w.rec[lane] = it;
    int L = a.seq_lens[it.x];  // clamped exactly as the plan clamps it
    L = L < 0 ? 0 : (L > a.max_kv_len ? a.max_kv_len : L);
    w.req[lane] = make_int2(a.rpi ? a.rpi[it.x] : it.x, L - a.q_len);
  }
}

__device__ __forceinline__ TileCursor seg_at(const DecodeArgs& a, SegWindow& w, int s, int s1, int lane) {
  if ((unsigned)(s - w.base) >= 64u) load_window(a, w, s, s1, lane);
  const int i = s - w.base;
  const int4 r = w.rec[i];
  const int2 q = w.req[i];
  return TileCursor{s,
                    __builtin_amdgcn_readfirstlane(r.x),
                    __builtin_amdgcn_readfirstlane(q.x),
                    __builtin_amdgcn_readfirstlane(r.y),
                    __builtin_amdgcn_readfirstlane(r.z),
                    __builtin_amdgcn_readfirstlane(r.w),
                    __builtin_amdgcn_readfirstlane(q.y)};
}

// The tile after c (tiles of STEP tokens): the next tile of its segment, else the first tile of the
// next non-empty segment of the chunk.  Past the end only seg changes (to
// s1), so the cursor keeps the last non-empty segment's request and range.
template <int STEP>
__device__ __forceinline__ TileCursor next_tile(const DecodeArgs& a, SegWindow& w, TileCursor c, int s1, int lane) {
  c.t0 += STEP;
  if (c.t0 < c.kv_end) return c;
  for (int s = c.seg + 1; s < s1; ++s) {
    const TileCursor n = seg_at(a, w, s, s1, lane);
    if (n.t0 < n.kv_end) return n;
  }
  c.seg = s1;
  return c;
}

// Empty segments (requests with no KV) in [from, to): O = 0, lse = -inf for
// the lane's output row (new token qi, query head h).
template <int D>
__device__ __forceinline__ void finish_empty(const DecodeArgs& a, SegWindow& w, int from, int to, int s1, int qi,
                                             int h, bool head_ok, int j, int lane) {
  qi = opaque(qi);
  h = opaque(h);
  j = opaque(j);
  const bool rows_ok = (D == 128) || (j < 2);
  for (int s = from; s < to; ++s) {
    const TileCursor e = seg_at(a, w, s, s1, lane);
    if (e.part >= 0) {
      const int64_t r0 = ((int64_t)e.part * a.q_len + qi) * a.hq + h;
      if (head_ok && rows_ok) {
        float* po = a.part_o + r0 * D;
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 8; ++r) *reinterpret_cast<floatx4*>(po + 32 * j + 4 * r) = z;
      }
      if (head_ok && j == 0) a.part_lse[r0] = kNegInf;
      continue;
    }
    const int64_t r0 = ((int64_t)e.b * a.q_len + qi) * a.hq + h;
    if (head_ok && rows_ok) {
      uint16_t* orow = static_cast<uint16_t*>(a.out) + r0 * D;
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < 4; ++r) stg16(orow + 32 * j + 8 * r, z);
    }
    if (head_ok && j == 0 && a.lse) a.lse[r0] = kNegInf;
  }
}

}  // namespace pkv
