// Split-KV merge, a second kernel of the decode call.
//
// Every split of a request that has more than one split writes its
// normalised partial output O_s and its log2-sum-exp to scratch; this kernel
// combines them with log-sum-exp algebra, lse = log Σ_s exp(lse_s) and
// O = Σ_s exp(lse_s - lse)·O_s, in a fixed order (deterministic).  The merge
// runs as its own launch because the kernel boundary is the cheap way to make
// the partials of every XCD visible: an in-kernel "last split merges" scheme
// needs a device-scope release per wave, which writes back the L2 each time.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// One wave per (request, output row of the request, query head) of a request
// with more than one split.
// Lane = (split group sg = lane / 16, channel group c = lane % 16 holding 8
// channels): the lane folds splits sg, sg + 4, ... into a running
// log-sum-exp (max M, weight sum T, weighted O), with every split's loads
// independent of the arithmetic; the four split groups are then combined by
// xor shuffles in a fixed order, so the result is run-to-run deterministic.
constexpr int kMergeThreads = 64;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  // y = (new token i) * Hq + query head: the request's output row i, head h
  const int b = blockIdx.x, y = blockIdx.y;
  const int rows = a.q_len * a.hq;
  const int32_t* __restrict__ req = a.ws + a.req_off;
  const int num = a.ws[WS_NUM_ITEMS];
  const int s0 = req[b];
  const int s1 = req[b + 1] < num ? req[b + 1] : num;
  const int ns = s1 - s0;
  if (ns <= 1) return;
  const int lane = threadIdx.x, sg = lane >> 4, cg = lane & 15;
  const bool d_ok = (D == 128) || (cg < D / 8);
  float M = kNegInf, T = 0.f;
  floatx4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = sg; s < ns; s += 4) {
    const float ls = a.part_lse[(int64_t)(s0 + s) * rows + y];
    const float* po = a.part_o + ((int64_t)(s0 + s) * rows + y) * D + 8 * (d_ok ? cg : 0);
    const floatx4 p0 = *reinterpret_cast<const floatx4*>(po), p1 = *reinterpret_cast<const floatx4*>(po + 4);
    if (ls == kNegInf) continue;  // an empty split contributes nothing
    if (ls > M) {
      const float sc = exp2_fast(M - ls);  // 0 while M is -inf
      T *= sc;
      o0 *= sc;
      o1 *= sc;
      M = ls;
    }
    const float w = exp2_fast(ls - M);
    T += w;
    o0 += w * p0;
    o1 += w * p1;
  }
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float Mo = __shfl_xor(M, off);
    const float Mn = fmaxf(M, Mo);
    const float sa = M == kNegInf ? 0.f : exp2_fast(M - Mn), sb = Mo == kNegInf ? 0.f : exp2_fast(Mo - Mn);
    T = T * sa + __shfl_xor(T, off) * sb;
    floatx4 q0, q1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q0[k] = __shfl_xor(o0[k], off);
      q1[k] = __shfl_xor(o1[k], off);
    }
    o0 = o0 * sa + q0 * sb;
    o1 = o1 * sa + q1 * sb;
    M = Mn;
  }
  if (sg != 0) return;
  const float inv = T > 0.f ? 1.f / T : 0.f;
  if (d_ok) {
    u32x4 w;
    w[0] = pack_bf16x2(o0[0] * inv, o0[1] * inv);
    w[1] = pack_bf16x2(o0[2] * inv, o0[3] * inv);
    w[2] = pack_bf16x2(o1[0] * inv, o1[1] * inv);
    w[3] = pack_bf16x2(o1[2] * inv, o1[3] * inv);
    stg16(static_cast<uint16_t*>(a.out) + ((int64_t)b * rows + y) * D + 8 * cg, w);
  }
  if (cg == 0 && a.lse) a.lse[(int64_t)b * rows + y] = T > 0.f ? (M + __log2f(T)) * kLn2 : kNegInf;
}

}  // namespace pkv
