// Split-KV merge, a second kernel of the decode call.
//
// Every split of a request that has more than one split writes its
// normalised partial output O_s and its log2-sum-exp to scratch; the merge
// combines them with log-sum-exp algebra, lse = log Σ_s exp(lse_s) and
// O = Σ_s exp(lse_s - lse)·O_s, in a fixed order (deterministic).  The merge
// runs as its own launch because the kernel boundary is the cheap way to make
// the partials of every XCD visible: an in-kernel "last split merges" scheme
// needs a device-scope release per wave, which writes back the L2 each time.
#pragma once

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// Requests with a few splits each: one wave per (request, output row of the
// request, query head) of a request with more than one split, in one pass.
// Lane = (split group sg = lane / 16, channel group c = lane % 16 holding 8
// channels): the lane folds splits sg, sg + 4, ... into a running
// log-sum-exp (max M, weight sum T, weighted O), with every split's loads
// independent of the arithmetic; the four split groups are then combined by
// xor shuffles in a fixed order, so the result is run-to-run deterministic.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_few_kernel(DecodeArgs a) {
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

// Requests with many splits: one workgroup of NW waves per (request, output
// row of the request, query head) of a request with more than one split, in
// two passes:
//  1. every wave reads all the split lse values (lane-parallel, four loads in
//     flight per lane) and forms their maximum M and total T = Σ_s 2^(lse_s-M)
//     with xor butterflies, so the waves agree bit for bit;
//  2. split group sg = 4·wave + lane / 16 and channel group c = lane % 16
//     (8 channels) sum 2^(lse_s - M)·O_s over the splits sg, sg + 4·NW, ...;
//     the weights are fixed, so the loads of successive splits do not wait
//     on one another.  The split groups are added in a fixed order (xor
//     shuffles in the wave, then the waves in index order through LDS), so the
//     result is run-to-run deterministic.
// For requests with dozens or hundreds of splits (one long request holds the
// whole device); the one-pass kernel above is faster when there are few.
constexpr int kMergeLoads = 4;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_merge_many_kernel(DecodeArgs a) {
  // y = (new token i) * Hq + query head: the request's output row i, head h
  const int b = blockIdx.x, y = blockIdx.y;
  const int rows = a.q_len * a.hq;
  const int32_t* __restrict__ req = a.ws + a.req_off;
  const int num = a.ws[WS_NUM_ITEMS];
  const int s0 = req[b];
  const int s1 = req[b + 1] < num ? req[b + 1] : num;
  const int ns = s1 - s0;
  if (ns <= 1) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float* __restrict__ lse_p = a.part_lse + (int64_t)s0 * rows + y;

  // pass 1: M and T over all splits
  float M = kNegInf, T = 0.f;
  for (int base = lane; base < ns; base += 64 * kMergeLoads) {
    float v[kMergeLoads];
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k) {
      const int s = base + 64 * k;
      v[k] = s < ns ? lse_p[(int64_t)s * rows] : kNegInf;
    }
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k) {
      if (v[k] == kNegInf) continue;  // an empty split contributes nothing
      if (v[k] > M) {
        T *= exp2_fast(M - v[k]);  // 0 while M is -inf
        M = v[k];
      }
      T += exp2_fast(v[k] - M);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float Mo = __shfl_xor(M, off), To = __shfl_xor(T, off);
    const float Mn = fmaxf(M, Mo);
    const float sa = M == kNegInf ? 0.f : exp2_fast(M - Mn), sb = Mo == kNegInf ? 0.f : exp2_fast(Mo - Mn);
    T = T * sa + To * sb;
    M = Mn;
  }
  T = __shfl(T, 0, 64);  // M agrees in every lane; T up to rounding: take lane 0's

  // pass 2: the weighted sum of the partial outputs (all weights 0 when
  // every split is empty, M = -inf)
  const int sg = wv * 4 + (lane >> 4), cg = lane & 15;
  const bool d_ok = (D == 128) || (cg < D / 8);
  const float* __restrict__ po_base = a.part_o + ((int64_t)s0 * rows + y) * D + 8 * (d_ok ? cg : 0);
  floatx4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int base = sg; base < ns; base += 4 * NW * kMergeLoads) {
    float ls[kMergeLoads];
    floatx4 p0[kMergeLoads], p1[kMergeLoads];
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k) {
      const int s = base + 4 * NW * k;
      const int sl = s < ns ? s : 0;  // out-of-range slots read split 0 and weigh 0
      const float* po = po_base + (int64_t)sl * rows * D;
      ls[k] = s < ns ? lse_p[(int64_t)sl * rows] : kNegInf;
      p0[k] = *reinterpret_cast<const floatx4*>(po);
      p1[k] = *reinterpret_cast<const floatx4*>(po + 4);
    }
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k) {
      // partial outputs are finite (an empty split stores zeros)
      const float w = ls[k] == kNegInf ? 0.f : exp2_fast(ls[k] - M);
      o0 += w * p0[k];
      o1 += w * p1[k];
    }
  }
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    floatx4 q0, q1;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      q0[k] = __shfl_xor(o0[k], off);
      q1[k] = __shfl_xor(o1[k], off);
    }
    o0 += q0;
    o1 += q1;
  }
  {
    __shared__ floatx4 red[NW - 1][16][2];
    if (wv > 0 && lane < 16) {
      red[wv - 1][lane][0] = o0;
      red[wv - 1][lane][1] = o1;
    }
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) {
      o0 += red[w][cg][0];
      o1 += red[w][cg][1];
    }
  }
  if (lane >= 16) return;
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

// Waves per merge workgroup for a batch whose work list holds up to
// `capacity` segments: 1 (the one-pass kernel) when requests have a few
// splits each, 4 or 8 (the two-pass kernel) when one request can have dozens
// or hundreds.
inline int merge_waves(int64_t capacity, int64_t batch) {
  const int64_t per = batch > 0 ? capacity / batch : capacity;
  return per >= 64 ? 8 : (per >= 16 ? 4 : 1);
}

}  // namespace pkv
