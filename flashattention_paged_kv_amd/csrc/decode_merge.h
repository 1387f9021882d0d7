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

// One 256-thread workgroup per (request, query head) of a request with more
// than one split: sixteen groups of 16 lanes take every 16th split (each lane
// owns 8 channels), then the groups are combined through LDS.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  constexpr int NG = kMergeThreads / 16;
  __shared__ float sh_m[NG];
  __shared__ float sh_t[NG];
  __shared__ floatx4 sh_o[NG][16][2];
  const int b = blockIdx.x, h = blockIdx.y;
  const int32_t* __restrict__ req = a.ws + a.req_off;
  const int num = a.ws[WS_NUM_ITEMS];
  const int s0 = req[b];
  const int s1 = req[b + 1] < num ? req[b + 1] : num;
  const int ns = s1 - s0;
  if (ns <= 1) return;
  const int grp = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const bool d_ok = (D == 128) || (l16 < D / 8);
  float M = kNegInf;
  for (int s = grp; s < ns; s += NG) M = fmaxf(M, a.part_lse[(int64_t)(s0 + s) * a.hq + h]);
  if (l16 == 0) sh_m[grp] = M;
  __syncthreads();
  M = sh_m[0];
#pragma unroll
  for (int k = 1; k < NG; ++k) M = fmaxf(M, sh_m[k]);
  float tot = 0.f;
  floatx4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = grp; s < ns; s += NG) {
    const float ls = a.part_lse[(int64_t)(s0 + s) * a.hq + h];
    const float w = ls == kNegInf ? 0.f : exp2_fast(ls - M);
    tot += w;
    if (d_ok) {
      const float* po = a.part_o + ((int64_t)(s0 + s) * a.hq + h) * D + 8 * l16;
      o0 += w * *reinterpret_cast<const floatx4*>(po);
      o1 += w * *reinterpret_cast<const floatx4*>(po + 4);
    }
  }
  if (l16 == 0) sh_t[grp] = tot;
  sh_o[grp][l16][0] = o0;
  sh_o[grp][l16][1] = o1;
  __syncthreads();
  if (grp != 0) return;
  tot = 0.f;
  o0 = floatx4{0.f, 0.f, 0.f, 0.f};
  o1 = o0;
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    tot += sh_t[k];
    o0 += sh_o[k][l16][0];
    o1 += sh_o[k][l16][1];
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (d_ok) {
    u32x4 w;
    w[0] = pack_bf16x2(o0[0] * inv, o0[1] * inv);
    w[1] = pack_bf16x2(o0[2] * inv, o0[3] * inv);
    w[2] = pack_bf16x2(o1[0] * inv, o1[1] * inv);
    w[3] = pack_bf16x2(o1[2] * inv, o1[3] * inv);
    stg16(static_cast<uint16_t*>(a.out) + ((int64_t)b * a.hq + h) * D + 8 * l16, w);
  }
  if (l16 == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : kNegInf;
}

}  // namespace pkv
