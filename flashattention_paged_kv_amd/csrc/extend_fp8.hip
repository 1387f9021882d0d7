// EXTEND with 8-bit (OCP E4M3) K/V, the Sage formula of the FlashInfer PrimTS
// Sage page (README block, code §1 and §4) for the new-token rows of a batch:
//
//   S = sm_scale · sfQ[t,h] · sfK[b,g,⌊j/k_block⌋] · (q8 · k8_j),  j <= p_b + i
//   P8 = E4M3(448 · exp(S - m)),  l = Σ exp(S - m)  (unquantised)
//   O = sfV[b,g,:] · (Σ_j P8_j · v8_j) / (448 · l)  (+ v_mean[b,g,:])
//
// One sfQ per row (the page's default q_block = 1).  The structure is the
// bf16 extend's (work item = request, query tile, kv head; 256 rows as 8
// waves x 32 rows; key tiles staged through LDS by direct global -> LDS
// loads, 2-stage ring; causal mask bottom-right aligned), with 8-bit tiles
// (128 bytes per row) and the gfx950 fp8 MFMA 32x32x64
// (f8f6f4, unit block scales); 8-bit rows let a 2-stage ring hold 256-key
// tiles, computed in four 64-key parts:
//  * Sᵀ = K8·Q8ᵀ: K rows from LDS are the A operand (32 bytes per lane),
//    the wave's Q8 rows the B operand (registers); each lane gets one row
//    and 16 keys of every 32-key block, as in the bf16 kernel.  The Q and K
//    scales (positive, as quantisation scales are) enter before the row max:
//    per 16-key sub-block (sfK staged in LDS with the slot indices) the max
//    raw score times the sub-block's factor, and fma(raw, factor, -m) in the
//    exponent.
//  * The reference max m is never below a score already seen, so 448·p never
//    exceeds 448 and P8 is a plain E4M3 conversion of fp32 448·p (the 448
//    rides in the exponent).  When a row's max passes m, m moves to that max
//    plus a power-of-two headroom, so later small rises skip the rescale.
//  * Oᵀ += V8ᵀ·P8ᵀ: the contraction runs over the 64 keys in the order each
//    lane holds its probabilities, (32-key block, 8-key group, 4 keys); the
//    V8ᵀ operands are gathered in that same order by 8-bit transposing LDS
//    reads (ds_read_b64_tr_b8: a 16-lane group reads 8 rows of 16 bytes and
//    lane c receives byte c of every row), whose source rows are chosen per
//    lane to be exactly those keys.
// The epilogue applies sfV per channel, 1/(448 l) and v_mean.
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int D8 = 128;                 // head_dim (bytes per 8-bit row)
constexpr int kBN8 = 256;               // keys per tile, computed in four 64-key parts
constexpr int kHalf8 = 64;
constexpr int kParts8 = kBN8 / kHalf8;
constexpr int kWaves8 = kExtendRows / 32;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kStages8 = 2;
constexpr int kSlotStages8 = 3;
constexpr float kLog2_448 = 8.807354922057604f;
constexpr float kHeadroom8 = 2.f;  // log2 units above a new row max

struct Smem8 {
  static constexpr int RB = D8;                        // bytes per key row
  static constexpr int MAT = kBN8 * RB;                // one matrix tile (32 KB)
  static constexpr int VOFF = kStages8 * MAT;          // V tiles follow the K tiles
  static constexpr int ROWS_PER_KB = 1024 / RB;        // rows written by one 64-lane 16-byte load (8)
  static constexpr int NQ = kBN8 / ROWS_PER_KB / kWaves8;  // such loads per wave and matrix (4)
  static constexpr int SLOT_BYTES = kBN8 * 4;          // req_to_token entries of a tile
  static constexpr int SFK_BYTES = 256;                // sfK of the tile's 16-key sub-blocks (16 used)
  static constexpr int SLOT0 = 2 * kStages8 * MAT;
  static constexpr int SFK0 = SLOT0 + kSlotStages8 * SLOT_BYTES;
  static constexpr int TOTAL = SFK0 + kSlotStages8 * SFK_BYTES;
};

// 16-byte chunk c of key row r sits at chunk position c ^ swz8(r).  Two
// 128-byte rows share one 256-byte line of the LDS banks, so a row's bank
// group is its chunk position plus 8 for odd rows.  The mask takes bits 1..3
// of r, permuted (bit 1 -> bit 0, bit 2 -> bit 1, bit 3 -> bit 2), XOR the
// row's parity:
//  * K reads (16 consecutive rows, one chunk column, per 16 lanes): the even
//    rows take 8 distinct positions and so do the odd ones, so the 16 rows
//    cover the 16 bank groups;
//  * transposing V reads (rows {0..3, 8..11} or {4..7, 12..15} of a 16-key
//    window, one chunk column per 16 lanes, columns c and c + 1 side by side
//    in 32 lanes): the masks of a row set differ in bits 1..2 within each
//    parity and in bit 0 across parities, so the positions are distinct
//    within 16 lanes and within 32 lanes.
// The mask depends on r % 16 only, so rows 16, 32, ... further take the same
// per-lane offsets plus an immediate.
__device__ __forceinline__ int swz8(int row) {
  const int h = row >> 1;
  return (((h & 1) << 1) | (h & 4) | ((h >> 1) & 1)) ^ (row & 1);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ u32x2 lds_read_tr8(const char* base, uint32_t off) {
  lds_char* p = (lds_char*)(const_cast<char*>(base)) + off;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2*>(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ floatx16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, floatx16 c) {
  // fp8 E4M3 for both operands (format 0), block scales 2^0 (E8M0 127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0,1 (OCP E4M3, nearest even)
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);       // bytes 2,3
  return (uint32_t)w;
}

__device__ __forceinline__ int tile_row8(int wave, int q, int lane) {
  return (wave * Smem8::NQ + q) * Smem8::ROWS_PER_KB + lane / 8;
}

__device__ __forceinline__ void read_slots8(const char* slots, int wave, int lane, int (&sv)[Smem8::NQ]) {
#pragma unroll
  for (int q = 0; q < Smem8::NQ; ++q) sv[q] = *reinterpret_cast<const int*>(slots + 4 * tile_row8(wave, q, lane));
}

__device__ __forceinline__ void issue_rows8(const int (&sv)[Smem8::NQ], char* stage, const uint8_t* __restrict__ kbase,
                                            const uint8_t* __restrict__ vbase, uint32_t row_bytes, uint32_t last_slot,
                                            int wave, int lane) {
  const int p = lane & 7;
#pragma unroll
  for (int q = 0; q < Smem8::NQ; ++q) {
    const int r = tile_row8(wave, q, lane);
    const int64_t off = row_offset(clamp_slot_u32(sv[q], last_slot), row_bytes) + 16 * (p ^ swz8(r));
    const uint32_t dst = lds_addr(stage) + (wave * Smem8::NQ + q) * 1024;
    dma16(kbase + off, dst);
    dma16(vbase + off, dst + Smem8::VOFF);
  }
}

// req_to_token entries of a tile's 256 keys and the sfK of its sixteen 16-key
// sub-blocks (one wave; positions past kv_end read the last valid entry).
__device__ __forceinline__ void issue_slots8(const int32_t* __restrict__ rtt_row, const float* __restrict__ sfk_row,
                                             int k_block, int t0, int kv_end, char* slot_stage, char* sfk_stage,
                                             int lane) {
#pragma unroll
  for (int c = 0; c < kBN8 / 64; ++c) dma4(rtt_row + min(t0 + 64 * c + lane, kv_end - 1), lds_addr(slot_stage) + 256 * c);
  dma4(sfk_row + min(t0 + 16 * (lane & 15), kv_end - 1) / k_block, lds_addr(sfk_stage));
}

__device__ __forceinline__ void zero_rows_past_end8(char* stage, int t0, int kv_end, int wave, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < Smem8::NQ; ++q) {
    if (t0 + tile_row8(wave, q, lane) >= kv_end) {
      char* dst = stage + (wave * Smem8::NQ + q) * 1024 + 16 * lane;
      *reinterpret_cast<u32x4*>(dst) = z;
      *reinterpret_cast<u32x4*>(dst + Smem8::VOFF) = z;
    }
  }
}

struct RowState8 {
  floatx16 acc[D8 / 32];
  float m, lpart;
};

}  // namespace

template <int UNUSED>
__global__ __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2))) void extend_fp8_kernel(ExtendArgs a) {
  using S = Smem8;
  __shared__ __attribute__((aligned(1024))) char smem[S::TOTAL];

  const int32_t* __restrict__ ws = a.ws;
  const int xi = (int)blockIdx.x / a.hkv;  // 1-D grid as in the bf16 extend: one kv head per XCD
  if (xi >= ws[WS_NUM_ITEMS]) return;
  const int4 it = reinterpret_cast<const int4*>(ws + a.items_off)[xi];
  const int b = it.x, qt = it.y, kv_end = it.z;
  const int g = (int)blockIdx.x - xi * a.hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, jh = lane >> 5;

  int64_t q0 = a.cu_seqlens_q[b], q1 = a.cu_seqlens_q[b + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
  const int n = (int)(q1 - q0);
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_kv_len ? a.max_kv_len : L);
  const int p = L - n;
  const int bt = a.block_tokens;

  const int row = wave * 32 + l32;
  const int hl = row / bt;
  const int ti = qt * bt + (row - hl * bt);
  const bool row_ok = hl < a.group && ti < n;
  const int h = g * a.group + (hl < a.group ? hl : 0);
  const int pos = p + (row_ok ? ti : (n > 0 ? n - 1 : 0));
  int wave_max_pos = pos, wave_min_pos = pos;
#pragma unroll
  for (int sh = 1; sh < 32; sh <<= 1) {
    wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, sh));
    wave_min_pos = min(wave_min_pos, __shfl_xor(wave_min_pos, sh));
  }

  // Q8 rows as the B operand: lane holds q8[row][64 ks + 32 jh .. +32]; the
  // row's score factor sm_scale·log2(e)·sfQ
  i32x8 qop[2];
  float rowc = 0.f;
  {
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + ((q0 + (row_ok ? ti : 0)) * a.hq + h) * (int64_t)D8;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 lo = row_ok ? ldg16(qrow + 64 * ks + 32 * jh) : z;
      const u32x4 hi = row_ok ? ldg16(qrow + 64 * ks + 32 * jh + 16) : z;
      qop[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    if (row_ok) rowc = a.sfq[(q0 + ti) * a.hq + h] * a.scale_log2;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // Q landed here, not "outstanding" inside the loop
  }

  const int row_idx = a.rpi ? a.rpi[b] : b;
  const int32_t* __restrict__ rtt_row = a.rtt + (int64_t)row_idx * a.rtt_stride;
  const float* __restrict__ sfk_row = a.sfk + ((int64_t)b * a.hkv + g) * a.sfk_stride;
  const uint32_t row_bytes = (uint32_t)(a.hkv * D8);
  const uint32_t last_slot = (uint32_t)(a.pool_slots - 1);
  const uint8_t* __restrict__ kbase = static_cast<const uint8_t*>(a.k_pool) + (int64_t)g * D8;
  const uint8_t* __restrict__ vbase = static_cast<const uint8_t*>(a.v_pool) + (int64_t)g * D8;

  RowState8 rs;
#pragma unroll
  for (int db = 0; db < D8 / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) rs.acc[db][r] = 0.f;
  rs.m = kNegInf;
  rs.lpart = 0.f;

  // per-lane LDS offsets.  K: key l32 (+32 kb, +64 per half: immediates),
  // 16-byte chunks 4 ks + 2 jh + u.  V (transposing reads): 16-lane group
  // q16 = lane / 16 serves channels 32 db + 16 (q16 % 2) .. +16 and key half
  // jh; its lane i16 names source row e = i16 / 2 (key 8 (e / 4) + 4 jh + e % 4
  // of the read's 16-key window) and the 8-byte half i16 % 2 of the chunk.
  int ko[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int u = 0; u < 2; ++u) ko[ks][u] = l32 * S::RB + (((4 * ks + 2 * jh + u) ^ swz8(l32)) << 4);
  int vo[D8 / 32];
  {
    const int q16 = lane >> 4, i16 = lane & 15, e = i16 >> 1, hb = i16 & 1;
    const int key = 8 * (e >> 2) + 4 * (q16 >> 1) + (e & 3);
#pragma unroll
    for (int db = 0; db < D8 / 32; ++db)
      vo[db] = opaque(S::VOFF + key * S::RB + (((2 * db + (q16 & 1)) ^ swz8(key)) << 4) + 8 * hb);
  }

  char* const kv0 = smem;
  auto slot_stage = [&](int u) { return smem + S::SLOT0 + (u % kSlotStages8) * S::SLOT_BYTES; };
  auto sfk_stage = [&](int u) { return smem + S::SFK0 + (u % kSlotStages8) * S::SFK_BYTES; };
  const int ntiles = (kv_end + kBN8 - 1) / kBN8;

  if (ntiles > 0) {
    if (wave == 0) {
      for (int t = 0; t < 2 && t < ntiles; ++t)
        issue_slots8(rtt_row, sfk_row, a.k_block, t * kBN8, kv_end, slot_stage(t), sfk_stage(t), lane);
      wait_vmem<0>();
    }
    __syncthreads();
    int sv[S::NQ];
    read_slots8(slot_stage(0), wave, lane, sv);
    issue_rows8(sv, kv0, kbase, vbase, row_bytes, last_slot, wave, lane);
    wait_vmem<0>();
    zero_rows_past_end8(kv0, 0, kv_end, wave, lane);
  }
  __syncthreads();

  // one 64-key part: scores, scales, mask, reference max, P8, PV
  auto half = [&](const char* kt, const char* st, const float* sfk4, int t0h, bool masked, auto&& mid)
      __attribute__((always_inline)) {
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* kr = kt + 32 * kb * S::RB;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kr + ko[ks][0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kr + ko[ks][1]);
        const i32x8 kop = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[kb] = mfma_fp8_32x32x64(kop, qop[ks], ks == 0 ? floatx16{} : s[kb]);
      }
      if (kb == 0) mid();
    }
    // scores in log2 units are raw · f_sb, f_sb = sm_scale·log2(e)·sfQ·sfK of
    // the key's 16-key sub-block sb; with positive scales the row max is the
    // largest of (max raw score of sb) · f_sb, and the exponentials take
    // fma(raw, f_sb, -m) below, so no score is scaled on its own
    float f[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) f[sb] = rowc * sfk4[sb];
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) <= pos - t0h - 4 * jh ? s[kb][r] : kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int kb = sb >> 1, r0 = 8 * (sb & 1);
      float m3 = fmaxf(fmaxf(s[kb][r0], s[kb][r0 + 1]), s[kb][r0 + 2]);
      m3 = fmaxf(fmaxf(m3, s[kb][r0 + 3]), s[kb][r0 + 4]);
      m3 = fmaxf(fmaxf(m3, s[kb][r0 + 5]), s[kb][r0 + 6]);
      m3 = fmaxf(m3, s[kb][r0 + 7]);
      mx = fmaxf(mx, m3 * f[sb]);
    }
    mx = max_xor32(mx);
    // reference max with headroom: when a row's max passes it, it moves to
    // that max plus kHeadroom8, so most tiles skip the rescale; every score
    // stays at or below it, so 448·p <= 448 for every quantised probability
    // (the power-of-two headroom only shifts the codes' exponents)
    if (__any(mx > rs.m)) {
      const float m_new = mx > rs.m ? mx + kHeadroom8 : rs.m;
      const float alpha = m_new == kNegInf ? 1.f : exp2_fast(rs.m - m_new);
      rs.lpart *= alpha;
#pragma unroll
      for (int db = 0; db < D8 / 32; ++db) rs.acc[db] *= alpha;
      rs.m = m_new;
    }
    // 448·p = exp2(s - m + log2 448): the quantised probability's factor rides
    // in the exponent, so P8 is a plain conversion and l sums 448·p
    const float mu = (rs.m == kNegInf ? 0.f : rs.m) - kLog2_448;
    // P8ᵀ operand: dword 4 kb + q holds keys 32 kb + 8 q + 4 jh + 0..3
    i32x8 pop;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[kb][4 * q + e], f[2 * kb + (q >> 1)], -mu));
        rs.lpart += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        pop[4 * kb + q] = (int)pack_fp8x4(pv[0], pv[1], pv[2], pv[3]);
      }
    // Oᵀ += V8ᵀ·P8ᵀ: V8ᵀ dwords (2 rd, 2 rd + 1) come from transposing read rd
    // over keys 32 (rd / 2) + 16 (rd % 2) .. +16 (8-key groups 2 rd, 2 rd + 1)
#pragma unroll
    for (int db = 0; db < D8 / 32; ++db) {
      i32x8 vop;
#pragma unroll
      for (int rd = 0; rd < 4; ++rd) {
        const u32x2 w = lds_read_tr8(st + 16 * rd * S::RB, vo[db]);
        vop[2 * rd] = (int)w[0];
        vop[2 * rd + 1] = (int)w[1];
      }
      rs.acc[db] = mfma_fp8_32x32x64(vop, pop, rs.acc[db]);
    }
  };
  auto nothing = [&]() __attribute__((always_inline)) {};

  auto step = [&](int tile, auto J_) __attribute__((always_inline)) {
    constexpr int J = decltype(J_)::value;
    constexpr int J1 = (J + 1) % 2;
    const int t0 = tile * kBN8;
    const bool sl2 = wave == 0 && tile + 2 < ntiles;
    const bool kv1 = tile + 1 < ntiles;
    int sv[S::NQ];
    if (kv1) read_slots8(slot_stage(tile + 1), wave, lane, sv);
    float sk[4 * kParts8];
#pragma unroll
    for (int c = 0; c < kParts8; ++c) {
      const floatx4 f4 = *reinterpret_cast<const floatx4*>(sfk_stage(tile) + 16 * c);
      sk[4 * c] = f4[0];
      sk[4 * c + 1] = f4[1];
      sk[4 * c + 2] = f4[2];
      sk[4 * c + 3] = f4[3];
    }
    auto loads = [&]() __attribute__((always_inline)) {
      if (sl2)
        issue_slots8(rtt_row, sfk_row, a.k_block, t0 + 2 * kBN8, kv_end, slot_stage(tile + 2), sfk_stage(tile + 2),
                     lane);
      if (kv1) issue_rows8(sv, kv0 + J1 * S::MAT, kbase, vbase, row_bytes, last_slot, wave, lane);
    };
    const char* kt = kv0 + J * S::MAT;
    if (t0 <= wave_max_pos) {
      half(kt, kt, sk, t0, t0 + kHalf8 - 1 > wave_min_pos, loads);
#pragma unroll
      for (int c = 1; c < kParts8; ++c) {
        const int tc = t0 + kHalf8 * c;
        if (tc > wave_max_pos) break;  // causally invisible to every row of the wave
        half(kt + kHalf8 * c * S::RB, kt + kHalf8 * c * S::RB, sk + 4 * c, tc, tc + kHalf8 - 1 > wave_min_pos,
             nothing);
      }
    } else {
      loads();
    }
    wait_vmem<0>();
    if (kv1) zero_rows_past_end8(kv0 + J1 * S::MAT, t0 + kBN8, kv_end, wave, lane);
    __syncthreads();
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    step(tile, std::integral_constant<int, 0>());
    if (tile + 1 < ntiles) step(tile + 1, std::integral_constant<int, 1>());
  }
  wait_vmem<0>();

  // epilogue: Oᵀ[d][row] -> out[token][h][d], with sfV, 1/(448 l) and v_mean
  const float l = rs.lpart + __shfl_xor(rs.lpart, 32);  // 448 · Σ p
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float* sfv = a.sfv + ((int64_t)b * a.hkv + g) * D8;
  const float* vmean = a.v_mean ? a.v_mean + ((int64_t)b * a.hkv + g) * D8 : nullptr;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((q0 + ti) * a.hq + h) * (int64_t)D8;
#pragma unroll
  for (int db = 0; db < D8 / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * db + 8 * rq + 4 * jh;
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = rs.acc[db][4 * rq + k] * inv * sfv[d0 + k] + (vmean ? vmean[d0 + k] : 0.f);
      u32x2 w;
      w[0] = pack_bf16x2(o[0], o[1]);
      w[1] = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<u32x2*>(orow + d0) = w;
    }
  if (jh == 0 && a.lse) a.lse[(q0 + ti) * a.hq + h] = l > 0.f ? (rs.m + __log2f(l) - kLog2_448) * kLn2 : kNegInf;
}

hipError_t launch_extend_fp8(const ExtendArgs& a, int64_t capacity, hipStream_t s) {
  if (capacity <= 0) return hipSuccess;
  dim3 grid((unsigned)(capacity * a.hkv));
  hipLaunchKernelGGL(extend_fp8_kernel<0>, grid, dim3(kThreads8), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
