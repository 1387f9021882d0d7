// EXTEND: causal varlen attention of new tokens over their request's cached
// prefix and themselves, bf16 inputs, fp32 accumulation, bf16 MFMA on gfx950.
//
// The score matrix never leaves the chip (FlashAttention page, §2): a
// workgroup walks the key range in 64-key tiles, gathers each K and V tile
// through req_to_token into LDS (double buffered, staged through registers
// one tile ahead), and keeps a running max / sum per row (online softmax).
//
// Work item = (request b, query tile t, kv head g).  Its 128 rows are the
// (query head, token) pairs of the G query heads that share kv head g, for
// block = 128 / G consecutive new tokens (head-major rows), so every K/V byte
// gathered into LDS serves all G heads.  Four waves own 32 rows each.
//
// Per wave and key tile, with 32x32x16 bf16 MFMAs:
//  * Sᵀ = K·Qᵀ: K rows from LDS are the A operand (16-byte reads), the
//    wave's Q rows the B operand (registers).  The Sᵀ layout gives each lane
//    ONE row and 16 keys of every 32-key block, so the row max / sum are
//    per-lane plus one xor-32 shuffle, and P is already in the Pᵀ B-operand
//    layout of the next product;
//  * Oᵀ += Vᵀ·Pᵀ: the Vᵀ A operand is read from the row-major V tile with the
//    LDS transpose read (ds_read_b64_tr_b16: each 16-lane group receives a
//    4-key x 16-channel block transposed), in the key order of the Sᵀ
//    output.
// Causal mask (bottom-right aligned): row token i of a request with prefix
// p sees keys 0..p+i; key tiles entirely above a wave's rows skip the MFMAs.
#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kBN = kExtendTileN;  // keys per tile (64)
constexpr int kThreads = 256;      // 4 waves x 32 rows

// One stage holds a K tile and a V tile, rows of D*2 bytes, unpadded.  The
// 16-byte chunk c of key row r sits at chunk position c ^ (r % CH): rows of
// consecutive keys start on different banks, so 16-byte K row reads and the
// 8-byte transpose reads of V are free of bank conflicts.
template <int D>
struct ExtSmem {
  static constexpr int RB = D * 2;          // bytes per key row
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int MAT = kBN * RB;      // one matrix tile
  static constexpr int STAGE = 2 * MAT;     // K then V
  static constexpr int ROWS_PER_KB = 1024 / RB;  // rows written by one 64-lane 16-byte load
};

template <int D>
__device__ __forceinline__ int swz_off(int row, int chunk) {
  return row * ExtSmem<D>::RB + ((chunk ^ (row & (ExtSmem<D>::CH - 1))) << 4);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x2 lds_read_tr16(const char* base, uint32_t off) {
  // transposing 8-byte LDS read (gfx950): see the kernel header
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* p = (lds_char*)(const_cast<char*>(base)) + off;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Full tiles go global -> LDS directly (gfx950 global_load_lds_dwordx4): each
// 64-lane load writes 1 KiB of consecutive LDS, lane i at byte 16 i, i.e.
// row i / CH, chunk position i % CH; the lane fetches the global chunk that
// the swizzle puts there.  No registers, no LDS store instructions.
template <int D>
struct TileSlots {
  static constexpr int NQ = kBN / ExtSmem<D>::ROWS_PER_KB / 4;  // 16-byte loads per lane per matrix
  int s[NQ];  // raw req_to_token entries; -1 past kv_end (clamped when used)
};

// Row of the tile handled by (wave, load q, lane); the lane writes LDS chunk
// position lane % CH of that row and so fetches global chunk (lane % CH) ^ swizzle.
template <int D>
__device__ __forceinline__ int tile_row(int wave, int q, int lane) {
  return (wave * TileSlots<D>::NQ + q) * ExtSmem<D>::ROWS_PER_KB + lane / ExtSmem<D>::CH;
}

template <int D>
__device__ __forceinline__ int tile_chunk(int row, int lane) {
  return (lane % ExtSmem<D>::CH) ^ (row & (ExtSmem<D>::CH - 1));
}

template <int D>
__device__ __forceinline__ void load_tile_slots(TileSlots<D>& sl, const int32_t* __restrict__ rtt_row, int t0,
                                                int kv_end, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < TileSlots<D>::NQ; ++q) {
    const int key = t0 + tile_row<D>(wave, q, lane);
    sl.s[q] = key < kv_end ? rtt_row[key] : -1;
  }
}

template <int D>
__device__ __forceinline__ void dma_tile(const TileSlots<D>& sl, char* stage, const uint16_t* __restrict__ kbase,
                                         const uint16_t* __restrict__ vbase, int64_t row_elems, int64_t pool_slots,
                                         int wave, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int q = 0; q < TileSlots<D>::NQ; ++q) {
    const int r = tile_row<D>(wave, q, lane);
    const int64_t slot = clamp_slot(sl.s[q], pool_slots);  // rows past kv_end read a valid row
    const int64_t off = slot * row_elems + 8 * tile_chunk<D>(r, lane);
    char* dst = stage + (wave * TileSlots<D>::NQ + q) * 1024;
    __builtin_amdgcn_global_load_lds(kbase + off, (lds_void*)dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vbase + off, (lds_void*)(dst + ExtSmem<D>::MAT), 16, 0, 0);
  }
}

// Rows past kv_end (only in a request's last, partial tile) are fetched from a
// clamped slot and then overwritten with zeros by the wave that fetched them,
// after its own loads have landed: a poisoned V row times a zero probability
// would still be NaN.  Bit q of the mask marks load q of this lane as such a row.
template <int D>
__device__ __forceinline__ int invalid_mask(const TileSlots<D>& sl) {
  int mask = 0;
#pragma unroll
  for (int q = 0; q < TileSlots<D>::NQ; ++q) mask |= (sl.s[q] < 0) << q;
  return mask;
}

template <int D>
__device__ __forceinline__ void zero_invalid_rows(int mask, char* stage, int wave, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < TileSlots<D>::NQ; ++q)
    if (mask & (1 << q)) {
      char* dst = stage + (wave * TileSlots<D>::NQ + q) * 1024 + 16 * lane;
      *reinterpret_cast<u32x4*>(dst) = z;
      *reinterpret_cast<u32x4*>(dst + ExtSmem<D>::MAT) = z;
    }
}

__device__ __forceinline__ void wait_vmem_all() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace

// Per-row state and the compute of one key tile (Sᵀ, mask, online softmax, Oᵀ).
template <int D>
struct RowState {
  floatx16 acc[D / 32];
  float m, lpart;
};

template <int D>
__device__ __forceinline__ void compute_tile(RowState<D>& rs, const char* cur, const u32x4 (&qop)[D / 16], int t0,
                                             int pos, int wave_min_pos, float c, int lane) {
  constexpr int QK_STEPS = D / 16;
  constexpr int DB = D / 32;
  const int l32 = lane & 31, jh = lane >> 5;
  // ---- Sᵀ for two 32-key blocks (raw scores; the scale is folded in below)
  floatx16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    const int key = 32 * kb + l32;
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(cur + swz_off<D>(key, 2 * ks + jh));
      s[kb] = mfma32x32x16(as_bf16x8(kv), as_bf16x8(qop[ks]), s[kb]);
    }
  }
  // ---- causal mask only where the tile crosses some row's diagonal
  if (t0 + kBN - 1 > wave_min_pos) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * jh + (r & 3);
        s[kb][r] = key <= pos ? s[kb][r] : kNegInf;
      }
  }
  float mx = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
  // ---- lazy rescale: the reference max moves only when a row's max exceeds it
  //      by more than 8 (log2 units), so exp2(s - m) <= 256 while acc and l keep
  //      referring to the same m
  if (__any(mx > rs.m + 8.f)) {
    const float m_new = fmaxf(rs.m, mx);
    const float alpha = m_new == kNegInf ? 1.f : exp2_fast(rs.m - m_new);
    rs.lpart *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) rs.acc[db] *= alpha;
    rs.m = m_new;
  }
  const float m_use = rs.m == kNegInf ? 0.f : rs.m;
  float ps = 0.f;
  u32x4 pop[4];  // Pᵀ B operands, one per 16-key k-step
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = exp2_fast(__builtin_fmaf(s[kb][8 * half + e], c, -m_use));
        ps += pv[e];
      }
      u32x4 w;
      w[0] = pack_bf16x2(pv[0], pv[1]);
      w[1] = pack_bf16x2(pv[2], pv[3]);
      w[2] = pack_bf16x2(pv[4], pv[5]);
      w[3] = pack_bf16x2(pv[6], pv[7]);
      pop[2 * kb + half] = w;
    }
  rs.lpart += ps;
  // ---- Oᵀ += Vᵀ·Pᵀ.  k-step ks2 covers keys 16 ks2 .. +16; this lane's 8 keys are
  //      {16 ks2 + 8 (e/4) + 4 jh + e%4}: two transposed 4-key reads
  const int g16 = lane >> 4, i16 = lane & 15;
  const int dsub = 16 * (g16 & 1);
  const int jj = g16 >> 1;
  const char* vt = cur + ExtSmem<D>::MAT;
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    const int key_a = 16 * ks2 + 4 * jj + (i16 >> 2);
    const int key_b = key_a + 8;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + dsub + 4 * (i16 & 3);
      const u32x2 va = lds_read_tr16(vt, swz_off<D>(key_a, col >> 3) + ((col & 7) << 1));
      const u32x2 vb = lds_read_tr16(vt, swz_off<D>(key_b, col >> 3) + ((col & 7) << 1));
      u32x4 vop = {va[0], va[1], vb[0], vb[1]};
      rs.acc[db] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(pop[ks2]), rs.acc[db]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void extend_bf16_kernel(ExtendArgs a) {
  constexpr int QK_STEPS = D / 16;  // k-steps of Sᵀ = K·Qᵀ
  constexpr int DB = D / 32;        // 32-channel blocks of Oᵀ
  // two separate arrays, so the compiler can tell loads into one stage from reads of the other
  __shared__ __attribute__((aligned(1024))) char smem0[ExtSmem<D>::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[ExtSmem<D>::STAGE];

  const int32_t* __restrict__ ws = a.ws;
  if ((int)blockIdx.x >= ws[WS_NUM_ITEMS]) return;
  const int4 it = reinterpret_cast<const int4*>(ws + a.items_off)[blockIdx.x];
  const int b = it.x, qt = it.y, kv_end = it.z;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, jh = lane >> 5;

  // request geometry, clamped exactly as the plan clamps it
  int64_t q0 = a.cu_seqlens_q[b], q1 = a.cu_seqlens_q[b + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.total_q ? a.total_q : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.total_q ? a.total_q : q1);
  const int n = (int)(q1 - q0);
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_kv_len ? a.max_kv_len : L);
  const int p = L - n;
  const int bt = a.block_tokens;

  // this lane's row (head-major within the work item)
  const int row = wave * 32 + l32;
  const int hl = row / bt;
  const int ti = qt * bt + (row - hl * bt);  // token index within the request's new tokens
  const bool row_ok = hl < a.group && ti < n;
  const int h = g * a.group + (hl < a.group ? hl : 0);
  const int pos = p + (row_ok ? ti : (n > 0 ? n - 1 : 0));  // absolute position of the row
  int wave_max_pos = pos, wave_min_pos = pos;
#pragma unroll
  for (int sh = 1; sh < 32; sh <<= 1) {
    wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, sh));
    wave_min_pos = min(wave_min_pos, __shfl_xor(wave_min_pos, sh));
  }

  // Q rows as the B operand of Sᵀ = K·Qᵀ: lane holds Q[row][16 ks + 8 jh .. +8]
  u32x4 qop[QK_STEPS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((q0 + (row_ok ? ti : 0)) * a.hq + h) * (int64_t)D;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) qop[ks] = row_ok ? ldg16(qrow + 16 * ks + 8 * jh) : z;
  }

  const int row_idx = a.rpi ? a.rpi[b] : b;
  const int32_t* __restrict__ rtt_row = a.rtt + (int64_t)row_idx * a.rtt_stride;
  const int64_t row_elems = (int64_t)a.hkv * D;
  const uint16_t* __restrict__ kbase = static_cast<const uint16_t*>(a.k_pool) + (int64_t)g * D;
  const uint16_t* __restrict__ vbase = static_cast<const uint16_t*>(a.v_pool) + (int64_t)g * D;
  const float c = a.scale_log2;  // > 0 (checked by the host API)

  RowState<D> rs;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) rs.acc[db][r] = 0.f;
  rs.m = kNegInf;
  rs.lpart = 0.f;

  const int ntiles = (kv_end + kBN - 1) / kBN;
  char* const stage0 = smem0;
  char* const stage1 = smem1;
  // two alternating slot sets: one feeds this step's loads, the other is refilled
  TileSlots<D> sl_a, sl_b;
  // tile 0 into stage 0, slots of tile 1 ahead
  if (ntiles > 0) {
    load_tile_slots<D>(sl_b, rtt_row, 0, kv_end, wave, lane);
    load_tile_slots<D>(sl_a, rtt_row, kBN, kv_end, wave, lane);
    dma_tile<D>(sl_b, stage0, kbase, vbase, row_elems, a.pool_slots, wave, lane);
    const int bad = invalid_mask<D>(sl_b);
    wait_vmem_all();
    if (bad) zero_invalid_rows<D>(bad, stage0, wave, lane);
  }
  __syncthreads();

  // One step: prefetch tile t+1 into `nxt` (global -> LDS), compute tile t
  // from `cur`, then publish tile t+1 to the workgroup.
  auto step = [&](int tile, const char* cur, char* nxt, TileSlots<D>& use, TileSlots<D>& fill) {
    const int t0 = tile * kBN;
    const bool has_next = tile + 1 < ntiles;
    int bad = 0;
    if (has_next) {
      // index lookups for tile t+2 go out before the tile t+1 loads, so waiting
      // for them (a step later) never waits for the bulk loads
      load_tile_slots<D>(fill, rtt_row, t0 + 2 * kBN, kv_end, wave, lane);
      dma_tile<D>(use, nxt, kbase, vbase, row_elems, a.pool_slots, wave, lane);
      bad = invalid_mask<D>(use);
    }
    if (t0 <= wave_max_pos) compute_tile<D>(rs, cur, qop, t0, pos, wave_min_pos, c, lane);
    wait_vmem_all();
    if (bad) zero_invalid_rows<D>(bad, nxt, wave, lane);
    __syncthreads();
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    step(tile, stage0, stage1, sl_a, sl_b);
    if (tile + 1 < ntiles) step(tile + 1, stage1, stage0, sl_b, sl_a);
  }

  // ---- epilogue: Oᵀ[d][row] -> out[token][h][d]
  float l = rs.lpart + __shfl_xor(rs.lpart, 32);
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((q0 + ti) * a.hq + h) * (int64_t)D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * db + 8 * rq + 4 * jh;
      u32x2 w;
      w[0] = pack_bf16x2(rs.acc[db][4 * rq + 0] * inv, rs.acc[db][4 * rq + 1] * inv);
      w[1] = pack_bf16x2(rs.acc[db][4 * rq + 2] * inv, rs.acc[db][4 * rq + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d0) = w;
    }
  if (jh == 0 && a.lse) a.lse[(q0 + ti) * a.hq + h] = l > 0.f ? (rs.m + __log2f(l)) * kLn2 : kNegInf;
}

hipError_t launch_extend_bf16(const ExtendArgs& a, int head_dim, int64_t capacity, hipStream_t s) {
  if (capacity <= 0) return hipSuccess;
  dim3 grid((unsigned)capacity, (unsigned)a.hkv);
  if (head_dim == 128) hipLaunchKernelGGL(extend_bf16_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(extend_bf16_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
