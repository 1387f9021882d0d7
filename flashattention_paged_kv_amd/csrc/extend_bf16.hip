// EXTEND: causal varlen attention of new tokens over their request's cached
// prefix and themselves, bf16 inputs, fp32 accumulation, bf16 MFMA on gfx950.
//
// The score matrix never leaves the chip (FlashAttention page, §2): a
// workgroup walks the key range in 64-key tiles, gathers each K and V tile
// through req_to_token into LDS and keeps a running max / sum per row
// (online softmax).
//
// Work item = (request b, query tile t, kv head g).  Its 256 rows are the
// (query head, token) pairs of the G query heads that share kv head g, for
// block = 256 / G consecutive new tokens (head-major rows), so every K/V byte
// brought into LDS serves 256 rows.  Eight waves own 32 rows each; one
// workgroup fills a CU (two waves per SIMD).
//
// Data movement is asynchronous and register-free: global -> LDS loads
// (gfx950 global_load_lds_*) fill a ring of two 128-key K/V stages and a
// ring of three req_to_token stages.  While tile t is computed (as two
// 64-key halves), the K/V rows of tile t+1 and the req_to_token entries of
// tile t+2 are in flight; the loads are issued between the first MFMAs of the
// tile so their address work hides under the matrix cores.  The tile loop is
// unrolled by the K/V ring period (2), so every LDS address is a per-lane
// offset computed once plus an immediate.
//
// Per wave and 64-key half tile, with 32x32x16 bf16 MFMAs:
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
#include <type_traits>

#include "device_common.h"
#include "lds_dma.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int kBN = 2 * kExtendTileN;     // keys per tile (128), computed in halves of 64
constexpr int kHalf = kExtendTileN;
constexpr int kWaves = kExtendRows / 32;  // 8 waves x 32 rows
constexpr int kThreads = 64 * kWaves;
constexpr int kKVStages = 2;
constexpr int kSlotStages = 3;  // req_to_token entries are requested 2 tiles ahead (indexed at run time)

// LDS holds the K tiles of all stages, then the V tiles of all stages, then
// the slot stages, so a tile's K (or V) rows sit at a per-lane offset plus an
// immediate below 64 KiB for every stage (DS instructions take a 16-bit
// offset).  Rows are D*2 bytes, unpadded, with the 16-byte chunks of each row
// XOR-swizzled against bank conflicts:
//  * K: chunk c of key r at position c ^ (r % CH) -- the 16-byte row reads of
//    the Sᵀ product touch one chunk of many consecutive keys;
//  * V: chunk c of key r at position c ^ swz_v(r).  A transposing read of a
//    16-lane group touches the 32-byte chunk pair (c, c + 1) of 4
//    consecutive keys, and the two groups of 32 lanes read the pairs c and
//    c + 2 of the same keys, i.e. the aligned quad of chunks 4 (c / 4) ..
//    +3.  For head_dim 128 (256-byte rows, one row per line of the 64 banks)
//    swz_v(r) = 4 (r % 4) + 2 ((r / 4) % 2) sends the 4 keys' quads to 4
//    different quads, so 32 lanes read 16 distinct 16-byte bank groups; an
//    even mask keeps the pairs aligned.  For head_dim 64 the mask is
//    2 (r % 8) % 8.
template <int D>
struct ExtSmem {
  static constexpr int RB = D * 2;                        // bytes per key row
  static constexpr int CH = D / 8;                        // 16-byte chunks per row
  static constexpr int MAT = kBN * RB;                    // one matrix tile
  static constexpr int STAGE = MAT;                       // stride between stages' K (or V) tiles
  static constexpr int VOFF = kKVStages * MAT;            // a stage's V tile, from its K tile
  static constexpr int ROWS_PER_KB = 1024 / RB;           // rows written by one 64-lane 16-byte load
  static constexpr int NQ = kBN / ROWS_PER_KB / kWaves;   // such loads per wave and matrix
  static constexpr int SLOT_BYTES = kBN * 4;              // req_to_token entries of one tile
  static constexpr int TOTAL = 2 * kKVStages * MAT + kSlotStages * SLOT_BYTES;
};

template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (ExtSmem<D>::CH - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) + 2 * ((row >> 2) & 1) : (2 * (row & 7)) & (ExtSmem<D>::CH - 1);
}
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * ExtSmem<D>::RB + ((chunk ^ swz_k<D>(row)) << 4);
}
template <int D>
__device__ __forceinline__ int v_off(int row, int chunk) {
  return row * ExtSmem<D>::RB + ((chunk ^ swz_v<D>(row)) << 4);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x2 lds_read_tr16(const char* base, uint32_t off) {
  // transposing 8-byte LDS read (gfx950): see the kernel header
  lds_char* p = (lds_char*)(const_cast<char*>(base)) + off;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the tile handled by (wave, load q, lane); the lane writes LDS chunk
// position lane % CH of that row and so fetches the global chunk the swizzle
// puts there.
template <int D>
__device__ __forceinline__ int tile_row(int wave, int q, int lane) {
  return (wave * ExtSmem<D>::NQ + q) * ExtSmem<D>::ROWS_PER_KB + lane / ExtSmem<D>::CH;
}

// K and V rows of one tile into a stage, from the slots in a slot stage, in
// two halves: read_kv_slots fetches this lane's slots from LDS, issue_kv_rows
// starts the global -> LDS row loads (so the LDS latency of the first can be
// hidden behind other work).
template <int D>
__device__ __forceinline__ void read_kv_slots(const char* slots, int wave, int lane, int (&sv)[ExtSmem<D>::NQ]) {
#pragma unroll
  for (int q = 0; q < ExtSmem<D>::NQ; ++q) sv[q] = *reinterpret_cast<const int*>(slots + 4 * tile_row<D>(wave, q, lane));
}

template <int D>
__device__ __forceinline__ void issue_kv_rows(const int (&sv)[ExtSmem<D>::NQ], char* stage,
                                              const uint16_t* __restrict__ kbase, const uint16_t* __restrict__ vbase,
                                              uint32_t row_elems, uint32_t last_slot, int wave, int lane) {
  const int p = lane % ExtSmem<D>::CH;
#pragma unroll
  for (int q = 0; q < ExtSmem<D>::NQ; ++q) {
    const int r = tile_row<D>(wave, q, lane);
    const int64_t row_off = row_offset(clamp_slot_u32(sv[q], last_slot), row_elems);
    const uint32_t dst = lds_addr(stage) + (wave * ExtSmem<D>::NQ + q) * 1024;
    dma16(kbase + row_off + 8 * (p ^ swz_k<D>(r)), dst);
    dma16(vbase + row_off + 8 * (p ^ swz_v<D>(r)), dst + ExtSmem<D>::VOFF);
  }
}

template <int D>
__device__ __forceinline__ void issue_kv(const char* slots, char* stage, const uint16_t* __restrict__ kbase,
                                         const uint16_t* __restrict__ vbase, uint32_t row_elems,
                                         uint32_t last_slot, int wave, int lane) {
  int sv[ExtSmem<D>::NQ];
  read_kv_slots<D>(slots, wave, lane, sv);
  issue_kv_rows<D>(sv, stage, kbase, vbase, row_elems, last_slot, wave, lane);
}

// req_to_token entries of the 64 keys of a tile (one wave; keys past kv_end
// read the last valid entry, their rows are zeroed later).
__device__ __forceinline__ void issue_slots(const int32_t* __restrict__ rtt_row, int t0, int kv_end,
                                            char* slot_stage, int lane) {
  dma4(rtt_row + min(t0 + lane, kv_end - 1), lds_addr(slot_stage));
  dma4(rtt_row + min(t0 + 64 + lane, kv_end - 1), lds_addr(slot_stage) + 256);
}

// Rows past kv_end that this lane fetched are overwritten with zeros once its
// own loads have landed: a poisoned V row times a zero probability would
// still be NaN.
template <int D>
__device__ __forceinline__ void zero_rows_past_end(char* stage, int t0, int kv_end, int wave, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < ExtSmem<D>::NQ; ++q) {
    if (t0 + tile_row<D>(wave, q, lane) >= kv_end) {
      char* dst = stage + (wave * ExtSmem<D>::NQ + q) * 1024 + 16 * lane;
      *reinterpret_cast<u32x4*>(dst) = z;
      *reinterpret_cast<u32x4*>(dst + ExtSmem<D>::VOFF) = z;
    }
  }
}

// Per-lane LDS byte offsets of the Vᵀ transpose reads for each 32-channel block,
// measured from a stage's K tile: key 4 jj + i16/4 (its swizzle is the same for
// every 16-key step and +8), the chunk pair of channel 32 db + dsub + 4 (i16 % 4).
// The V tiles' distance from the K tiles is folded in here and hidden from the
// optimiser, so the stage and key-step parts of every read stay below 64 KiB
// and are encoded as the instruction's immediate offset.
template <int D>
__device__ __forceinline__ void v_read_bases(int (&vb)[D / 32], int lane) {
  const int g16 = lane >> 4, i16 = lane & 15;
  const int key = 4 * (g16 >> 1) + (i16 >> 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int col = 32 * db + 16 * (g16 & 1) + 4 * (i16 & 3);
    vb[db] = opaque(ExtSmem<D>::VOFF + v_off<D>(key, col >> 3) + ((col & 7) << 1));
  }
}

// Per-lane LDS byte offsets of the K row reads of the Sᵀ product, one per
// 16-channel k-step: key lane % 32 (key + 32 has the same swizzle), chunk 2 ks + jh.
template <int D>
__device__ __forceinline__ void k_read_offsets(int (&ko)[D / 16], int lane) {
  const int key = lane & 31, jh = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) ko[ks] = k_off<D>(key, 2 * ks + jh);
}

template <int D>
struct RowState {
  floatx16 acc[D / 32];
  float m, lpart;
};

// One key tile in two parts.  qk_tile: Sᵀ of both 32-key blocks (each
// block's MFMA chain in turn, K operands read from LDS four MFMAs ahead), the
// causal mask on diagonal tiles (MASKED), the tile's row max, the lazy
// rescale and the exponentials, leaving the tile's probabilities as the bf16
// Pᵀ operands `pop` (k-step ks2 = 2 kb + half); `mid` runs between the first
// MFMAs (the step's global -> LDS loads are issued there).  pv_tile: Oᵀ += Vᵀ·Pᵀ.
template <int D, bool MASKED, typename Mid>
__device__ __forceinline__ void qk_tile(RowState<D>& rs, u32x4 (&pop)[4], const char* cur,
                                        const u32x4 (&qop)[D / 16], const int (&koff)[D / 16], int t0, int pos,
                                        float c, int lane, Mid&& mid) {
  constexpr int QK_STEPS = D / 16;
  constexpr int DB = D / 32;
  const int jh = lane >> 5;
  floatx16 s[2];
  {
    // K operand n = QK_STEPS kb + ks is read four MFMAs before its use; the
    // sched_barriers keep exactly that order (and the register window small)
    constexpr int NK = 2 * QK_STEPS, AHEAD = 4;
    auto kread = [&](int n) {
      return *reinterpret_cast<const u32x4*>(cur + 32 * (n / QK_STEPS) * ExtSmem<D>::RB + koff[n % QK_STEPS]);
    };
    u32x4 kop[NK];
#pragma unroll
    for (int n = 0; n < AHEAD; ++n) kop[n] = kread(n);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      __builtin_amdgcn_sched_barrier(0);
      s[n / QK_STEPS] = mfma32x32x16(as_bf16x8(kop[n]), as_bf16x8(qop[n % QK_STEPS]), s[n / QK_STEPS]);
      if (n + AHEAD < NK) kop[n + AHEAD] = kread(n + AHEAD);
      if (n == AHEAD) mid();  // the caller's loads start under the MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (MASKED) {
    // key t0 + 32 kb + 8 (r/4) + 4 jh + r%4 is visible iff its offset from
    // t0 + 4 jh is <= lim: one subtraction, then compares with constants
    const int lim = pos - t0 - 4 * jh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) <= lim ? s[kb][r] : kNegInf;
  }
  // row max: two chains of three-input maxima
  float mx0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]), mx1 = fmaxf(fmaxf(s[1][0], s[1][1]), s[1][2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) {
    mx0 = fmaxf(fmaxf(mx0, s[0][r]), s[0][r + 1]);
    mx1 = fmaxf(fmaxf(mx1, s[1][r]), s[1][r + 1]);
  }
  float mx = fmaxf(fmaxf(mx0, s[0][15]), fmaxf(mx1, s[1][15]));
  mx = max_xor32(mx) * c;
  // lazy rescale: the reference max moves only when a row's max exceeds it by
  // more than 8 (log2 units), so exp2(s - m) <= 256 while acc and l keep
  // referring to the same m
  if (__any(mx > rs.m + 8.f)) {
    const float m_new = fmaxf(rs.m, mx);
    const float alpha = m_new == kNegInf ? 1.f : exp2_fast(rs.m - m_new);
    rs.lpart *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) rs.acc[db] *= alpha;
    rs.m = m_new;
  }
  const float m_use = rs.m == kNegInf ? 0.f : rs.m;
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = exp2_fast(__builtin_fmaf(s[ks2 >> 1][8 * (ks2 & 1) + e], c, -m_use));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pop[ks2][w] = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);
      rs.lpart += pv[2 * w] + pv[2 * w + 1];
    }
  }
}

// Oᵀ += Vᵀ·Pᵀ over the tile's 4 key steps.  Step ks2 covers keys 16 ks2 ..
// +16; this lane's 8 keys are {16 ks2 + 8 (e/4) + 4 jh + e%4}: two transposed
// 4-key reads per 32-channel block, read one step ahead.
template <int D>
__device__ __forceinline__ void pv_tile(RowState<D>& rs, const u32x4 (&pop)[4], const char* cur,
                                        const int (&vbase_off)[D / 32]) {
  constexpr int DB = D / 32;
  const char* vt = cur;  // the V tile's offset is part of vbase_off
  // operands of MFMA n = DB ks2 + db are read one key step (DB MFMAs) ahead;
  // the sched_barriers keep that order
  constexpr int NM = 4 * DB;
  auto vread = [&](int n) {
    const int ks2 = n / DB, db = n % DB;
    const u32x2 va = lds_read_tr16(vt + 16 * ks2 * ExtSmem<D>::RB, vbase_off[db]);
    const u32x2 vb = lds_read_tr16(vt + (16 * ks2 + 8) * ExtSmem<D>::RB, vbase_off[db]);
    return u32x4{va[0], va[1], vb[0], vb[1]};
  };
  u32x4 vop[NM];
#pragma unroll
  for (int n = 0; n < DB; ++n) vop[n] = vread(n);
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    __builtin_amdgcn_sched_barrier(0);
    rs.acc[n % DB] = mfma32x32x16(as_bf16x8(vop[n]), as_bf16x8(pop[n / DB]), rs.acc[n % DB]);
    if (n + DB < NM) vop[n + DB] = vread(n + DB);
  }
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void extend_bf16_kernel(ExtendArgs a) {
  using S = ExtSmem<D>;
  constexpr int QK_STEPS = D / 16;  // k-steps of Sᵀ = K·Qᵀ
  constexpr int DB = D / 32;        // 32-channel blocks of Oᵀ
  __shared__ __attribute__((aligned(1024))) char smem[S::TOTAL];

  const int32_t* __restrict__ ws = a.ws;
  // 1-D grid, workgroup = item * Hkv + kv head: workgroups go to the 8 XCDs
  // round-robin, so with Hkv a multiple of 8 each XCD serves one kv head for
  // all items and the query tiles that re-read a head's K/V rows share its L2
  const int xi = (int)blockIdx.x / a.hkv;
  if (xi >= ws[WS_NUM_ITEMS]) return;
  const int4 it = reinterpret_cast<const int4*>(ws + a.items_off)[xi];
  const int b = it.x, qt = it.y, kv_end = it.z;
  const int g = (int)blockIdx.x - xi * a.hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS targets on the scalar unit
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
    // let the compiler see Q land here (vmcnt(0), other counters untouched), so
    // it does not wait for "outstanding" loads inside the tile loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  const int row_idx = a.rpi ? a.rpi[b] : b;
  const int32_t* __restrict__ rtt_row = a.rtt + (int64_t)row_idx * a.rtt_stride;
  const uint32_t row_elems = (uint32_t)(a.hkv * D);
  const uint32_t last_slot = (uint32_t)(a.pool_slots - 1);
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
  int vbo[DB];
  v_read_bases<D>(vbo, lane);

  int ko[QK_STEPS];
  k_read_offsets<D>(ko, lane);
  char* const kv0 = smem;  // K tile of stage J at kv0 + J * STAGE, its V tile VOFF further
  char* const slot0 = smem + 2 * kKVStages * S::MAT;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // Tile u's req_to_token entries go to slot stage u % 3 (requested by wave 0
  // at step u-2), its K/V rows to stage u % 2 (requested at step u-1).  Each
  // step ends with all of its own loads landed (tile t+1 and the entries of
  // tile t+2) before the barrier publishes them.
  auto slot_stage = [&](int u) { return slot0 + (u % kSlotStages) * S::SLOT_BYTES; };
  // prologue: entries of tiles 0 and 1, then the K/V rows of tile 0
  if (ntiles > 0) {
    if (wave == 0) {
      for (int t = 0; t < 2 && t < ntiles; ++t) issue_slots(rtt_row, t * kBN, kv_end, slot_stage(t), lane);
      wait_vmem<0>();
    }
    __syncthreads();
    issue_kv<D>(slot_stage(0), kv0, kbase, vbase, row_elems, last_slot, wave, lane);
    wait_vmem<0>();
    zero_rows_past_end<D>(kv0, 0, kv_end, wave, lane);
  }
  __syncthreads();
  auto qk = [&](int t0, const char* stage, u32x4 (&pop)[4], auto&& mid) __attribute__((always_inline)) {
    if (t0 + kHalf - 1 > wave_min_pos)
      qk_tile<D, true>(rs, pop, stage, qop, ko, t0, pos, c, lane, mid);
    else
      qk_tile<D, false>(rs, pop, stage, qop, ko, t0, pos, c, lane, mid);
  };
  auto nothing = [&]() __attribute__((always_inline)) {};
  // One step over 128-key tile `tile` (K/V stage J = tile % 2, compile time):
  // read the slots of tile+1 from LDS, compute the first 64-key half with the
  // loads of the entries of tile+2 and the rows of tile+1 issued between its
  // first MFMAs, then the second half (skipped when causally invisible).
  auto step = [&](int tile, auto J_) __attribute__((always_inline)) {
    constexpr int J = decltype(J_)::value;
    constexpr int J1 = (J + 1) % 2;
    const int t0 = tile * kBN;
    const bool sl2 = wave == 0 && tile + 2 < ntiles;
    const bool kv1 = tile + 1 < ntiles;
    int sv[S::NQ];
    if (kv1) read_kv_slots<D>(slot_stage(tile + 1), wave, lane, sv);
    auto loads = [&]() __attribute__((always_inline)) {
      if (sl2) issue_slots(rtt_row, t0 + 2 * kBN, kv_end, slot_stage(tile + 2), lane);
      if (kv1) issue_kv_rows<D>(sv, kv0 + J1 * S::STAGE, kbase, vbase, row_elems, last_slot, wave, lane);
    };
    if (t0 <= wave_max_pos) {
      u32x4 pop[4];
      qk(t0, kv0 + J * S::STAGE, pop, loads);
      pv_tile<D>(rs, pop, kv0 + J * S::STAGE, vbo);
      if (t0 + kHalf <= wave_max_pos) {
        u32x4 pop2[4];
        qk(t0 + kHalf, kv0 + J * S::STAGE + kHalf * S::RB, pop2, nothing);
        pv_tile<D>(rs, pop2, kv0 + J * S::STAGE + kHalf * S::RB, vbo);
      }
    } else {
      loads();
    }
    wait_vmem<0>();
    if (kv1) zero_rows_past_end<D>(kv0 + J1 * S::STAGE, t0 + kBN, kv_end, wave, lane);
    __syncthreads();
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    step(tile, std::integral_constant<int, 0>());
    if (tile + 1 < ntiles) step(tile + 1, std::integral_constant<int, 1>());
  }
  wait_vmem<0>();

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
  dim3 grid((unsigned)(capacity * a.hkv));
  if (head_dim == 128) hipLaunchKernelGGL(extend_bf16_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(extend_bf16_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
