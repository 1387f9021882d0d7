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

template <int D>
struct ExtSmem {
  // K rows padded to D*2+16 bytes, V rows to D*2+32 bytes: conflict-free 16-byte
  // row reads for K and transpose reads for V.
  static constexpr int KS = D * 2 + 16;
  static constexpr int VS = D * 2 + 32;
  static constexpr int KBYTES = kBN * KS;
  static constexpr int VBYTES = kBN * VS;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int TOTAL = 2 * STAGE;
};

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

// Register staging of one K/V tile: thread t loads 16 bytes of rows t/16 + 16k.
template <int D>
struct Stage {
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = kThreads / CH;        // rows per load instruction
  static constexpr int NL = kBN / RPI;             // loads per thread per matrix
  u32x4 k[NL];
  u32x4 v[NL];
};

template <int D>
__device__ __forceinline__ void gather_tile(Stage<D>& st, const int32_t* __restrict__ rtt_row, int t0, int kv_end,
                                            int64_t pool_slots, const uint16_t* __restrict__ kbase,
                                            const uint16_t* __restrict__ vbase, int64_t row_elems) {
  const int tid = threadIdx.x;
  const int c = tid % Stage<D>::CH;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < Stage<D>::NL; ++k) {
    const int key = t0 + tid / Stage<D>::CH + k * Stage<D>::RPI;
    if (key < kv_end) {
      const int64_t slot = clamp_slot(rtt_row[key], pool_slots);
      st.k[k] = ldg16(kbase + slot * row_elems + 8 * c);
      st.v[k] = ldg16(vbase + slot * row_elems + 8 * c);
    } else {
      st.k[k] = z;
      st.v[k] = z;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& st, char* smem) {
  const int tid = threadIdx.x;
  const int c = tid % Stage<D>::CH;
#pragma unroll
  for (int k = 0; k < Stage<D>::NL; ++k) {
    const int r = tid / Stage<D>::CH + k * Stage<D>::RPI;
    *reinterpret_cast<u32x4*>(smem + r * ExtSmem<D>::KS + 16 * c) = st.k[k];
    *reinterpret_cast<u32x4*>(smem + ExtSmem<D>::KBYTES + r * ExtSmem<D>::VS + 16 * c) = st.v[k];
  }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void extend_bf16_kernel(ExtendArgs a) {
  constexpr int KS = ExtSmem<D>::KS, VS = ExtSmem<D>::VS;
  constexpr int QK_STEPS = D / 16;  // k-steps of Sᵀ = K·Qᵀ
  constexpr int DB = D / 32;        // 32-channel blocks of Oᵀ
  __shared__ __attribute__((aligned(16))) char smem[ExtSmem<D>::TOTAL];

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
  const bool row_ok = hl < a.group && ti < n && ti < (qt + 1) * bt;
  const int h = g * a.group + (hl < a.group ? hl : 0);
  const int pos = p + (row_ok ? ti : (n > 0 ? n - 1 : 0));  // absolute position of the row
  // the wave's highest position decides which key tiles it must compute
  int wave_max_pos = pos;
  wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, 1));
  wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, 2));
  wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, 4));
  wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, 8));
  wave_max_pos = max(wave_max_pos, __shfl_xor(wave_max_pos, 16));

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

  floatx16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kNegInf, lpart = 0.f;

  const int ntiles = (kv_end + kBN - 1) / kBN;
  Stage<D> st;
  if (ntiles > 0) {
    gather_tile<D>(st, rtt_row, 0, kv_end, a.pool_slots, kbase, vbase, row_elems);
    store_tile<D>(st, smem);
  }
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int t0 = tile * kBN;
    char* cur = smem + (tile & 1) * ExtSmem<D>::STAGE;
    if (tile + 1 < ntiles) gather_tile<D>(st, rtt_row, t0 + kBN, kv_end, a.pool_slots, kbase, vbase, row_elems);

    if (t0 <= wave_max_pos) {
      // ---- Sᵀ for two 32-key blocks
      floatx16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const char* krow = cur + (32 * kb + l32) * KS + 16 * jh;
#pragma unroll
        for (int ks = 0; ks < QK_STEPS; ++ks) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + 32 * ks);
          s[kb] = mfma32x32x16(as_bf16x8(kv), as_bf16x8(qop[ks]), s[kb]);
        }
      }
      // ---- mask, online softmax (log2 domain)
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + 32 * kb + 8 * (r >> 2) + 4 * jh + (r & 3);
          const float v = key <= pos ? s[kb][r] * a.scale_log2 : kNegInf;
          s[kb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;  // a row with no visible key yet
      const float alpha = exp2_fast(m - m_use);
      m = m_new;
      float ps = 0.f;
      u32x4 pop[4];  // Pᵀ B operands, one per 16-key k-step
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = exp2_fast(s[kb][8 * half + e] - m_use);
            ps += pv[e];
          }
          u32x4 w;
          w[0] = pack_bf16x2(pv[0], pv[1]);
          w[1] = pack_bf16x2(pv[2], pv[3]);
          w[2] = pack_bf16x2(pv[4], pv[5]);
          w[3] = pack_bf16x2(pv[6], pv[7]);
          pop[2 * kb + half] = w;
        }
      lpart = lpart * alpha + ps;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      // ---- Oᵀ += Vᵀ·Pᵀ.  k-step ks2 covers keys 16 ks2 .. +16; this lane's 8 keys are
      //      {16 ks2 + 8 (e/4) + 4 jh + e%4}: two transposed 4-key reads.
      const int g16 = lane >> 4, i16 = lane & 15;
      const int dsub = 16 * (g16 & 1);
      const int jj = g16 >> 1;
      const char* vt = cur + ExtSmem<D>::KBYTES;
#pragma unroll
      for (int ks2 = 0; ks2 < 4; ++ks2) {
        const int key_a = 16 * ks2 + 4 * jj + (i16 >> 2);
        const int key_b = key_a + 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = 32 * db + dsub + 4 * (i16 & 3);
          const u32x2 va = lds_read_tr16(vt, key_a * VS + 2 * col);
          const u32x2 vb = lds_read_tr16(vt, key_b * VS + 2 * col);
          u32x4 vop = {va[0], va[1], vb[0], vb[1]};
          acc[db] = mfma32x32x16(as_bf16x8(vop), as_bf16x8(pop[ks2]), acc[db]);
        }
      }
    }
    if (tile + 1 < ntiles) store_tile<D>(st, smem + ((tile + 1) & 1) * ExtSmem<D>::STAGE);
    __syncthreads();
  }

  // ---- epilogue: Oᵀ[d][row] -> out[token][h][d]
  float l = lpart + __shfl_xor(lpart, 32);
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + ((q0 + ti) * a.hq + h) * (int64_t)D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * db + 8 * rq + 4 * jh;
      u32x2 w;
      w[0] = pack_bf16x2(acc[db][4 * rq + 0] * inv, acc[db][4 * rq + 1] * inv);
      w[1] = pack_bf16x2(acc[db][4 * rq + 2] * inv, acc[db][4 * rq + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + d0) = w;
    }
  if (jh == 0 && a.lse) a.lse[(q0 + ti) * a.hq + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

hipError_t launch_extend_bf16(const ExtendArgs& a, int head_dim, int64_t capacity, hipStream_t s) {
  if (capacity <= 0) return hipSuccess;
  dim3 grid((unsigned)capacity, (unsigned)a.hkv);
  if (head_dim == 128) hipLaunchKernelGGL(extend_bf16_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(extend_bf16_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
