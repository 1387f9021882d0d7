// Device helpers for gfx950 (CDNA4, wave64): vector types, bf16 packing,
// MFMA wrappers and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;  // MFMA bf16 operand
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Returns x unchanged but opaque to the optimiser, so the addresses derived
// from it in rarely run code (a segment's epilogue inside the tile loop) are
// computed there, not hoisted out of the loop into registers it needs.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ldg8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Loads of data read once (the decode's K/V rows), with the non-temporal
// hint (global_load ... nt) when STREAM is set: such lines are not kept in
// the caches.  Whether that pays depends on the layout read (the decode
// launchers choose per launch).
template <bool STREAM>
__device__ __forceinline__ u32x4 ldg16_once(const void* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return ldg16(p);
}
template <bool STREAM>
__device__ __forceinline__ u32x2 ldg8_once(const void* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  else return ldg8(p);
}

__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round two floats to bf16 (nearest-even) and pack them (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  float2_t f = {a, b};
  bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

// Low / high 16-bit halves of two dwords combined: {lo16(x), lo16(y)} and {hi16(x), hi16(y)}.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max of v over lanes l and l ^ 32: v_permlane32_swap trades the upper half
// of one copy for the lower half of the other, so no LDS round trip is taken
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max of v over lanes l and l ^ 16 (v_permlane16_swap: odd and even 16-lane rows)
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int W>
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, W);
}

__device__ __forceinline__ int clamp_slot(int s, int64_t pool_slots) {
  // negative or too large slots are clamped so a read never leaves the pool
  return (uint32_t)s < (uint64_t)pool_slots ? s : (s < 0 ? 0 : (int)(pool_slots - 1));
}

// Cheaper clamp for hot loops: `last` = pool_slots - 1 (< 2^31); a negative
// slot becomes a huge unsigned value and is clamped to the last row.
__device__ __forceinline__ uint32_t clamp_slot_u32(int s, uint32_t last) { return min((uint32_t)s, last); }

// Byte/element offset of a pool row: 32 x 32 -> 64-bit multiply.
__device__ __forceinline__ int64_t row_offset(uint32_t slot, uint32_t row_elems) {
  return (int64_t)((uint64_t)slot * (uint64_t)row_elems);
}

}  // namespace pkv
