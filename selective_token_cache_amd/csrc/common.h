// Shared device helpers for the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcu.h"

namespace dcu {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t b = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}
// fp32 -> bf16 bit pattern, round to nearest even
__device__ __forceinline__ uint32_t f_to_bf_bits(float f) { return pack_bf2(f, 0.0f) & 0xffffu; }

// ---------------------------------------------------------------------------- streaming loads
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load marked non-temporal (data read once; keep it from displacing reused lines)
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------- wave reductions
// The value of lane l ^ OFF (OFF = 16 or 32) through the gfx950 permlane swaps (VALU, no LDS round
// trip). Given the same operand twice, a swap returns in every lane l the values of lanes l & ~OFF
// and l | OFF; the partner is the one that is not lane l.
template <int OFF>
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t x) {
  static_assert(OFF == 16 || OFF == 32, "permlane swap distance");
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const bool upper = (lane & OFF) != 0;
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return upper ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return upper ? r[0] : r[1];
  }
}
template <int OFF, typename T>
__device__ __forceinline__ T xor_lane(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, xor_lane_u32<OFF>(__builtin_bit_cast(uint32_t, v)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = xor_lane_u32<OFF>(uint32_t(u));
    const uint64_t hi = xor_lane_u32<OFF>(uint32_t(u >> 32));
    return __builtin_bit_cast(T, lo | (hi << 32));
  }
}

// Butterfly over the wave in the fixed order 32, 16, 8, 4, 2, 1 (every lane ends with the same
// value); the first two exchanges use the permlane swaps, the rest LDS-free shuffles of the
// compiler's choice. Each step adds the partner's value: the result does not depend on how the
// partner value travels.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v += xor_lane<32>(v);
  v += xor_lane<16>(v);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  T o = xor_lane<32>(v);
  v = o > v ? o : v;
  o = xor_lane<16>(v);
  v = o > v ? o : v;
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) {
    o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off, kWave);
  return v;
}

// inclusive prefix sum across the wave (lane order)
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// exclusive prefix sum over a whole workgroup (blockDim.x a multiple of 64, <= 1024).
// `lds` must hold 17 ints. Returns the exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int inc = wave_incl_scan(v);
  if (lane == kWave - 1) lds[wid] = inc;
  __syncthreads();
  if (threadIdx.x < kWave) {  // wave 0 scans the (at most 16) wave totals
    const int tv = lane < nw ? lds[lane] : 0;
    const int ti = wave_incl_scan(tv);
    if (lane < nw) lds[lane] = ti - tv;
    if (lane == kWave - 1) lds[16] = ti;
  }
  __syncthreads();
  int res = lds[wid] + inc - v;
  *total = lds[16];
  __syncthreads();
  return res;
}

// block-wide sum of ints (order-free, exact)
__device__ __forceinline__ int block_sum_int(int v, int* lds) {
  int total;
  (void)block_excl_scan(v, lds, &total);
  return total;
}

}  // namespace dcu

// ------------------------------------------------------------------------------ host helpers
#define DCU_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return DCU_EHIP;    \
  } while (0)

static inline bool dcu_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
