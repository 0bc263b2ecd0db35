// Measured peaks of this device, for the roofline fractions the benchmark reports next to the
// nominal figures: a plain streaming read of device memory (HBM bandwidth as a kernel sees it) and a
// loop of independent bf16 MFMAs (the matrix-core rate at the clock the chip holds under load).
// Measurement utilities, not steps of the method.
#include "common.h"
#include "dcu_measure.h"

namespace dcu {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each thread reads kUnroll 16-byte chunks per round, one wave-wide 1 KB contiguous run per load;
// the chunks are folded into a word that is stored only if it hits a value no input produces in
// practice, so no load can be dropped.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_nt(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = load_nt(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// kChains independent accumulators per wave, so the matrix pipe never waits on a result. The
// 32 x 32 x 16 form (32768 flops per instruction) is used: with 8 chains of it the loop reaches the
// nominal rate at 8 waves per CU, where 8 chains of the 16 x 16 x 32 form stay latency-bound
// (measured on this device: 2.45 against 1.39 PFLOP/s at 2048 workgroups).
constexpr int kChains = 8;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink) {
  const uint32_t t = threadIdx.x;
  // small distinct bf16 operands (about 2^-8): the sums stay finite for any iteration count
  const uint32_t w = 0x3b803b80u ^ ((t & 7u) << 16);
  const u32x4 a = u32x4{w, w ^ 1u, w ^ 2u, w ^ 3u};
  const u32x4 b = u32x4{w ^ 4u, w ^ 5u, w ^ 6u, w ^ 7u};
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc[j], 0,
                                                       0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (s == -1.0f) sink[t] = s;
}

}  // namespace
}  // namespace dcu

extern "C" int dcu_measure_stream_read(const void* buf, int64_t bytes, int32_t grid,
                                       uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || grid <= 0) return DCU_EINVAL;
  if (bytes % 16 != 0 || !dcu_aligned16(buf)) return DCU_EUNSUPPORTED;
  hipLaunchKernelGGL(dcu::k_stream_read, dim3(unsigned(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}

extern "C" int dcu_measure_mfma_loop(int32_t grid, int32_t iters, float* sink, void* stream) {
  if (!sink || grid <= 0 || iters <= 0) return DCU_EINVAL;
  hipLaunchKernelGGL(dcu::k_mfma_loop, dim3(unsigned(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), int(iters), sink);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
