// dcu_distance: per-token cosine distance between a layer's input now and its cached input of the
// previous step, and the per-group mean of those distances.
// Dynamic-dLLM reading notes, Key design 1 (DCU): the d_i^{t,l} equation and the layer dynamics
// s^{t,l} = (1/N) sum_i d_i^{t,l}.
//
// Design (HBM-bound: both rows must be read once, 4*d bytes per bf16 row pair):
//  * one wave64 per row pair, 4 rows per 256-thread workgroup; each lane streams 16-byte chunks of
//    both rows with 8 chunks in flight per operand;
//  * the dot product and both squared norms accumulate in fp64 (bf16*bf16 products are exact, so
//    the only rounding is in the fp64 sums); the distance 1 - cos is formed in fp64 and rounded
//    once to fp32. An fp32 one-pass form would lose the ~1e-5 distances to cancellation;
//  * a bitwise OR of (a XOR b) flags identical rows, which give exactly 0;
//  * the group mean is a second, tiny kernel: one workgroup per group sums the fp32 distances in
//    fp64 in a fixed order (deterministic, no atomics, no workspace).
#include "common.h"

namespace dcu {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kUnroll = 8;

struct Acc {
  double dot0 = 0.0, dot1 = 0.0, na0 = 0.0, na1 = 0.0, nb0 = 0.0, nb1 = 0.0;
  uint32_t diff = 0u;
};

__device__ __forceinline__ void acc_bf16_word(Acc& s, uint32_t wa, uint32_t wb) {
  s.diff |= wa ^ wb;
  const double a0 = bf_lo(wa), a1 = bf_hi(wa);
  const double b0 = bf_lo(wb), b1 = bf_hi(wb);
  s.dot0 = fma(a0, b0, s.dot0);
  s.dot1 = fma(a1, b1, s.dot1);
  s.na0 = fma(a0, a0, s.na0);
  s.na1 = fma(a1, a1, s.na1);
  s.nb0 = fma(b0, b0, s.nb0);
  s.nb1 = fma(b1, b1, s.nb1);
}

__device__ __forceinline__ void acc_f32_pair(Acc& s, uint32_t wa0, uint32_t wa1, uint32_t wb0,
                                             uint32_t wb1) {
  s.diff |= (wa0 ^ wb0) | (wa1 ^ wb1);
  const double a0 = __uint_as_float(wa0), a1 = __uint_as_float(wa1);
  const double b0 = __uint_as_float(wb0), b1 = __uint_as_float(wb1);
  s.dot0 = fma(a0, b0, s.dot0);
  s.dot1 = fma(a1, b1, s.dot1);
  s.na0 = fma(a0, a0, s.na0);
  s.na1 = fma(a1, a1, s.na1);
  s.nb0 = fma(b0, b0, s.nb0);
  s.nb1 = fma(b1, b1, s.nb1);
}

// the distance from a wave's per-lane sums (butterfly over the wave, then 1 - cos in fp64);
// every lane returns the same value
__device__ __forceinline__ double finish_distance(const Acc& s) {
  const double dot = wave_sum(s.dot0 + s.dot1);
  const double na = wave_sum(s.na0 + s.na1);
  const double nb = wave_sum(s.nb0 + s.nb1);
  const uint32_t diff = wave_or(s.diff);
  double d;
  if (diff == 0u) {
    d = 0.0;
  } else if (na == 0.0 && nb == 0.0) {
    d = 0.0;
  } else if (na == 0.0 || nb == 0.0) {
    d = 1.0;
  } else {
    d = 1.0 - dot / sqrt(na * nb);
    d = d < 0.0 ? 0.0 : (d > 2.0 ? 2.0 : d);
  }
  return d;
}

// distance of one row pair by one wave: fp64 sums of the products, XOR flag for identical rows;
// every lane returns the same value
template <bool kBf16>
__device__ __forceinline__ double row_distance(const uint4* __restrict__ a,
                                               const uint4* __restrict__ b, int chunks, int lane) {
  Acc s;
  for (int base = 0; base < chunks; base += kWave * kUnroll) {
    uint4 ra[kUnroll], rb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = base + u * kWave + lane;
      if (c < chunks) {
        ra[u] = load_nt(a + c);
        rb[u] = load_nt(b + c);
      } else {
        ra[u] = make_uint4(0, 0, 0, 0);
        rb[u] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if constexpr (kBf16) {
        acc_bf16_word(s, ra[u].x, rb[u].x);
        acc_bf16_word(s, ra[u].y, rb[u].y);
        acc_bf16_word(s, ra[u].z, rb[u].z);
        acc_bf16_word(s, ra[u].w, rb[u].w);
      } else {
        acc_f32_pair(s, ra[u].x, ra[u].y, rb[u].x, rb[u].y);
        acc_f32_pair(s, ra[u].z, ra[u].w, rb[u].z, rb[u].w);
      }
    }
  }
  return finish_distance(s);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void k_distance(const uint4* __restrict__ xc,
                                                  const uint4* __restrict__ xp, int64_t rows,
                                                  int chunks, float* __restrict__ dist) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= rows) return;
  const double d = row_distance<kBf16>(xc + row * chunks, xp + row * chunks, chunks, lane);
  if (lane == 0) dist[row] = float(d);
}

// Listed rows only (closed-loop chaining: the previous layer scattered exactly these rows, every
// other row of x_cur equals x_prev bit for bit and has distance 0). Workgroup (blk, b) first marks
// the listed positions of sequence b in an LDS bitmap (the list is a few hundred words), then wave w
// writes 0 for position 4 blk + w if it is not listed, and computes the distance of list slot
// 4 blk + w if that slot is counted; with roll, that row of x_cur is then copied into x_prev (the
// cache roll of the row). Every position's distance is written by exactly one wave.
// Latency: the count, the wave's own slot and the first kListPre entries of the list are loaded
// together (all in bounds whatever the count), and a row that fits in one round of loads is rolled
// from the registers it was read into.
constexpr int kMaxRowsBitmap = 65536;  // positions per sequence (LDS bitmap of 8 KB)
constexpr int kListPre = 4;            // list entries per thread loaded before the count is known

template <bool kBf16>
__device__ __forceinline__ void acc_chunk(Acc& s, const uint4& a, const uint4& b) {
  if constexpr (kBf16) {
    acc_bf16_word(s, a.x, b.x);
    acc_bf16_word(s, a.y, b.y);
    acc_bf16_word(s, a.z, b.z);
    acc_bf16_word(s, a.w, b.w);
  } else {
    acc_f32_pair(s, a.x, a.y, b.x, b.y);
    acc_f32_pair(s, a.z, a.w, b.z, b.w);
  }
}

template <bool kBf16>
__global__ __launch_bounds__(256) void k_distance_rows(const uint4* __restrict__ xc,
                                                       uint4* __restrict__ xp, int N, int chunks,
                                                       const int32_t* __restrict__ sel_idx,
                                                       const int32_t* __restrict__ sel_count,
                                                       int roll, float* __restrict__ dist) {
  __shared__ uint32_t listed[kMaxRowsBitmap / 32];
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.y;
  const int j = blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  const int32_t* lst = sel_idx + int64_t(b) * N;
  int cnt = sel_count[b];
  const int pos = j < N ? lst[j] : -1;
  int pre[kListPre];
#pragma unroll
  for (int k = 0; k < kListPre; ++k) {
    const int i = threadIdx.x + k * 256;
    pre[k] = i < N ? lst[i] : -1;
  }
  const int words = (N + 31) / 32;
  for (int i = threadIdx.x; i < words; i += blockDim.x) listed[i] = 0u;
  cnt = cnt < 0 ? 0 : (cnt > N ? N : cnt);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kListPre; ++k) {
    const int i = threadIdx.x + k * 256, p = pre[k];
    if (i < cnt && p >= 0 && p < N) atomicOr(&listed[p >> 5], 1u << (p & 31));
  }
  for (int i = threadIdx.x + kListPre * 256; i < cnt; i += blockDim.x) {
    const int p = lst[i];
    if (p >= 0 && p < N) atomicOr(&listed[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  if (j < N && lane == 0 && ((listed[j >> 5] >> (j & 31)) & 1u) == 0u)
    dist[int64_t(b) * N + j] = 0.0f;
  if (j >= cnt || pos < 0 || pos >= N) return;
  const int64_t row = int64_t(b) * N + pos;
  const uint4* a = xc + row * chunks;
  uint4* p = xp + row * chunks;
  if (chunks <= kWave * kUnroll) {
    // the whole row in one round of loads: distance, then the roll from the same registers
    uint4 ra[kUnroll], rb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = u * kWave + lane;
      ra[u] = c < chunks ? load_nt(a + c) : make_uint4(0, 0, 0, 0);
      rb[u] = c < chunks ? load_nt(p + c) : make_uint4(0, 0, 0, 0);
    }
    Acc sacc;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc_chunk<kBf16>(sacc, ra[u], rb[u]);
    const double d = finish_distance(sacc);
    if (lane == 0) dist[row] = float(d);
    if (roll) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = u * kWave + lane;
        if (c < chunks) p[c] = ra[u];
      }
    }
    return;
  }
  const double d = row_distance<kBf16>(a, p, chunks, lane);
  if (lane == 0) dist[row] = float(d);
  if (roll)
    for (int c = lane; c < chunks; c += kWave) p[c] = a[c];
}

// one workgroup per group; fixed per-thread strides and a fixed reduction tree
__global__ __launch_bounds__(256) void k_group_mean(const float* __restrict__ dist, int64_t N,
                                                    float* __restrict__ mean) {
  __shared__ double part[4];
  const float* p = dist + int64_t(blockIdx.x) * N;
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < N; i += blockDim.x) acc += double(p[i]);
  acc = wave_sum(acc);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = (part[0] + part[1]) + (part[2] + part[3]);
    mean[blockIdx.x] = float(tot / double(N));
  }
}

}  // namespace
}  // namespace dcu

extern "C" int dcu_distance(const void* x_cur, const void* x_prev, int32_t dtype, int64_t G,
                            int64_t N, int64_t d, float* dist, float* mean, void* stream) {
  if (!x_cur || !x_prev || !dist || G <= 0 || N <= 0 || d <= 0) return DCU_EINVAL;
  if (dtype != DCU_BF16 && dtype != DCU_F32) return DCU_EINVAL;
  const int64_t per_chunk = dtype == DCU_BF16 ? 8 : 4;
  if (d % per_chunk != 0) return DCU_EUNSUPPORTED;
  if (!dcu_aligned16(x_cur) || !dcu_aligned16(x_prev)) return DCU_EUNSUPPORTED;
  if (G > (int64_t(1) << 31) - 1) return DCU_EUNSUPPORTED;
  const int64_t chunks = d / per_chunk;
  if (chunks > (int64_t(1) << 30)) return DCU_EUNSUPPORTED;
  const int64_t rows = G * N;
  const int64_t blocks = (rows + dcu::kRowsPerBlock - 1) / dcu::kRowsPerBlock;
  if (blocks > (int64_t(1) << 31) - 1) return DCU_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* a = static_cast<const uint4*>(x_cur);
  const uint4* b = static_cast<const uint4*>(x_prev);
  if (dtype == DCU_BF16)
    hipLaunchKernelGGL(dcu::k_distance<true>, dim3(unsigned(blocks)), dim3(256), 0, s, a, b, rows,
                       int(chunks), dist);
  else
    hipLaunchKernelGGL(dcu::k_distance<false>, dim3(unsigned(blocks)), dim3(256), 0, s, a, b, rows,
                       int(chunks), dist);
  DCU_LAUNCH_CHECK();
  if (mean) {
    hipLaunchKernelGGL(dcu::k_group_mean, dim3(unsigned(G)), dim3(256), 0, s, dist, N, mean);
    DCU_LAUNCH_CHECK();
  }
  return DCU_OK;
}

extern "C" int dcu_distance_rows(const void* x_cur, void* x_prev, int32_t dtype, int64_t B,
                                 int64_t N, int64_t d, const int32_t* sel_idx,
                                 const int32_t* sel_count, float* dist, int32_t roll,
                                 void* stream) {
  if (!x_cur || !x_prev || !sel_idx || !sel_count || !dist || B <= 0 || N <= 0 || d <= 0)
    return DCU_EINVAL;
  if (dtype != DCU_BF16 && dtype != DCU_F32) return DCU_EINVAL;
  const int64_t per_chunk = dtype == DCU_BF16 ? 8 : 4;
  if (d % per_chunk != 0) return DCU_EUNSUPPORTED;
  if (!dcu_aligned16(x_cur) || !dcu_aligned16(x_prev)) return DCU_EUNSUPPORTED;
  if (B > 65535 || N > dcu::kMaxRowsBitmap) return DCU_EUNSUPPORTED;
  const int64_t chunks = d / per_chunk;
  if (chunks > (int64_t(1) << 30)) return DCU_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned((N + dcu::kRowsPerBlock - 1) / dcu::kRowsPerBlock), unsigned(B));
  const uint4* xc = static_cast<const uint4*>(x_cur);
  uint4* xp = static_cast<uint4*>(x_prev);
  if (dtype == DCU_BF16)
    hipLaunchKernelGGL(dcu::k_distance_rows<true>, grid, dim3(256), 0, s, xc, xp, int(N),
                       int(chunks), sel_idx, sel_count, int(roll), dist);
  else
    hipLaunchKernelGGL(dcu::k_distance_rows<false>, grid, dim3(256), 0, s, xc, xp, int(N),
                       int(chunks), sel_idx, sel_count, int(roll), dist);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
