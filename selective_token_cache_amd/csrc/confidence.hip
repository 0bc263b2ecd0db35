// dllm_confidence: per candidate position, the argmax of its logits and that argmax's softmax
// probability (temperature 1) over the whole vocabulary.
// Fast-dLLM++ reading notes, Key designs / overall framework: each masked position's marginal
// argmax and its confidence c_i feed the commit rule.
//
// Design (HBM-bound stream of R*V logits, VALU close to balance):
//  * one 512-thread workgroup per row; each thread walks its 16-byte chunks in increasing index
//    order with 4 chunks in flight, keeping a running (max, sum of exp, argmax) triple;
//  * a chunk's 8 exponentials are summed in fp32 and added into an fp64 running sum, rescaled only
//    when the running max grows; exp(v - m) is the hardware exp2 of (v - m) * log2(e);
//  * the argmax keeps the first (lowest) index reaching the max: per thread chunks are visited in
//    increasing order and only a strictly larger chunk max moves it; across threads equal maxima
//    resolve to the smaller index;
//  * the 512 triples combine in a fixed butterfly / tree order, so results are deterministic.
#include <math.h>

#include "common.h"

namespace dcu {
namespace {

constexpr int kThreads = 512;
constexpr int kInFlight = 4;
constexpr float kLog2e = 1.4426950408889634f;

struct Tri {
  float m;
  double s;
  int idx;
};

__device__ __forceinline__ Tri combine(Tri a, Tri b) {
  Tri r;
  r.m = a.m > b.m ? a.m : b.m;
  if (r.m == -INFINITY) {
    r.s = 0.0;
  } else {
    r.s = a.s * double(__builtin_amdgcn_exp2f((a.m - r.m) * kLog2e)) +
          b.s * double(__builtin_amdgcn_exp2f((b.m - r.m) * kLog2e));
  }
  if (a.m == r.m && b.m == r.m)
    r.idx = a.idx < b.idx ? a.idx : b.idx;
  else
    r.idx = a.m == r.m ? a.idx : b.idx;
  return r;
}

template <int kElems>
__device__ __forceinline__ void absorb(Tri& t, const float (&v)[kElems], int base) {
  float cm = v[0];
#pragma unroll
  for (int j = 1; j < kElems; ++j) cm = v[j] > cm ? v[j] : cm;
  if (cm > t.m) {
    if (t.m != -INFINITY) t.s *= double(__builtin_amdgcn_exp2f((t.m - cm) * kLog2e));
    t.m = cm;
    int first = kElems - 1;
#pragma unroll
    for (int j = kElems - 1; j >= 0; --j) first = v[j] == cm ? j : first;
    t.idx = base + first;
  }
  if (t.m == -INFINITY) return;
  // exp(v - m) as exp2((v - m) log2 e): the difference is taken first, so the maximum's own term
  // is exactly 1 and no rounding of m log2 e scales every term (a bias growing with |m|)
  float cs = 0.0f;
#pragma unroll
  for (int j = 0; j < kElems; ++j) cs += __builtin_amdgcn_exp2f((v[j] - t.m) * kLog2e);
  t.s += double(cs);
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_confidence(const uint4* __restrict__ logits,
                                                         int64_t ld_chunks, int V,
                                                         float* __restrict__ conf,
                                                         int32_t* __restrict__ token) {
  constexpr int kElems = kBf16 ? 8 : 4;
  const int64_t r = blockIdx.x;
  const uint4* row = logits + r * ld_chunks;
  const int nchunks = (V + kElems - 1) / kElems;
  Tri t{-INFINITY, 0.0, 0x7fffffff};
  for (int c0 = threadIdx.x; c0 < nchunks; c0 += kThreads * kInFlight) {
    uint4 raw[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int c = c0 + u * kThreads;
      raw[u] = c < nchunks ? load_nt(row + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int c = c0 + u * kThreads;
      if (c >= nchunks) break;
      const int base = c * kElems;
      float v[kElems];
      if constexpr (kBf16) {
        v[0] = bf_lo(raw[u].x); v[1] = bf_hi(raw[u].x);
        v[2] = bf_lo(raw[u].y); v[3] = bf_hi(raw[u].y);
        v[4] = bf_lo(raw[u].z); v[5] = bf_hi(raw[u].z);
        v[6] = bf_lo(raw[u].w); v[7] = bf_hi(raw[u].w);
      } else {
        v[0] = __uint_as_float(raw[u].x); v[1] = __uint_as_float(raw[u].y);
        v[2] = __uint_as_float(raw[u].z); v[3] = __uint_as_float(raw[u].w);
      }
      if (base + kElems > V) {
#pragma unroll
        for (int j = 0; j < kElems; ++j)
          if (base + j >= V) v[j] = -INFINITY;
      }
      absorb<kElems>(t, v, base);
    }
  }
  // wave butterfly, then a fixed tree over the 8 waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    Tri o;
    o.m = __shfl_xor(t.m, off, kWave);
    o.s = __shfl_xor(t.s, off, kWave);
    o.idx = __shfl_xor(t.idx, off, kWave);
    t = combine(t, o);
  }
  __shared__ float sm[kThreads / kWave];
  __shared__ double ss[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sm[wid] = t.m;
    ss[wid] = t.s;
    si[wid] = t.idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    Tri w[kThreads / kWave];
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) w[i] = Tri{sm[i], ss[i], si[i]};
#pragma unroll
    for (int span = 1; span < kThreads / kWave; span <<= 1)
#pragma unroll
      for (int i = 0; i + span < kThreads / kWave; i += 2 * span) w[i] = combine(w[i], w[i + span]);
    conf[r] = float(1.0 / w[0].s);
    token[r] = w[0].idx;
  }
}

}  // namespace
}  // namespace dcu

extern "C" int dllm_confidence(const void* logits, int32_t dtype, int64_t R, int64_t V,
                               int64_t ld, float* conf, int32_t* token, void* stream) {
  if (!logits || !conf || !token || R <= 0 || V <= 0 || ld < V) return DCU_EINVAL;
  if (dtype != DCU_BF16 && dtype != DCU_F32) return DCU_EINVAL;
  const int64_t per_chunk = dtype == DCU_BF16 ? 8 : 4;
  if (ld % per_chunk != 0 || !dcu_aligned16(logits)) return DCU_EUNSUPPORTED;
  if (V > int64_t(INT32_MAX) - 16 || R > int64_t(INT32_MAX)) return DCU_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* p = static_cast<const uint4*>(logits);
  if (dtype == DCU_BF16)
    hipLaunchKernelGGL(dcu::k_confidence<true>, dim3(unsigned(R)), dim3(dcu::kThreads), 0, s, p,
                       ld / per_chunk, int(V), conf, token);
  else
    hipLaunchKernelGGL(dcu::k_confidence<false>, dim3(unsigned(R)), dim3(dcu::kThreads), 0, s, p,
                       ld / per_chunk, int(V), conf, token);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
