// dllm_apd: the per-position signals and threshold of adaptive parallel decoding, in one stream
// over this step's logits and the previous step's.
// Dynamic-dLLM reading notes, Key design 3: with z the softmax distribution of a position,
// concentration c = 1 - (second-largest probability), temporal instability
// H = 1 - cos(z^t, z^{t+1}) against the previous step's distribution, and the threshold update
// tau^t = tau^{t+1} - alpha c + beta H; the confidence (largest probability) and argmax come out of
// the same pass.
//
// Design (HBM-bound: 2 * V logits per row, one 512-thread workgroup per row, the structure of
// dllm_confidence):
//  * each thread walks its 16-byte chunks in increasing index order, 4 chunks of each operand in
//    flight, keeping the running max m and argmax, the two largest values (a multiset: a tie at
//    the top makes both equal), and with e = exp(z - m), q = exp(z_prev - m_prev):
//      S = sum e, D = sum e q, Q = sum e^2, P = sum q^2;
//    chunk sums of 8 terms in fp32 are added into fp64 accumulators; S and D are rescaled by
//    exp(m_old - m_new) and Q by its square when the running max grows. m_prev is the previous
//    step's row max (kept by the caller), so q <= 1 needs no rescaling;
//  * cos(z^t, z^{t+1}) = D / sqrt(Q P): the normalisers of both softmaxes cancel;
//  * the 512 partial states combine in a fixed butterfly / tree order (deterministic).
#include <math.h>

#include "common.h"

namespace dcu {
namespace {

constexpr int kThreads = 512;
constexpr int kInFlight = 4;
constexpr float kLog2e = 1.4426950408889634f;

struct St {
  float m, m2;  // largest and second-largest logit seen (multiset)
  int idx;      // lowest index of the largest
  double s, d, q, p;
};

__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ St combine(St a, St b) {
  St r;
  r.m = a.m > b.m ? a.m : b.m;
  r.m2 = fmaxf(fminf(a.m, b.m), fmaxf(a.m2, b.m2));
  if (a.m == r.m && b.m == r.m)
    r.idx = a.idx < b.idx ? a.idx : b.idx;
  else
    r.idx = a.m == r.m ? a.idx : b.idx;
  if (r.m == -INFINITY) {
    r.s = r.d = r.q = 0.0;
  } else {
    const double fa = double(ex(a.m - r.m)), fb = double(ex(b.m - r.m));
    r.s = a.s * fa + b.s * fb;
    r.d = a.d * fa + b.d * fb;
    r.q = a.q * (fa * fa) + b.q * (fb * fb);
  }
  r.p = a.p + b.p;
  return r;
}

template <int kElems>
__device__ __forceinline__ void absorb(St& t, const float (&v)[kElems], const float (&w)[kElems],
                                       int base, bool prev, float mp) {
  float cm = v[0];
#pragma unroll
  for (int j = 1; j < kElems; ++j) cm = v[j] > cm ? v[j] : cm;
  // the two largest values of the multiset seen so far (a >= b); a chunk whose max does not exceed
  // the second largest cannot change them (the common case once the row's peak has been seen)
  if (cm > t.m2) {
    float a = t.m, b = t.m2;
#pragma unroll
    for (int j = 0; j < kElems; ++j) {
      const float x = v[j];
      if (x > a) {
        b = a;
        a = x;
      } else if (x > b) {
        b = x;
      }
    }
    t.m2 = b;
  }
  if (cm > t.m) {
    if (t.m != -INFINITY) {
      const double f = double(ex(t.m - cm));
      t.s *= f;
      t.d *= f;
      t.q *= f * f;
    }
    t.m = cm;
    int first = kElems - 1;
#pragma unroll
    for (int j = kElems - 1; j >= 0; --j) first = v[j] == cm ? j : first;
    t.idx = base + first;
  }
  if (t.m == -INFINITY) return;
  float cs = 0.0f, cd = 0.0f, cq = 0.0f, cp = 0.0f;
#pragma unroll
  for (int j = 0; j < kElems; ++j) {
    const float e = ex(v[j] - t.m);
    cs += e;
    cq += e * e;
    if (prev) {
      const float qv = ex(w[j] - mp);
      cd += e * qv;
      cp += qv * qv;
    }
  }
  t.s += double(cs);
  t.q += double(cq);
  t.d += double(cd);
  t.p += double(cp);
}

template <bool kBf16>
__device__ __forceinline__ void unpack(const uint4& raw, float (&v)[kBf16 ? 8 : 4]) {
  if constexpr (kBf16) {
    v[0] = bf_lo(raw.x); v[1] = bf_hi(raw.x);
    v[2] = bf_lo(raw.y); v[3] = bf_hi(raw.y);
    v[4] = bf_lo(raw.z); v[5] = bf_hi(raw.z);
    v[6] = bf_lo(raw.w); v[7] = bf_hi(raw.w);
  } else {
    v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
    v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void k_apd(const uint4* __restrict__ logits,
                                                  const uint4* __restrict__ prev, int64_t ld_chunks,
                                                  int V, float alpha, float beta,
                                                  float* __restrict__ tau, float* __restrict__ zmax,
                                                  float* __restrict__ conf,
                                                  int32_t* __restrict__ token,
                                                  float* __restrict__ c_out,
                                                  float* __restrict__ h_out) {
  constexpr int kElems = kBf16 ? 8 : 4;
  const int64_t r = blockIdx.x;
  const uint4* row = logits + r * ld_chunks;
  const uint4* prow = prev ? prev + r * ld_chunks : nullptr;
  const bool has_prev = prev != nullptr;
  const float mp = has_prev ? zmax[r] : 0.0f;
  const int nchunks = (V + kElems - 1) / kElems;
  St t{-INFINITY, -INFINITY, 0x7fffffff, 0.0, 0.0, 0.0, 0.0};
  for (int c0 = threadIdx.x; c0 < nchunks; c0 += kThreads * kInFlight) {
    uint4 raw[kInFlight], rawp[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int c = c0 + u * kThreads;
      raw[u] = c < nchunks ? load_nt(row + c) : make_uint4(0, 0, 0, 0);
      rawp[u] = (has_prev && c < nchunks) ? load_nt(prow + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int c = c0 + u * kThreads;
      if (c >= nchunks) break;
      const int base = c * kElems;
      float v[kElems], w[kElems];
      unpack<kBf16>(raw[u], v);
      unpack<kBf16>(rawp[u], w);
      if (base + kElems > V) {
#pragma unroll
        for (int j = 0; j < kElems; ++j)
          if (base + j >= V) {
            v[j] = -INFINITY;
            w[j] = -INFINITY;
          }
      }
      absorb<kElems>(t, v, w, base, has_prev, mp);
    }
  }
  // wave butterfly, then a fixed tree over the 8 waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    St o;
    o.m = __shfl_xor(t.m, off, kWave);
    o.m2 = __shfl_xor(t.m2, off, kWave);
    o.idx = __shfl_xor(t.idx, off, kWave);
    o.s = __shfl_xor(t.s, off, kWave);
    o.d = __shfl_xor(t.d, off, kWave);
    o.q = __shfl_xor(t.q, off, kWave);
    o.p = __shfl_xor(t.p, off, kWave);
    t = combine(t, o);
  }
  __shared__ St sw[kThreads / kWave];
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sw[wid] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    St w[kThreads / kWave];
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) w[i] = sw[i];
#pragma unroll
    for (int span = 1; span < kThreads / kWave; span <<= 1)
#pragma unroll
      for (int i = 0; i + span < kThreads / kWave; i += 2 * span) w[i] = combine(w[i], w[i + span]);
    const St f = w[0];
    const double pmax = 1.0 / f.s;
    const double p2 = f.m2 == -INFINITY ? 0.0 : double(ex(f.m2 - f.m)) / f.s;
    const double c = 1.0 - p2;
    const double h = has_prev ? 1.0 - f.d / sqrt(f.q * f.p) : 0.0;
    conf[r] = float(pmax);
    token[r] = f.idx;
    tau[r] = float(double(tau[r]) - double(alpha) * c + double(beta) * h);
    zmax[r] = f.m;
    if (c_out) c_out[r] = float(c);
    if (h_out) h_out[r] = float(h);
  }
}

}  // namespace
}  // namespace dcu

extern "C" int dllm_apd(const void* logits, const void* logits_prev, int32_t dtype, int64_t R,
                        int64_t V, int64_t ld, float alpha, float beta, float* tau, float* zmax,
                        float* conf, int32_t* token, float* c_conc, float* h_instab,
                        void* stream) {
  if (!logits || !tau || !zmax || !conf || !token || R <= 0 || V <= 0 || ld < V)
    return DCU_EINVAL;
  if (dtype != DCU_BF16 && dtype != DCU_F32) return DCU_EINVAL;
  if (!(alpha >= 0.0f) || !(beta >= 0.0f) || alpha - alpha != 0.0f || beta - beta != 0.0f)
    return DCU_EINVAL;  // negative, NaN or infinite
  const int64_t per_chunk = dtype == DCU_BF16 ? 8 : 4;
  if (ld % per_chunk != 0 || !dcu_aligned16(logits)) return DCU_EUNSUPPORTED;
  if (logits_prev && !dcu_aligned16(logits_prev)) return DCU_EUNSUPPORTED;
  if (V > int64_t(INT32_MAX) - 16 || R > int64_t(INT32_MAX)) return DCU_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4* p = static_cast<const uint4*>(logits);
  const uint4* q = static_cast<const uint4*>(logits_prev);
  if (dtype == DCU_BF16)
    hipLaunchKernelGGL(dcu::k_apd<true>, dim3(unsigned(R)), dim3(dcu::kThreads), 0, s, p, q,
                       ld / per_chunk, int(V), alpha, beta, tau, zmax, conf, token, c_conc,
                       h_instab);
  else
    hipLaunchKernelGGL(dcu::k_apd<false>, dim3(unsigned(R)), dim3(dcu::kThreads), 0, s, p, q,
                       ld / per_chunk, int(V), alpha, beta, tau, zmax, conf, token, c_conc,
                       h_instab);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
