// frechet_commit: how many candidate positions commit at the end of a denoising step.
// Fast-dLLM++ reading notes, Key design 1 (Theorem 4.1: Frechet lower bound
// L_n = max{0, sum_{j<=n} c_(j) - (n-1)} and competitor bound U_n = 1 - c_(n)) and Key design 2
// (commit n* = max{n : L_n - U_n > delta}, else n* = 1; one sort and one prefix sum per step).
//
// Design: one 1024-thread workgroup per sequence (m <= 8192 candidates).
//  1. 64-bit keys (descending-orderable confidence bits << 32 | slot) are bitonic-sorted in LDS,
//     giving (c desc, slot asc);
//  2. prefix sums in fp64. When every c is 0 or in [2^-17, 1] (always the case for softmax
//     confidences of a vocabulary below 2^17) every term is a multiple of 2^-40 and every partial
//     sum is below 2^13, so the sums are exact in any order and a parallel block scan equals the
//     sequential sum bit for bit. Otherwise one thread takes the sequential sum in sorted order;
//  3. each n evaluates G_n > delta; n* is the block-wide maximum such n (no monotonicity assumed).
// The same kernel applies the two rules that page compares against (its motivation section): the
// factor rule, n* = max{n : (n+1)(1 - c_(n)) < f}, and the threshold rule, every candidate with
// c_i >= tau (a prefix of the sorted order); both in fp64, both commit at least one candidate.
// With per-candidate thresholds (adaptive parallel decoding, Dynamic-dLLM notes Key design 3) every
// candidate with c_i >= tau_i commits (fp32 compare); those lead the order, at least one commits.
#include "common.h"

#pragma clang fp contract(off)

namespace dcu {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxM = 8192;

__device__ __forceinline__ uint32_t desc_key(float c) {
  // ascending-orderable float bits, then complemented so that larger c sorts first
  uint32_t u = __float_as_uint(c);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~u;
}

__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    double o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void k_frechet(const float* __restrict__ conf,
                                                      const int32_t* __restrict__ m_valid, int m,
                                                      int rule, double param,
                                                      const float* __restrict__ tau,
                                                      int32_t* __restrict__ n_commit,
                                                      int32_t* __restrict__ order) {
  const double delta = param;
  // per-candidate thresholds: the pass flag is the key's top bit (passing candidates sort first),
  // the confidence bits sit below it and the slot in the low 31 bits
  const bool per_tau = rule == DCU_COMMIT_TAU;
  const int vshift = per_tau ? 31 : 32;
  const uint64_t slot_mask = per_tau ? 0x7fffffffull : 0xffffffffull;
  extern __shared__ uint64_t keys[];  // P2 entries
  __shared__ double wsum[kThreads / kWave];
  __shared__ int s_flag[17];
  __shared__ int s_best[kThreads / kWave];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  int mv = m_valid ? m_valid[b] : m;
  mv = mv < 0 ? 0 : (mv > m ? m : mv);
  const float* c = conf + int64_t(b) * m;
  int32_t* ord = order + int64_t(b) * m;
  if (mv == 0) {
    for (int i = t; i < m; i += kThreads) ord[i] = -1;
    if (t == 0) n_commit[b] = 0;
    return;
  }
  int P2 = 1;
  while (P2 < mv) P2 <<= 1;
  // load keys and test the exactness precondition
  int bad = 0, npass = 0;
  for (int i = t; i < P2; i += kThreads) {
    if (i < mv) {
      const float v = c[i];
      const float av = fabsf(v);
      bad |= !(v == 0.0f || (av >= 0x1p-17f && av <= 1.0f));
      uint64_t k = (uint64_t(desc_key(v)) << vshift) | uint32_t(i);
      if (per_tau) {
        const bool pass = v >= tau[int64_t(b) * m + i];
        npass += pass ? 1 : 0;
        k |= uint64_t(pass ? 0 : 1) << 63;
      }
      keys[i] = k;
    } else {
      keys[i] = ~uint64_t(0);
    }
  }
  const int nbad = block_sum_int(bad, s_flag);
  const int n_pass = per_tau ? block_sum_int(npass, s_flag) : 0;
  // bitonic sort, ascending keys
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P2; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = keys[i], bb = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > bb) == up) {
            keys[i] = bb;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // sorted values, then inclusive prefix sums in fp64
  const int E = (mv + kThreads - 1) / kThreads;
  const int i0 = t * E;
  // value of sorted entry i (inverse of desc_key)
  auto value_at = [&](int i) -> double {
    const uint32_t dk = uint32_t(keys[i] >> vshift);
    uint32_t u = ~dk;
    u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
    return double(__uint_as_float(u));
  };
  int best = 0;
  if (per_tau) {
    best = n_pass;  // the passing candidates lead the order
  } else if (rule != DCU_COMMIT_FRECHET) {
    // per-candidate tests, no sums: (n+1)(1 - c_(n)) < f, or c_(n) >= tau
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i >= mv) break;
      const double cn = value_at(i);
      const bool ok = rule == DCU_COMMIT_FACTOR ? (double(i + 2) * (1.0 - cn) < param)
                                                : (cn >= param);
      if (ok) best = i + 1;
    }
  } else if (nbad == 0) {
    double loc = 0.0;
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i < mv) loc += value_at(i);
    }
    const double inc = wave_incl_scan_f64(loc);
    if ((t & (kWave - 1)) == kWave - 1) wsum[t / kWave] = inc;
    __syncthreads();
    double before = 0.0;
    for (int w = 0; w < t / kWave; ++w) before += wsum[w];
    double S = before + inc - loc;
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i >= mv) break;
      const double cn = value_at(i);
      S += cn;
      const double n = double(i + 1);
      const double Ln = (S - (n - 1.0)) > 0.0 ? (S - (n - 1.0)) : 0.0;
      const double G = Ln - (1.0 - cn);
      if (G > delta) best = i + 1;
    }
  } else if (t == 0) {
    double S = 0.0;
    for (int i = 0; i < mv; ++i) {
      const double cn = value_at(i);
      S += cn;
      const double n = double(i + 1);
      const double Ln = (S - (n - 1.0)) > 0.0 ? (S - (n - 1.0)) : 0.0;
      const double G = Ln - (1.0 - cn);
      if (G > delta) best = i + 1;
    }
  }
  best = wave_max(best);
  if ((t & (kWave - 1)) == 0) s_best[t / kWave] = best;
  __syncthreads();
  if (t == 0) {
    int bst = 0;
    for (int w = 0; w < kThreads / kWave; ++w) bst = s_best[w] > bst ? s_best[w] : bst;
    n_commit[b] = bst > 0 ? bst : 1;
  }
  for (int i = t; i < m; i += kThreads) ord[i] = i < mv ? int32_t(keys[i] & slot_mask) : -1;
}

// the positions of the first min(n_commit, P) committed slots of each sequence, -1 after them
__global__ __launch_bounds__(256) void k_commit_positions(const int32_t* __restrict__ order,
                                                          const int32_t* __restrict__ n_commit,
                                                          const int32_t* __restrict__ slot_pos,
                                                          int m, int P,
                                                          int32_t* __restrict__ key_pos) {
  const int b = blockIdx.x;
  int n = n_commit[b];
  n = n < 0 ? 0 : (n > m ? m : n);
  for (int k = threadIdx.x; k < P; k += blockDim.x) {
    int32_t pos = -1;
    if (k < n) {
      const int slot = order[int64_t(b) * m + k];
      if (slot >= 0 && slot < m) pos = slot_pos[int64_t(b) * m + slot];
    }
    key_pos[int64_t(b) * P + k] = pos;
  }
}

}  // namespace
}  // namespace dcu

extern "C" int dllm_commit(const float* conf, const int32_t* m_valid, int32_t B, int32_t m,
                           int32_t rule, double param, const float* tau, int32_t* n_commit,
                           int32_t* order, void* stream) {
  if (!conf || !n_commit || !order || B <= 0 || m <= 0) return DCU_EINVAL;
  if (rule != DCU_COMMIT_FRECHET && rule != DCU_COMMIT_FACTOR && rule != DCU_COMMIT_THRESHOLD &&
      rule != DCU_COMMIT_TAU)
    return DCU_EINVAL;
  if (rule == DCU_COMMIT_TAU && !tau) return DCU_EINVAL;
  if (param != param || param - param != 0.0) return DCU_EINVAL;  // NaN or infinite
  if (rule == DCU_COMMIT_FRECHET && !(param >= 0.0)) return DCU_EINVAL;
  if (m > dcu::kMaxM) return DCU_EUNSUPPORTED;
  int P2 = 1;
  while (P2 < m) P2 <<= 1;
  const size_t lds = size_t(P2) * sizeof(uint64_t);
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(dcu::k_frechet),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
    return DCU_EHIP;
  hipLaunchKernelGGL(dcu::k_frechet, dim3(unsigned(B)), dim3(dcu::kThreads), lds,
                     static_cast<hipStream_t>(stream), conf, m_valid, int(m), int(rule), param,
                     rule == DCU_COMMIT_TAU ? tau : nullptr, n_commit, order);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}

extern "C" int frechet_commit(const float* conf, const int32_t* m_valid, int32_t B, int32_t m,
                              double delta, int32_t* n_commit, int32_t* order, void* stream) {
  if (!(delta >= 0.0)) return DCU_EINVAL;  // also rejects NaN
  return dllm_commit(conf, m_valid, B, m, DCU_COMMIT_FRECHET, delta, nullptr, n_commit, order,
                     stream);
}

extern "C" int dllm_commit_positions(const int32_t* order, const int32_t* n_commit,
                                     const int32_t* slot_pos, int32_t B, int32_t m, int32_t P,
                                     int32_t* key_pos, void* stream) {
  if (!order || !n_commit || !slot_pos || !key_pos || B <= 0 || m <= 0 || P <= 0)
    return DCU_EINVAL;
  hipLaunchKernelGGL(dcu::k_commit_positions, dim3(unsigned(B)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), order, n_commit, slot_pos, int(m), int(P),
                     key_pos);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
