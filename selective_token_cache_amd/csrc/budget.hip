// dcu_budget: split T = b_layer * L recompute slots across layers in proportion to the previous
// step's layer means.
// Dynamic-dLLM reading notes, Key design 1 (DCU), the per-layer budget equation
// B^{t,l} = (B_layer * LayerNum) * s^{t+1,l} / sum_k s^{t+1,k} (step t+1 is the previous step).
//
// The page gives a real-valued share; the integer budget is floor plus largest remainder (ties to
// the lower layer) in IEEE fp64 with a fixed operation order: S summed sequentially in ascending
// layer order, q_l = (T*s_l)/S, r_l = q_l - floor(q_l). Every step is exactly rounded and done in
// the same order as a sequential CPU evaluation, so the result is bit-for-bit reproducible.
// A mean is an average of distances in [0, 2]; a negative entry is read as 0. With every s_l >= 0
// the floors never sum past T (S is at least (1 - (L-1) 2^-53) times the exact sum and each q_l at
// most T s_l (1 + 2^-53)^2 / S, so sum_l q_l < T + 1 for T < 2^31, L <= 1024), hence the only
// correction is +1 on the T - sum floor(q_l) largest remainders.
// One workgroup per sequence, one thread per layer; latency-bound (L <= 1024 values).
#include "common.h"

#pragma clang fp contract(off)

namespace dcu {
namespace {

__global__ __launch_bounds__(1024) void k_budget(const float* __restrict__ s_prev, int B, int L,
                                                 int b_layer, int32_t* __restrict__ budget) {
  __shared__ float s_s[1024];
  __shared__ double s_r[1024];
  __shared__ double s_S;
  __shared__ int s_scan[17];
  const int b = blockIdx.x;
  const int l = threadIdx.x;
  const int T = b_layer * L;
  int32_t* out = budget + int64_t(b) * L;
  if (s_prev == nullptr) {
    if (l < L) out[l] = b_layer;
    return;
  }
  if (l < L) {
    const float v = s_prev[int64_t(l) * B + b];  // layer-major [L, B]
    s_s[l] = v > 0.0f ? v : 0.0f;
  }
  __syncthreads();
  if (l == 0) {
    double S = 0.0;
    for (int k = 0; k < L; ++k) S += double(s_s[k]);
    s_S = S;
  }
  __syncthreads();
  const double S = s_S;
  if (S == 0.0) {
    if (l < L) out[l] = b_layer;
    return;
  }
  int f = 0;
  double r = 0.0;
  if (l < L) {
    const double q = (double(T) * double(s_s[l])) / S;
    const double fl = floor(q);
    r = q - fl;
    f = int(fl);
    s_r[l] = r;
  }
  const int sumf = block_sum_int(l < L ? f : 0, s_scan);  // includes a __syncthreads
  const int R = T - sumf;                                  // >= 0 (see above)
  if (l < L) {
    int rank = 0;
    for (int k = 0; k < L; ++k) {
      const double rk = s_r[k];
      rank += (rk > r || (rk == r && k < l)) ? 1 : 0;
    }
    if (rank < R) f += 1;
    out[l] = f;
  }
}

}  // namespace
}  // namespace dcu

extern "C" int dcu_budget(const float* s_prev, int32_t B, int32_t L, int32_t b_layer,
                          int32_t* budget, void* stream) {
  if (!budget || B <= 0 || L <= 0 || b_layer < 0) return DCU_EINVAL;
  if (int64_t(b_layer) * int64_t(L) > int64_t(INT32_MAX)) return DCU_EINVAL;
  if (L > 1024) return DCU_EUNSUPPORTED;
  const int threads = ((L + 63) / 64) * 64;
  hipLaunchKernelGGL(dcu::k_budget, dim3(unsigned(B)), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), s_prev, int(B), int(L), int(b_layer), budget);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
