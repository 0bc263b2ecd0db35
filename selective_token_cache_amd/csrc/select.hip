// dcu_select: per-sequence recompute set of one layer = forced windows united with the top-b
// tokens by distance outside the windows.
// Dynamic-dLLM reading notes, Key design 1 (top-B tokens by distance d_i are recomputed) and Key
// design 2 (a window of B_window positions around each key token unmasked at the previous step is
// always recomputed; the remaining budget is spent outside the window).
//
// Design: one 1024-thread workgroup per sequence, every thread owning E = ceil(N/1024) consecutive
// positions in registers (N <= 8192).
//  1. window mask and candidate flags (not in a window, d > 0); key = fp32 bits of d (monotone for
//     d >= 0), 0 for non-candidates;
//  2. exact k-th largest key by an 8-bit LDS radix select (4 histogram passes into two alternating
//     LDS histograms; after each, one wave scans the 256 bins from the top, 4 per lane, and clears
//     the other histogram: two barriers per pass);
//  3. keys equal to the threshold are taken lowest position first (a block scan gives each tied
//     key its rank);
//  4. a block scan compacts W u A into ascending positions.
// The result is exact integer work: bit-identical to a sort by (d desc, position asc).
#include "common.h"

namespace dcu {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxE = 8;  // N <= 8192

__global__ __launch_bounds__(kThreads) void k_select(const float* __restrict__ dist,
                                                     const int32_t* __restrict__ budgets, int L,
                                                     int layer, const int32_t* __restrict__ key_pos,
                                                     int P, int N, int b_window,
                                                     int32_t* __restrict__ sel_idx,
                                                     int32_t* __restrict__ sel_count,
                                                     float* __restrict__ mean) {
  __shared__ int hist[2][256];  // radix histograms, used alternately
  __shared__ int scan_lds[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int E = (N + kThreads - 1) / kThreads;
  const int i0 = t * E;
  const float* d = dist + int64_t(b) * N;
  const int32_t* keys = key_pos ? key_pos + int64_t(b) * P : nullptr;
  const int half = b_window / 2;
  int budget = budgets[int64_t(b) * L + layer];  // issued early: its latency overlaps the loads below
  if (t < 256) hist[0][t] = 0;  // ordered before the first pass by the block sum's barriers

  uint32_t key[kMaxE];
  bool inw[kMaxE];
  int ncand = 0;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    key[e] = 0u;
    inw[e] = false;
    const int i = i0 + e;
    if (e < E && i < N) {
      bool w = false;
      if (b_window > 0) {
        for (int k = 0; k < P; ++k) {
          const int p = keys[k];
          if (p < 0 || p >= N) continue;
          const int lo = p - half;
          w |= (i >= lo) && (i <= lo + b_window - 1);
        }
      }
      inw[e] = w;
      const float v = d[i];
      if (!w && v > 0.0f) {
        key[e] = __float_as_uint(v);
        ++ncand;
      }
    }
  }
  // optional layer mean, formed exactly as dcu_distance forms it (256 threads with fixed strides,
  // fp64, wave sums, then (w0 + w1) + (w2 + w3)); its loads overlap the ones above, and the barrier
  // of the block sum below publishes the wave partials
  __shared__ double mpart[4];
  if (mean) {
    double acc = 0.0;
    if (t < 256)
      for (int i = t; i < N; i += 256) acc += double(d[i]);
    acc = wave_sum(acc);
    if (t < 256 && (t & (kWave - 1)) == 0) mpart[t / kWave] = acc;
  }
  const int nC = block_sum_int(ncand, scan_lds);
  if (mean && t == 0)
    mean[b] = float(((mpart[0] + mpart[1]) + (mpart[2] + mpart[3])) / double(N));
  budget = budget < 0 ? 0 : budget;
  const int k = budget < nC ? budget : nC;

  // threshold key K and how many keys equal to K are taken
  uint32_t K = 0xffffffffu;
  int take_eq = 0;
  bool all = false;
  if (k == nC) {
    all = true;
  } else if (k > 0) {
    uint32_t prefix = 0u;
    int remaining = k;
    const int lane = t & (kWave - 1);
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
      int* H = hist[pass & 1];
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) {
        if (key[e] != 0u && ((key[e] ^ prefix) & hi_mask) == 0u)
          atomicAdd(&H[(key[e] >> shift) & 255u], 1);
      }
      __syncthreads();  // histogram complete
      if (t < kWave) {
        // wave 0: lane l holds bins 255-4l .. 252-4l (descending); an inclusive scan over the lanes
        // finds the bin that holds the remaining-th largest key
        const int b0 = 255 - 4 * lane;
        const int c0 = H[b0], c1 = H[b0 - 1], c2 = H[b0 - 2], c3 = H[b0 - 3];
        const int sum = c0 + c1 + c2 + c3;
        const int inc = wave_incl_scan(sum);
        const int exc = inc - sum;
        if (exc < remaining && inc >= remaining) {
          const int r = remaining - exc;
          int bin, rem;
          if (r <= c0) {
            bin = b0; rem = r;
          } else if (r <= c0 + c1) {
            bin = b0 - 1; rem = r - c0;
          } else if (r <= c0 + c1 + c2) {
            bin = b0 - 2; rem = r - c0 - c1;
          } else {
            bin = b0 - 3; rem = r - c0 - c1 - c2;
          }
          s_prefix = prefix | (uint32_t(bin) << shift);
          s_remaining = rem;
        }
        // the other histogram is free (its pass ended two barriers ago): clear it for the next
        int* Hn = hist[(pass + 1) & 1];
        Hn[b0] = 0; Hn[b0 - 1] = 0; Hn[b0 - 2] = 0; Hn[b0 - 3] = 0;
      }
      __syncthreads();  // threshold bin published
      prefix = s_prefix;
      remaining = s_remaining;
    }
    K = prefix;
    take_eq = remaining;
  }

  // rank of each key equal to K among the tied keys (position order)
  int neq = 0;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) neq += (key[e] != 0u && key[e] == K) ? 1 : 0;
  int dummy_total;
  int eq_before = block_excl_scan(neq, scan_lds, &dummy_total);

  bool u[kMaxE];
  int nu = 0;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    bool sel = false;
    if (key[e] != 0u) {
      if (all) {
        sel = true;
      } else if (k > 0) {
        if (key[e] > K) {
          sel = true;
        } else if (key[e] == K) {
          sel = eq_before < take_eq;
          ++eq_before;
        }
      }
    }
    u[e] = inw[e] || sel;
    nu += u[e] ? 1 : 0;
  }
  int total;
  int pos = block_excl_scan(nu, scan_lds, &total);
  int32_t* out = sel_idx + int64_t(b) * N;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    if (u[e]) out[pos++] = i0 + e;
  }
  for (int i = total + t; i < N; i += kThreads) out[i] = -1;
  if (t == 0) sel_count[b] = total;
}

}  // namespace
}  // namespace dcu

extern "C" int dcu_select(const float* dist, const int32_t* budgets, int32_t L, int32_t layer,
                          const int32_t* key_pos, int32_t P, int32_t B, int32_t N,
                          int32_t b_window, int32_t* sel_idx, int32_t* sel_count, float* mean,
                          void* stream) {
  if (!dist || !budgets || !sel_idx || !sel_count) return DCU_EINVAL;
  if (B <= 0 || N <= 0 || L <= 0 || P < 0 || b_window < 0) return DCU_EINVAL;
  if (layer < 0 || layer >= L) return DCU_EINVAL;
  if (P > 0 && !key_pos) return DCU_EINVAL;
  if (N > dcu::kThreads * dcu::kMaxE) return DCU_EUNSUPPORTED;
  hipLaunchKernelGGL(dcu::k_select, dim3(unsigned(B)), dim3(dcu::kThreads), 0,
                     static_cast<hipStream_t>(stream), dist, budgets, int(L), int(layer), key_pos,
                     int(P), int(N), int(b_window), sel_idx, sel_count, mean);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
