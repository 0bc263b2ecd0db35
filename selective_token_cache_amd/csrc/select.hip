// dcu_select: per-sequence recompute set of one layer = forced windows united with the top-b
// tokens by distance outside the windows.
// Dynamic-dLLM reading notes, Key design 1 (top-B tokens by distance d_i are recomputed) and Key
// design 2 (a window of B_window positions around each key token unmasked at the previous step is
// always recomputed; the remaining budget is spent outside the window).
//
// Design: one workgroup per sequence (256 threads up to N = 2048, else 1024), every thread owning
// E = ceil(N / threads) <= 8 consecutive positions in registers (N <= 8192).
//  1. window mask and candidate flags (not in a window, d > 0); key = fp32 bits of d (monotone for
//     d >= 0), 0 for non-candidates;
//  2. the k-th largest key by an 8-bit LDS radix select (histograms of the keys that share the
//     prefix found so far, in two alternating LDS histograms; after each, one wave scans the 256
//     bins from the top, 4 per lane, and clears the other histogram: two barriers per pass). The
//     first histogram also gives the candidate count, so k = min(budget, candidates) needs no pass
//     of its own. A pass whose threshold bin is taken whole ends the search: every key at or above
//     that bin's lowest key is selected;
//  3. only when the last pass takes part of a run of equal keys are those taken lowest position
//     first (a block scan gives each tied key its rank);
//  4. a block scan compacts W u A into ascending positions.
// The result is exact integer work: bit-identical to a sort by (d desc, position asc).
#include "common.h"

namespace dcu {
namespace {

constexpr int kMaxE = 8;  // positions per thread

template <int kT>
__global__ __launch_bounds__(kT) void k_select(const float* __restrict__ dist,
                                               const int32_t* __restrict__ budgets, int L,
                                               int layer, const int32_t* __restrict__ key_pos,
                                               int P, int N, int b_window,
                                               int32_t* __restrict__ sel_idx,
                                               int32_t* __restrict__ sel_count,
                                               float* __restrict__ mean) {
  __shared__ int hist[2][256];  // radix histograms, used alternately
  __shared__ int scan_lds[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining, s_bin_count, s_k, s_nc;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int E = (N + kT - 1) / kT;
  const int i0 = t * E;
  const float* d = dist + int64_t(b) * N;
  const int32_t* keys = key_pos ? key_pos + int64_t(b) * P : nullptr;
  const int half = b_window / 2;
  int budget = budgets[int64_t(b) * L + layer];  // issued early: its latency overlaps the loads below
  for (int j = t; j < 256; j += kT) hist[0][j] = 0;

  uint32_t key[kMaxE];
  bool inw[kMaxE];
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
      if (!w && v > 0.0f) key[e] = __float_as_uint(v);
    }
  }
  // optional layer mean, formed exactly as dcu_distance forms it (256 threads with fixed strides,
  // fp64, wave sums, then (w0 + w1) + (w2 + w3)); its loads overlap the ones above, and the
  // barriers below publish the wave partials
  __shared__ double mpart[4];
  if (mean) {
    double acc = 0.0;
    if (t < 256)
      for (int i = t; i < N; i += 256) acc += double(d[i]);
    acc = wave_sum(acc);
    if (t < 256 && (t & (kWave - 1)) == 0) mpart[t / kWave] = acc;
  }
  budget = budget < 0 ? 0 : budget;
  __syncthreads();  // the first histogram is cleared before any thread counts into it

  // radix passes: prefix of the threshold key, how many keys at the threshold are still needed,
  // and how many keys share that prefix
  uint32_t prefix = 0u;
  int remaining = 0, bin_count = 0, k = 0, nC = 0;
  bool whole = false;  // the last bin found is taken whole: select key >= prefix
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
    if (pass == 0 && mean && t == 0)
      mean[b] = float(((mpart[0] + mpart[1]) + (mpart[2] + mpart[3])) / double(N));
    if (t < kWave) {
      // wave 0: lane l holds bins 255-4l .. 252-4l (descending); an inclusive scan over the lanes
      // finds the bin that holds the remaining-th largest key
      const int b0 = 255 - 4 * lane;
      const int c0 = H[b0], c1 = H[b0 - 1], c2 = H[b0 - 2], c3 = H[b0 - 3];
      const int sum = c0 + c1 + c2 + c3;
      const int inc = wave_incl_scan(sum);
      const int exc = inc - sum;
      int need = remaining;
      if (pass == 0) {
        // every candidate is in the first histogram: k = min(budget, candidates)
        const int total = __shfl(inc, kWave - 1, kWave);
        need = budget < total ? budget : total;
        if (lane == 0) {
          s_k = need;
          s_nc = total;
        }
      }
      if (need > 0 && exc < need && inc >= need) {
        const int r = need - exc;
        int bin, rem, cnt;
        if (r <= c0) {
          bin = b0; rem = r; cnt = c0;
        } else if (r <= c0 + c1) {
          bin = b0 - 1; rem = r - c0; cnt = c1;
        } else if (r <= c0 + c1 + c2) {
          bin = b0 - 2; rem = r - c0 - c1; cnt = c2;
        } else {
          bin = b0 - 3; rem = r - c0 - c1 - c2; cnt = c3;
        }
        s_prefix = prefix | (uint32_t(bin) << shift);
        s_remaining = rem;
        s_bin_count = cnt;
      }
      // the other histogram is free (its pass ended two barriers ago): clear it for the next
      int* Hn = hist[(pass + 1) & 1];
      Hn[b0] = 0; Hn[b0 - 1] = 0; Hn[b0 - 2] = 0; Hn[b0 - 3] = 0;
    }
    __syncthreads();  // threshold bin published
    if (pass == 0) {
      k = s_k;
      nC = s_nc;
      if (k == 0 || k == nC) break;  // none, or every candidate
    }
    prefix = s_prefix;
    remaining = s_remaining;
    bin_count = s_bin_count;
    if (remaining == bin_count) {  // the whole bin is taken (block-uniform: from LDS)
      whole = true;
      break;
    }
  }

  // keys equal to the threshold key when only part of them is taken: rank each by position
  const bool ties = k > 0 && k < nC && !whole;
  int eq_before = 0;
  if (ties) {
    int neq = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) neq += (key[e] != 0u && key[e] == prefix) ? 1 : 0;
    int dummy_total;
    eq_before = block_excl_scan(neq, scan_lds, &dummy_total);
  }

  int nu = 0;
  bool u[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    bool sel = false;
    if (key[e] != 0u && k > 0) {
      if (k == nC || whole) {
        sel = k == nC || key[e] >= prefix;
      } else if (key[e] > prefix) {
        sel = true;
      } else if (key[e] == prefix) {
        sel = eq_before < remaining;
        ++eq_before;
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
  for (int i = total + t; i < N; i += kT) out[i] = -1;
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
  if (N > 1024 * dcu::kMaxE) return DCU_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N <= 256 * dcu::kMaxE)
    hipLaunchKernelGGL(dcu::k_select<256>, dim3(unsigned(B)), dim3(256), 0, s, dist, budgets,
                       int(L), int(layer), key_pos, int(P), int(N), int(b_window), sel_idx,
                       sel_count, mean);
  else
    hipLaunchKernelGGL(dcu::k_select<1024>, dim3(unsigned(B)), dim3(1024), 0, s, dist, budgets,
                       int(L), int(layer), key_pos, int(P), int(N), int(b_window), sel_idx,
                       sel_count, mean);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}
