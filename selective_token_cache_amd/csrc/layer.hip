// dcu_selective_layer: recompute only the selected rows of one transformer layer.
// Dynamic-dLLM reading notes, Key design 1 (DCU): the selected tokens are recomputed and every other
// token reuses its cached values; attention is bidirectional over every cached row.
//
// The layer is pre-norm: xn = RMSNorm(x; g_attn), [q|k|v] = xn W_qkv^T, attention of the selected
// queries over all N cached keys/values (no mask, scale 1/sqrt(head_dim)), a = x + o W_o^T,
// an = RMSNorm(a; g_ffn), y = a + (silu(an W_gate^T) * an W_up^T) W_down^T. Optionally (rotary
// layout) q and k of a row at position p are turned pairwise (head dims i, i + dh/2) by
// p * theta^(-2i/dh) before k is cached.
//
// Kernels, in stream order (no host synchronisation; ragged per-sequence counts stay on device):
//  1. k_gather_rmsnorm  per-sequence row offsets (clamped to the workspace capacity) from the
//                     counts, the compacted row map (selected row -> global cache row), attention
//                     query-tile tables, the gather of the selected input rows + RMSNorm -> xn,
//                     and (rotary layout) each row's (cos, sin) table;
//  2. k_gemm<QKV>     xn W_qkv^T; epilogue writes q and scatters k, v straight into the caches
//                     (k_gemm<QKV_ROPE>: the same with the rotation of q and k); for a row
//                     capacity of at most 64, k_qkv_fused does 1 and 2 in one weight stream;
//  3. k_attn<DH>      flash-style attention of each 64-query tile over the cache (split over keys
//                     when there are too few tiles to fill the chip) + k_attn_combine;
//  4. k_gemm<RESID>   o W_o^T plus the residual gathered from x -> a (fp32);
//  5. k_resid_rmsnorm the split tiles of a finished (fixed-order sums of the pieces + residual)
//                     and RMSNorm of a -> an (bf16) in one pass, a wave per row, or a workgroup per
//                     row when every tile was split (k_resid_rmsnorm_row, the same body, for a row
//                     capacity of at most 64; k_gemm_fixup + k_rmsnorm_f32 for wider rows);
//  6. k_gemm<SWIGLU>  gate and up tiles computed together; epilogue silu(g)*u -> h (bf16);
//  7. k_gemm<DOWN>    h W_down^T plus a; epilogue scatters y back into y_out.
// Split-K projections are finished by k_gemm_fixup (fixed-order sums of the pieces + epilogue).
//
// GEMM design (gfx950): the persistent MFMA core in gemm.h (global->LDS DMA, swizzled LDS, XCD-aware
// tile walk) with fused epilogues, on 128x128 tiles (4 waves of 64x64, two workgroups per CU; the
// early-refill loop for QKV, output and down, and for gate/up up to two rounds of tiles); for a
// row capacity of at most 64, a weight-streaming form (64-row tiles, one workgroup per CU).
#include <math.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace dcu {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ------------------------------------------------------------------------------ workspace header
// int32 words at the start of the workspace
constexpr int kHdrM = 0;   // rows recomputed (sum of clamped counts)
constexpr int kHdrTq = 1;  // attention query tiles
constexpr int kQTile = 64;

struct Ptrs {
  int* hdr;
  int* seq_off;   // [B+1]
  int* tile_off;  // [B+1]
  int* tile_seq;  // [Tq_max]
  int* rowmap;    // [M_cap]
  uint16_t* xn;   // [M_cap, d] (later also an)
  uint16_t* q;    // [M_cap, d]
  uint16_t* o;    // [M_cap, d]
  float* a;       // [M_cap, d]
  uint16_t* h;    // [M_cap, F]
  float* opart;   // [S, M_cap, d]      (split attention only)
  float* ml;      // [S, M_cap, H, 2]   (split attention only)
  float2* rope;   // [M_cap, rope_dh / 2] (cos, sin) of each row's rotation angles
  int rope_dh;    // head_dim with rotary embedding, else 0
  float rope_l2t; // log2(theta)
};

// Rotation angle of head-dim pair i (i < dh/2) at position pos: pos * theta^(-2i/dh), in fp32
__device__ __forceinline__ float rope_angle(float pos, int i, int dh, float l2t) {
  return pos * exp2f(-float(2 * i) * (l2t / float(dh)));
}

// ------------------------------------------------------------------------------ 1+2. plan, gather, RMSNorm
constexpr int kMaxSeqs = 4096;  // sequences per call (LDS prefix of the per-sequence counts)

// Per-sequence row offsets (counts clamped to [0, N], running total clamped to M_cap) into LDS
// off[0..B]; every workgroup of the kernel evaluates the same prefix.
__device__ void row_offsets(const int32_t* __restrict__ sel_count, int B, int N, int M_cap,
                            int* off, int* scan_lds) {
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += blockDim.x) {
    const int b = c0 + threadIdx.x;
    int c = 0;
    if (b < B) {
      c = sel_count ? sel_count[b] : N;
      c = c < 0 ? 0 : (c > N ? N : c);
    }
    int tot;
    const int ex = block_excl_scan(c, scan_lds, &tot);
    if (b < B) off[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) off[B] = carry;
  __syncthreads();
  // clamp the running total to the row capacity (later sequences lose rows first)
  for (int b = threadIdx.x; b <= B; b += blockDim.x) off[b] = off[b] < M_cap ? off[b] : M_cap;
  __syncthreads();
}

// The row count, per-sequence row offsets and attention query-tile tables (tiles of 64 query rows
// per sequence) from the LDS offsets off[0..B], written by one workgroup for the later kernels
__device__ void publish_plan(const int* off, int B, const Ptrs& P) {
  const int M = off[B];
  int toff = 0;
  for (int b = 0; b < B; ++b) {  // uniform loop
    const int nt = (off[b + 1] - off[b] + kQTile - 1) / kQTile;
    for (int j = threadIdx.x; j < nt; j += blockDim.x) P.tile_seq[toff + j] = b;
    if (threadIdx.x == 0) {
      P.seq_off[b] = off[b];
      P.tile_off[b] = toff;
    }
    toff += nt;
  }
  if (threadIdx.x == 0) {
    P.seq_off[B] = M;
    P.tile_off[B] = toff;
    P.hdr[kHdrM] = M;
    P.hdr[kHdrTq] = toff;
  }
}

// Global cache row of compacted row r (-1 for a listed position outside [0, N)) and its position
__device__ __forceinline__ int row_of(const int* off, int B, int N, const int32_t* sel_idx, int r,
                                      int* pos_out) {
  int lo = 0, hi = B - 1;  // sequence of row r: the last b with off[b] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int b = lo, j = r - off[b];
  const int pos = !sel_idx ? j : sel_idx[int64_t(b) * N + j];
  const bool valid = pos >= 0 && pos < N;
  *pos_out = valid ? pos : -1;
  return valid ? b * N + pos : -1;
}

// RMSNorm of one row by one wave: out = x * (1 / sqrt(mean(x^2) + eps)) * gain, fp32 arithmetic,
// bf16 out. NC > 0: the lane's NC 8-element groups (lane, lane + 64, ...) are loaded at once and kept
// in registers, so the row costs a single round trip to memory; NC == 0: two passes over the row.
// The per-lane accumulation order is the same in both forms.
template <int NC, bool kF32>
__device__ __forceinline__ void rms_row(const void* __restrict__ row_v,
                                        const uint16_t* __restrict__ gain, int d, float eps,
                                        uint16_t* __restrict__ orow, int lane) {
  const int groups = d / 8;
  auto load = [&](int g, float (&v)[8]) {
    if constexpr (kF32) {
      const float4* row = static_cast<const float4*>(row_v);
      const float4 u = row[2 * g], w = row[2 * g + 1];
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
      v[4] = w.x; v[5] = w.y; v[6] = w.z; v[7] = w.w;
    } else {
      const uint4 u = static_cast<const uint4*>(row_v)[g];
      v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
      v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
    }
  };
  auto sumsq = [](const float (&v)[8]) {
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k += 2) ss += v[k] * v[k] + v[k + 1] * v[k + 1];
    return ss;
  };
  auto store = [&](int g, const float (&v)[8], float scale, const uint4 gg) {
    uint4 o;
    o.x = pack_bf2(v[0] * scale * bf_lo(gg.x), v[1] * scale * bf_hi(gg.x));
    o.y = pack_bf2(v[2] * scale * bf_lo(gg.y), v[3] * scale * bf_hi(gg.y));
    o.z = pack_bf2(v[4] * scale * bf_lo(gg.z), v[5] * scale * bf_hi(gg.z));
    o.w = pack_bf2(v[6] * scale * bf_lo(gg.w), v[7] * scale * bf_hi(gg.w));
    reinterpret_cast<uint4*>(orow)[g] = o;
  };
  float ss = 0.0f;
  if constexpr (NC > 0) {
    float v[NC][8];
    uint4 gg[NC];  // the gains are loaded with the row, not after its reduction
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int g = lane + c * kWave;
      if (g < groups) {
        load(g, v[c]);
        gg[c] = reinterpret_cast<const uint4*>(gain)[g];
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[c][k] = 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) ss += sumsq(v[c]);
    ss = wave_sum(ss);
    const float scale = 1.0f / sqrtf(ss / float(d) + eps);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int g = lane + c * kWave;
      if (g < groups) store(g, v[c], scale, gg[c]);
    }
  } else {
    for (int g = lane; g < groups; g += kWave) {
      float v[8];
      load(g, v);
      ss += sumsq(v);
    }
    ss = wave_sum(ss);
    const float scale = 1.0f / sqrtf(ss / float(d) + eps);
    for (int g = lane; g < groups; g += kWave) {
      float v[8];
      load(g, v);
      store(g, v, scale, reinterpret_cast<const uint4*>(gain)[g]);
    }
  }
}

// 8-element groups per lane held in registers for a row of d elements (0: two-pass form)
inline int rms_nc(int d, bool f32) {
  const int per_lane = (d / 8 + kWave - 1) / kWave;
  const int cap = f32 ? 8 : 16;
  for (int nc = 1; nc <= cap; nc *= 2)
    if (per_lane <= nc) return nc;
  return 0;
}

// Gather of the selected rows of x + RMSNorm -> xn (bf16). Also publishes, from workgroup 0, the
// row count, per-sequence offsets and attention query-tile tables that the later kernels read,
// and writes the row map (selected row -> global cache row) for every row it normalises.
template <int NC>
__global__ __launch_bounds__(256) void k_gather_rmsnorm(const uint16_t* __restrict__ x,
                                                        const int32_t* __restrict__ sel_idx,
                                                        const int32_t* __restrict__ sel_count,
                                                        int B, int N, int M_cap,
                                                        const uint16_t* __restrict__ gain, int d,
                                                        float eps, uint16_t* __restrict__ out,
                                                        Ptrs P) {
  __shared__ int off[kMaxSeqs + 1];
  __shared__ int scan_lds[17];
  // one sequence: this wave's first row r is slot r of the list, so its position is loaded with
  // the count instead of after it (r < M_cap <= N keeps the load in bounds)
  const int r_first = blockIdx.x * 4 + threadIdx.x / kWave;
  const int pos_first = (B == 1 && sel_idx && r_first < N) ? sel_idx[r_first] : 0;
  row_offsets(sel_count, B, N, M_cap, off, scan_lds);
  const int M = off[B];
  if (blockIdx.x == 0) publish_plan(off, B, P);
  const int lane = threadIdx.x & (kWave - 1);
  for (int r = blockIdx.x * 4 + threadIdx.x / kWave; r < M; r += gridDim.x * 4) {
    // sequence of row r: the last b with off[b] <= r
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int b = lo, j = r - off[b];
    const int pos = !sel_idx ? j : (B == 1 && r == r_first ? pos_first : sel_idx[int64_t(b) * N + j]);
    // a listed position outside [0, N) is skipped: its row map entry is -1, its normalised row is
    // zero, and every later stage leaves the caches and the output alone for it
    const bool valid = pos >= 0 && pos < N;
    const int grow = valid ? b * N + pos : -1;
    if (lane == 0) P.rowmap[r] = grow;
    if (P.rope_dh > 0) {  // (cos, sin) of the row's rotation angles, read by the QKV epilogue
      for (int i = lane; i < P.rope_dh / 2; i += kWave) {
        float sn = 0.0f, cs = 1.0f;
        if (valid) sincosf(rope_angle(float(pos), i, P.rope_dh, P.rope_l2t), &sn, &cs);
        P.rope[int64_t(r) * (P.rope_dh / 2) + i] = make_float2(cs, sn);
      }
    }
    if (valid) {
      rms_row<NC, false>(x + int64_t(grow) * d, gain, d, eps, out + int64_t(r) * d, lane);
    } else {
      for (int g = lane; g < d / 8; g += kWave)
        reinterpret_cast<uint4*>(out + int64_t(r) * d)[g] = make_uint4(0, 0, 0, 0);
    }
  }
}

// RMSNorm of the fp32 rows a -> bf16, one wave per row. With rows_done, also the number of rows of
// each sequence that the layer recomputes (its compacted rows with a valid position; the row map
// is complete once the gather kernel has run, which precedes this kernel on the stream).
template <int NC>
__global__ __launch_bounds__(256) void k_rmsnorm_f32(const float* __restrict__ a,
                                                     const int* __restrict__ hdr,
                                                     const uint16_t* __restrict__ gain, int d,
                                                     float eps, uint16_t* __restrict__ out,
                                                     int32_t* __restrict__ rows_done, int B,
                                                     const int* __restrict__ seq_off,
                                                     const int* __restrict__ rowmap) {
  const int M = hdr[kHdrM];
  if (rows_done) {
    for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
      int n = 0;
      for (int r = seq_off[b]; r < seq_off[b + 1]; ++r) n += rowmap[r] >= 0 ? 1 : 0;
      rows_done[b] = n;
    }
  }
  const int lane = threadIdx.x & (kWave - 1);
  for (int r = blockIdx.x * 4 + threadIdx.x / kWave; r < M; r += gridDim.x * 4)
    rms_row<NC, true>(a + int64_t(r) * d, gain, d, eps, out + int64_t(r) * d, lane);
}

// ------------------------------------------------------------------------------ 3/5/7/8. GEMM
enum { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_DOWN = 3, EPI_VPROJ = 4, EPI_QKV_ROPE = 5 };

struct GemmArgs {
  const uint16_t* A;    // [M, K] compacted rows (workspace)
  const uint16_t* W;    // [Nout, K] blocked (see gemm.h); SwiGLU: the fused gate/up [2 Nout, K]
  int K, Nout;          // Nout: W rows (SwiGLU: F)
  const int* hdr;
  const int* rowmap;
  int d;                // model width (row stride of x, caches, y, q, o, a)
  uint16_t* q;          // QKV: q rows
  uint16_t* kc;         // QKV: cache scatter targets
  uint16_t* vc;
  const uint16_t* x;    // RESID: residual rows (global, via rowmap)
  float* a;             // RESID: out; DOWN: residual in
  uint16_t* h;          // SWIGLU: out [M, F]
  uint16_t* y;          // DOWN: scatter target; VPROJ: V rows out (via the row map)
  float* part;          // split tail partial tiles [2 * grid, BM * BN] fp32
  int rope_dh;          // QKV: head_dim with rotary embedding (W_qkv from dcu_pack_qkv), else 0
  const float2* rope;   // QKV: [M, rope_dh / 2] (cos, sin) per row, written by the gather kernel
};

// QKV output columns n .. n+3 of compacted row m (global row grow; n a multiple of 4): Q to the q
// rows, K and V to the caches.
__device__ __forceinline__ void store_qkv(const GemmArgs& g, int m, int64_t grow, int n, float w0,
                                          float w1, float w2, float w3) {
  const int part = n / g.d, col = n - part * g.d;
  if (part != 0 && grow < 0) return;  // a skipped position: the caches keep their rows
  uint16_t* dst = part == 0 ? g.q + int64_t(m) * g.d : (part == 1 ? g.kc : g.vc) + grow * g.d;
  uint2 st;
  st.x = pack_bf2(w0, w1);
  st.y = pack_bf2(w2, w3);
  *reinterpret_cast<uint2*>(dst + col) = st;
}

// Rotary layout (dcu_pack_qkv): inside every Q and K head, packed columns 32k .. 32k+15 hold head
// dims 16k .. 16k+15 and packed columns 32k+16 .. 32k+31 hold dims h+16k .. h+16k+15 (h = dh/2), so
// an MFMA fragment and the one 16 columns to its right hold four whole rotation pairs in the same
// lane. x (packed columns n .. n+3, n in the first half of its 32-column group) pairs with y
// (n+16 .. n+19); cs0, cs1 are the (cos, sin) of the four pairs. Each half is written back as one
// 8-byte store at its own head dims (standard cache layout); V columns are stored as they are.
__device__ __forceinline__ float4 rope_cs(const GemmArgs& g, int m, int n, int which) {
  const int part = n / g.d, col = n - part * g.d;
  if (part == 2) return make_float4(0.f, 0.f, 0.f, 0.f);
  const int c = col & (g.rope_dh - 1);
  const int i = ((c >> 5) << 4) + (c & 15);  // head dim of the first pair
  return *reinterpret_cast<const float4*>(g.rope + int64_t(m) * (g.rope_dh >> 1) + i + 2 * which);
}
__device__ __forceinline__ void store_qkv_rope(const GemmArgs& g, int m, int64_t grow, int n,
                                               float4 x, float4 y, float4 cs0, float4 cs1) {
  const int part = n / g.d, col = n - part * g.d;
  if (part != 0 && grow < 0) return;  // a skipped position: the caches keep their rows
  uint16_t* dst = part == 0 ? g.q + int64_t(m) * g.d : (part == 1 ? g.kc : g.vc) + grow * g.d;
  uint2 a, b;
  if (part == 2) {
    a.x = pack_bf2(x.x, x.y); a.y = pack_bf2(x.z, x.w);
    b.x = pack_bf2(y.x, y.y); b.y = pack_bf2(y.z, y.w);
    *reinterpret_cast<uint2*>(dst + col) = a;
    *reinterpret_cast<uint2*>(dst + col + 16) = b;
    return;
  }
  const int dh = g.rope_dh, c = col & (dh - 1);
  const int i = ((c >> 5) << 4) + (c & 15);
  uint16_t* head = dst + (col - c);
  a.x = pack_bf2(x.x * cs0.x - y.x * cs0.y, x.y * cs0.z - y.y * cs0.w);
  a.y = pack_bf2(x.z * cs1.x - y.z * cs1.y, x.w * cs1.z - y.w * cs1.w);
  b.x = pack_bf2(y.x * cs0.x + x.x * cs0.y, y.y * cs0.z + x.y * cs0.w);
  b.y = pack_bf2(y.z * cs1.x + x.z * cs1.y, y.w * cs1.z + x.w * cs1.w);
  *reinterpret_cast<uint2*>(head + i) = a;
  *reinterpret_cast<uint2*>(head + i + (dh >> 1)) = b;
}

// Tail splitting: with a persistent grid of G workgroup slots and T output tiles, the last round holds
// T mod G tiles and leaves the other slots idle. Those tail tiles (all tiles when T < G) are cut
// along K into S segments whose fp32 partial tiles go to the workspace; k_gemm_fixup sums them in
// segment order and applies the epilogue (deterministic, no atomics). S depends on the row count, so
// it is chosen on the device; kernel and fixup evaluate the same function.
constexpr int kMaxSplitK = 16;  // few rows (batch 1) need many segments to fill the chip

struct SplitPlan {
  int full;  // tiles computed whole (ids 0 .. full-1)
  int rem;   // tail tiles (ids full .. full+rem-1), each in S segments
  int S;
  // CU-paired last round: workgroup j of an XCD shares its CU with workgroup j + G/16 (the
  // dispatcher fills every CU once before it places a second workgroup). After (full - G/2) / G
  // rounds of whole tiles, the first G/2 workgroups take the last G/2 whole tiles, one per CU, and
  // the second G/2 the rem * S <= G/2 segments of the other tiles, so every CU gets the same work
  bool paired;
};

enum SplitMode { kSplitTail = 0, kSplitStreaming = 1, kSplitFewTiles = 2 };

__host__ __device__ inline SplitPlan plan_split(int T, int G, int KT, int mode = kSplitTail) {
  SplitPlan p{T, 0, 1, false};
  if (T <= 0) return p;
  const bool streaming = mode == kSplitStreaming;
  // early-refill main loop: tiles run whole unless there are fewer tiles than CUs; between one and
  // two tiles per CU, one whole tile per CU and the rest cut in segments for the CUs' second slots
  if (mode == kSplitFewTiles && 2 * T >= G) {
    // the last round (T mod G tiles, or G when T is a multiple of G) decides: between one and two
    // tiles per CU, the CU-paired placement; otherwise whole tiles
    const int C = G / 2, last = T % G == 0 ? G : T % G, rem = last - C;
    if (rem <= 0 || rem >= C || (G & 15) != 0) return p;
    int S = C / rem;
    S = S < kMaxSplitK ? S : kMaxSplitK;
    while (S > 1 && KT / S < 8) --S;
    if (S > 1) p = SplitPlan{T - rem, rem, S, true};
    return p;
  }
  if (streaming) {
    // weight streaming (few rows): the time is the weight bytes over the bandwidth once enough
    // workgroups stream, so use the fewest segments that still keep the units within one round
    // (every segment adds a partial tile written and read back)
    int S = G / T;
    S = S < kMaxSplitK ? S : kMaxSplitK;
    while (S > 1 && KT / S < 8) --S;
    if (S > 1) p = SplitPlan{0, T, S, false};
    return p;
  }
  if (T < G) {
    // every tile: the S in [2, min(16, KT / 8, 2G / T)] minimising rounds / S (at most 2 rounds
    // of units), ties to the smaller S. rounds / S is 1 / S up to G / T and 2 / S above, so the
    // minimum is at the largest one-round S or at the largest S: two candidates in ascending order
    // (every workgroup of the GEMM and its fixup evaluates this at its start, so no loop)
    int smax = KT / 8 < kMaxSplitK ? KT / 8 : kMaxSplitK;
    smax = smax < 2 * G / T ? smax : 2 * G / T;
    const int Sa = smax < G / T ? smax : G / T;
    float best = 1.0f;
    for (int c = 0; c < 2; ++c) {
      const int S = c == 0 ? Sa : smax;
      if (S < 2 || (c == 1 && S == Sa)) continue;
      const float cost = float((T * S + G - 1) / G) / float(S);
      if (cost < best - 1e-6f) {
        best = cost;
        p.S = S;
      }
    }
    if (p.S > 1) p = SplitPlan{0, T, p.S, false};
    return p;
  }
  const int rem = T % G;
  if (rem == 0 || 2 * rem > G) return p;
  int S = G / rem;
  S = S < kMaxSplitK ? S : kMaxSplitK;
  while (S > 1 && KT / S < 8) --S;
  if (S > 1) p = SplitPlan{T - rem, rem, S, false};
  return p;
}

// Tile shape: 128x128 with 4 waves (64x64 each), two workgroups per CU. (A 256x256 tile with 8 waves
// is faster on the dense shape in isolation but exceeds the 256 registers per wave with the fused
// epilogues and spills.)
using CfgSmall = gemm::Cfg<128, 128, 64, 64, 2, 4>;
// Up to 64 rows (one or a few sequences) the projections stream their weights; a 64-row tile with
// three stages keeps twice the weight bytes in flight per CU (two K-tiles per workgroup, two
// workgroups per CU) for the same LDS budget.
using CfgSkinny = gemm::Cfg<64, 64, 32, 32, 4, 4>;
// When the caller's row bound is at most 64 (one sequence: budget plus window) the host launches a
// kernel of its own for the weight stream, one workgroup per CU with four stages: gate/up on
// 64 x 128 tiles (twice the weight rows per activation row fetched, 96 KB of LDS), the others on
// 64 x 64 tiles. Measured on the batch-1 shapes with cold weights, GEMM + split fixup, against the
// 64 x 64 tiles at two workgroups per CU: gate/up 48.9 -> 41.8 us (64 x 128), QKV 28.0 -> 26.5 (64 x
// 64, no K split, so no fixup), output 15.4 -> 11.7, down 28.1 -> 24.8; 64 x 128 tiles for the
// other three were slower (25.2, 14.1 and 26.2).
using CfgStream = gemm::Cfg<64, 128, 32, 64, 4, 4>;
template <int EPI>
using StreamCfg = typename std::conditional<EPI == EPI_SWIGLU, CfgStream, CfgSkinny>::type;
constexpr int kStreamSlots = 256;  // one workgroup per CU
static_assert(CfgStream::BM * CfgStream::BN * kStreamSlots <=
                  CfgSkinny::BM * CfgSkinny::BN * 2 * 256,
              "partial tiles of the streaming kernel fit the 64-row workspace");
constexpr int kGemmLdsChunks = CfgSmall::STAGES * CfgSmall::CHUNKS > CfgSkinny::STAGES * CfgSkinny::CHUNKS
                                   ? CfgSmall::STAGES * CfgSmall::CHUNKS
                                   : CfgSkinny::STAGES * CfgSkinny::CHUNKS;
static_assert(kGemmLdsChunks * 16 <= 80 * 1024, "two workgroups per CU");
static_assert(CfgSkinny::BM * CfgSkinny::BN <= CfgSmall::BM * CfgSmall::BN, "partial tile slots");
// the tile shape follows the device-side row count; kernel and fixup take the same decision
__device__ inline bool use_skinny(int M) { return M <= CfgSkinny::BM; }
// Main loop per projection. QKV, output and down (1-1.7 rounds of 512 tiles at ~1.1k rows) run the
// early-refill loop, whose DMAs have two K-tiles of latency, with their tiles whole: measured at
// batch 8, N = 1024, output 58.0 + 17.8 (split fixup) -> 60.4 + 6.8 us, down and QKV even.
// Gate/up runs it too up to two rounds of tiles, whole tiles with the CU-paired tail: closed loop
// (~500 rows, 1.5 rounds) 108.1 + 11.5 (split fixup) -> 105.9 + 6.7 us. At ~1.1k rows (3.4 rounds)
// it was even in time but fetched 754 instead of 584 MB per launch from beyond the L2 (the
// workgroups of an XCD drift further apart with two K-tiles in flight and share fewer activation
// and weight lines), and at M = 8192 it trails the two-stage loop by 13%; above two rounds gate/up
// keeps the two-stage loop and the tail split.
template <int EPI, class C>
constexpr bool early_refill() {
  return (EPI == EPI_QKV || EPI == EPI_QKV_ROPE || EPI == EPI_RESID || EPI == EPI_DOWN ||
          EPI == EPI_VPROJ) &&
         std::is_same<C, CfgSmall>::value;
}
template <int EPI, class C>
constexpr bool early_refill_few_rounds() {
  return EPI == EPI_SWIGLU && std::is_same<C, CfgSmall>::value;
}
constexpr int kEarlyRefillMaxRounds = 2;
template <int EPI, class C>
constexpr int split_mode() {
  return (std::is_same<C, CfgSkinny>::value || std::is_same<C, CfgStream>::value) ? kSplitStreaming
                                           : (early_refill<EPI, C>() ? kSplitFewTiles : kSplitTail);
}
// Gate/up: the early-refill loop (whole tiles, CU-paired tail) for T tiles on G workgroups up to
// two rounds, the two-stage loop with the tail split above. The GEMM and its fixup both decide here.
template <int EPI, class C>
__host__ __device__ constexpr bool gate_up_early_refill(int T, int G) {
  return early_refill_few_rounds<EPI, C>() && T <= kEarlyRefillMaxRounds * G;
}
template <int EPI, class C>
__host__ __device__ constexpr int split_mode_for(int T, int G) {
  return gate_up_early_refill<EPI, C>(T, G) ? kSplitFewTiles : split_mode<EPI, C>();
}

template <int EPI, class C>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, gemm::f32x4 (&acc)[C::FM][C::FN],
                                              int M, int m0, int n_t) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / C::WGN, wn = wid % C::WGN;
  const int cg = (lane >> 4) * 4;
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int m = m0 + wm * C::WM + fm * 16 + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int fn = 0; fn < C::FN / 2; ++fn) {
        const int j = n_t * (C::BN / 2) + wn * (C::WN / 2) + fn * 16 + cg;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = acc[fm][fn][i], up = acc[fm][fn + C::FN / 2][i];
          v[i] = gt / (1.0f + __expf(-gt)) * up;
        }
        uint2 st;
        st.x = pack_bf2(v[0], v[1]);
        st.y = pack_bf2(v[2], v[3]);
        *reinterpret_cast<uint2*>(g.h + int64_t(m) * g.Nout + j) = st;
      }
    }
  } else {
    // Every load of the epilogue (the row map, then the rotary table, the fp32 a or the residual
    // rows that depend on it) is issued before the first store, unconditionally, at addresses
    // clamped into the buffers (row M-1 for rows past M, the last column group for columns past
    // Nout, row 0 of x for a skipped position): loads and stores share one memory counter, so a load
    // issued after a store also waits for the store, and a load under a branch is waited for inside
    // that branch (a chain of round trips). Values read for rows or columns that are not stored are
    // never used.
    int grow[C::FM];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int m = m0 + wm * C::WM + fm * 16 + (lane & 15);
      grow[fm] = g.rowmap[m < M ? m : M - 1];
    }
    constexpr bool kF4 = EPI == EPI_QKV_ROPE || EPI == EPI_DOWN;
    float4 opnd[kF4 ? C::FM : 1][kF4 ? C::FN : 1];
    uint2 xres[EPI == EPI_RESID ? C::FM : 1][EPI == EPI_RESID ? C::FN : 1];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int m = m0 + wm * C::WM + fm * 16 + (lane & 15);
      const int mc = m < M ? m : M - 1;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        if constexpr (EPI == EPI_QKV_ROPE) {
          // (cos, sin) of the pairs of fragment pair fn/2 (two float4 each); every column index
          // maps into the row's table
          const int n = n_t * C::BN + wn * C::WN + (fn & ~1) * 16 + cg;
          opnd[fm][fn] = rope_cs(g, mc, n, fn & 1);
        } else if constexpr (EPI == EPI_DOWN) {
          int n = n_t * C::BN + wn * C::WN + fn * 16 + cg;
          n = n < g.Nout ? n : g.Nout - 4;
          opnd[fm][fn] = *reinterpret_cast<const float4*>(g.a + int64_t(mc) * g.d + n);
        } else if constexpr (EPI == EPI_RESID) {
          int n = n_t * C::BN + wn * C::WN + fn * 16 + cg;
          n = n < g.Nout ? n : g.Nout - 4;
          const int64_t xr = grow[fm] >= 0 ? int64_t(grow[fm]) : 0;
          xres[fm][fn] = *reinterpret_cast<const uint2*>(g.x + xr * g.d + n);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int m = m0 + wm * C::WM + fm * 16 + (lane & 15);
      if (m >= M) continue;
      const int64_t gr = int64_t(grow[fm]);
      if constexpr (EPI == EPI_QKV_ROPE) {
        static_assert(C::FN % 2 == 0, "fragment pairs");
#pragma unroll
        for (int fp = 0; fp < C::FN; fp += 2) {
          const int n = n_t * C::BN + wn * C::WN + fp * 16 + cg;
          if (n >= g.Nout) continue;
          const gemm::f32x4 x = acc[fm][fp], y = acc[fm][fp + 1];
          store_qkv_rope(g, m, gr, n, make_float4(x[0], x[1], x[2], x[3]),
                         make_float4(y[0], y[1], y[2], y[3]), opnd[fm][fp], opnd[fm][fp + 1]);
        }
      } else {
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          const int n = n_t * C::BN + wn * C::WN + fn * 16 + cg;
          if (n >= g.Nout) continue;
          const gemm::f32x4 v = acc[fm][fn];
          if constexpr (EPI == EPI_QKV) {
            store_qkv(g, m, gr, n, v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_DOWN) {
            if (gr < 0) continue;  // a skipped position: the output keeps its row
            const float4 p = opnd[fm][fn];
            uint2 st;
            st.x = pack_bf2(p.x + v[0], p.y + v[1]);
            st.y = pack_bf2(p.z + v[2], p.w + v[3]);
            *reinterpret_cast<uint2*>(g.y + gr * g.d + n) = st;
          } else if constexpr (EPI == EPI_RESID) {
            // a skipped position has no input row: its (unused) residual is taken as 0
            const uint2 xr = gr >= 0 ? xres[fm][fn] : make_uint2(0u, 0u);
            float4 o;
            o.x = bf_lo(xr.x) + v[0];
            o.y = bf_hi(xr.x) + v[1];
            o.z = bf_lo(xr.y) + v[2];
            o.w = bf_hi(xr.y) + v[3];
            *reinterpret_cast<float4*>(g.a + int64_t(m) * g.d + n) = o;
          } else {  // EPI_VPROJ
            if (gr < 0) continue;
            uint2 st;
            st.x = pack_bf2(v[0], v[1]);
            st.y = pack_bf2(v[2], v[3]);
            *reinterpret_cast<uint2*>(g.y + gr * g.d + n) = st;
          }
        }
      }
    }
  }
}

template <int EPI, class C>
__device__ __forceinline__ void gemm_body(const GemmArgs& g, int M, u32x4* smem) {
  static_assert(C::THREADS == 256, "one launch shape");
  u32x4* b0 = smem;
  u32x4* b1 = smem + C::CHUNKS;
  u32x4* b2 = smem + (C::STAGES > 2 ? 2 : 0) * C::CHUNKS;
  u32x4* b3 = smem + (C::STAGES > 3 ? 3 : 0) * C::CHUNKS;
  using Blocks = typename std::conditional<EPI == EPI_SWIGLU, gemm::GateUpBlocks<C::WN>,
                                           gemm::PlainBlocks>::type;
  Blocks wr;
  if constexpr (EPI == EPI_SWIGLU)
    wr = Blocks{g.W, g.Nout, g.K / C::BK};
  else
    wr = Blocks{g.W, g.Nout, g.K / C::BK};
  const int MT = (M + C::BM - 1) / C::BM;
  const int NT = wr.template tiles<C::BN>();
  const int KT = g.K / C::BK;
  const SplitPlan sp = plan_split(MT * NT, gridDim.x, KT, split_mode_for<EPI, C>(MT * NT, gridDim.x));
  const int units = sp.full + sp.rem * sp.S;
  int lin, zero;
  for (int round = 0;; ++round) {
    if (sp.paired) {
      const int f0 = sp.full - (gridDim.x >> 1);  // tiles of the full rounds
      if (round * int(gridDim.x) < f0) {
        gemm::next_tile(round, f0, f0, &lin, &zero);
      } else {
        if (round * int(gridDim.x) > f0) break;
        const int per = gridDim.x >> 4, x = blockIdx.x & 7, j = blockIdx.x >> 3;
        if (j < per) {
          lin = f0 + x * per + j;  // whole tile
        } else {
          const int v = x * per + (j - per);
          if (v >= sp.rem * sp.S) break;
          lin = sp.full + v;  // segment v % S of tail tile v / S
        }
      }
    } else if (!gemm::next_tile(round, units, units, &lin, &zero)) {
      break;
    }
    int tile, s = 0, kt0 = 0, kt1 = KT;
    if (lin < sp.full) {
      tile = lin;
    } else {
      const int v = lin - sp.full;
      tile = sp.full + v / sp.S;
      s = v % sp.S;
      kt0 = KT * s / sp.S;
      kt1 = KT * (s + 1) / sp.S;
    }
    const int m_t = tile % MT, n_t = tile / MT;  // consecutive tiles share the weight tile
    gemm::f32x4 acc[C::FM][C::FN];
    if constexpr (early_refill<EPI, C>()) {
      gemm::tile_mainloop_er<C>(acc, g.A, M, g.K, m_t * C::BM, n_t, wr, b0, b1, kt0, kt1);
    } else if constexpr (early_refill_few_rounds<EPI, C>()) {
      if (gate_up_early_refill<EPI, C>(MT * NT, gridDim.x))
        gemm::tile_mainloop_er<C>(acc, g.A, M, g.K, m_t * C::BM, n_t, wr, b0, b1, kt0, kt1);
      else
        gemm::tile_mainloop<C>(acc, g.A, M, g.K, m_t * C::BM, n_t, wr, b0, b1, b2, b3, kt0, kt1);
    } else {
      gemm::tile_mainloop<C>(acc, g.A, M, g.K, m_t * C::BM, n_t, wr, b0, b1, b2, b3, kt0, kt1);
    }
    if (lin < sp.full) {
      gemm_epilogue<EPI, C>(g, acc, M, m_t * C::BM, n_t);
    } else {
      // tile-local partial: [BM rows][BN weight rows of the tile]
      const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
      const int wm = wid / C::WGN, wn = wid % C::WGN;
      float* pt = g.part + int64_t(lin - sp.full) * (C::BM * C::BN);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int r = wm * C::WM + fm * 16 + (lane & 15);
        if (m_t * C::BM + r >= M) continue;  // rows past M are never read back
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
          const int c = wn * C::WN + fn * 16 + (lane >> 4) * 4;
          *reinterpret_cast<float4*>(pt + r * C::BN + c) =
              make_float4(acc[fm][fn][0], acc[fm][fn][1], acc[fm][fn][2], acc[fm][fn][3]);
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g) {
  __shared__ u32x4 smem[kGemmLdsChunks];
  const int M = g.hdr[kHdrM];
  if (M <= 0) return;
  if (use_skinny(M))
    gemm_body<EPI, CfgSkinny>(g, M, smem);
  else
    gemm_body<EPI, CfgSmall>(g, M, smem);
}

// The weight-streaming projection for a row capacity of at most 64 (the device row count is then
// at most 64 as well), one workgroup per CU
template <int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_stream(GemmArgs g) {
  __shared__ u32x4 smem[StreamCfg<EPI>::STAGES * StreamCfg<EPI>::CHUNKS];
  const int M = g.hdr[kHdrM];
  if (M <= 0) return;
  gemm_body<EPI, StreamCfg<EPI>>(g, M, smem);
}

// ------------------------------------------------------------------------------ 1+3 fused (few rows)
// For a row capacity of at most 64 the gather and the RMSNorm run inside the QKV weight stream.
// Every workgroup evaluates the row offsets and the row map of the <= 64 selected rows itself
// (workgroup 0 publishes them with the attention tables for the later kernels), its DMA sources
// are the selected rows of x themselves, and every activation fragment is multiplied by the
// RMSNorm gains right after its LDS read while the squares of the raw values are summed; the
// finished tile row is then scaled by the row's 1/sqrt(mean(x^2) + eps):
//   RMSNorm(x; g) W^T = s * ((x * g) W^T),  s = 1 / sqrt(mean(x^2) + eps) per row
// (x * g rounded to bf16 for the MFMA, where the two-launch form rounds x * s * g). The rotary
// (cos, sin) table of the workgroup's rows is built in LDS. Tiles run whole (no K split), one
// workgroup per CU. This removes the gather launch and the normalised rows' round trip through
// memory.
constexpr int kFusedMaxD = 8192;      // model width whose gains fit the LDS copy
constexpr int kFusedMaxRopeDh = 128;  // rotary head_dim whose (cos, sin) table fits LDS

template <int EPI>
__global__ __launch_bounds__(256, 1) void k_qkv_fused(GemmArgs g, Ptrs P,
                                                      const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ sel_idx,
                                                      const int32_t* __restrict__ sel_count,
                                                      int B, int N, int M_cap,
                                                      const uint16_t* __restrict__ gain,
                                                      float eps) {
  using C = CfgSkinny;
  static_assert(C::BM == 64 && C::BK == 64, "one row tile of 64");
  __shared__ u32x4 smem[C::STAGES * C::CHUNKS];
  __shared__ int off[kMaxSeqs + 1];
  __shared__ int scan_lds[17];
  __shared__ int s_row[C::BM], s_pos[C::BM];
  __shared__ u32x4 s_gain[kFusedMaxD / 8];
  __shared__ float2 s_rope[EPI == EPI_QKV_ROPE ? C::BM * (kFusedMaxRopeDh / 2) : 1];
  const int d = g.d;
  // one sequence: thread r's list entry is loaded together with the count (r < M_cap <= N)
  const int t = threadIdx.x;
  const int pre = (B == 1 && sel_idx && t < M_cap && t < N) ? sel_idx[t] : 0;
  // the gains next: their loads overlap the plan below
  for (int i = t; i < d / 8; i += blockDim.x) s_gain[i] = reinterpret_cast<const u32x4*>(gain)[i];
  row_offsets(sel_count, B, N, M_cap, off, scan_lds);
  const int M = off[B];
  if (blockIdx.x == 0) publish_plan(off, B, P);
  if (M <= 0) return;
  if (t < M) {
    int pos, grow;
    if (B == 1) {
      pos = sel_idx ? pre : t;
      pos = pos >= 0 && pos < N ? pos : -1;
      grow = pos;
    } else {
      grow = row_of(off, B, N, sel_idx, t, &pos);
    }
    s_row[t] = grow;
    s_pos[t] = pos;
    if (blockIdx.x == 0) P.rowmap[t] = grow;
  }
  __syncthreads();
  if constexpr (EPI == EPI_QKV_ROPE) {
    const int hp = g.rope_dh / 2;
    for (int e = threadIdx.x; e < M * hp; e += blockDim.x) {
      const int r = e / hp, i = e - r * hp;
      const int pos = s_pos[r];
      float sn = 0.0f, cs = 1.0f;
      if (pos >= 0) sincosf(rope_angle(float(pos), i, g.rope_dh, P.rope_l2t), &sn, &cs);
      s_rope[e] = make_float2(cs, sn);
    }
  }
  __syncthreads();
  GemmArgs lg = g;
  lg.rowmap = s_row;
  lg.rope = s_rope;
  const gemm::PlainBlocks wr{g.W, g.Nout, g.K / C::BK};
  const int NT = wr.template tiles<C::BN>();
  for (int n_t = blockIdx.x; n_t < NT; n_t += gridDim.x) {
    const uint16_t* src[C::NQ];
    gemm::dma_sources_rows<C>(
        src,
        [&](int row) {
          const int grow = s_row[row < M ? row : M - 1];
          return x + int64_t(grow >= 0 ? grow : 0) * d;  // a skipped position reads row 0 (unused)
        },
        n_t, wr, 0);
    float ss[C::FM];
#pragma unroll
    for (int f = 0; f < C::FM; ++f) ss[f] = 0.0f;
    // x * g for the MFMA, sum of x^2 of the lane's row (columns k .. k+7)
    auto gain_sumsq = [&](int f, int k, u32x4& fx) {
      const u32x4 gg = s_gain[k >> 3];
      const uint32_t xw[4] = {fx.x, fx.y, fx.z, fx.w};
      const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
      uint32_t o[4];
      float sq = ss[f];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 xp = __builtin_bit_cast(bf16x2, xw[j]);
        sq = __builtin_amdgcn_fdot2_f32_bf16(xp, xp, sq, false);  // + x0^2 + x1^2
        o[j] = pack_bf2(bf_lo(xw[j]) * bf_lo(gw[j]), bf_hi(xw[j]) * bf_hi(gw[j]));
      }
      ss[f] = sq;
      fx = u32x4{o[0], o[1], o[2], o[3]};
    };
    gemm::f32x4 acc[C::FM][C::FN];
    gemm::tile_mainloop_deep<C>(acc, src, smem, 0, g.K / C::BK, gain_sumsq);
    // the four lanes of a row (lane >> 4) hold its four column chunks of every K-tile
#pragma unroll
    for (int f = 0; f < C::FM; ++f) {
      float t = ss[f];
      t += __shfl_xor(t, 16, kWave);
      t += __shfl_xor(t, 32, kWave);
      const float scale = 1.0f / sqrtf(t / float(d) + eps);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[f][j] *= scale;
    }
    gemm_epilogue<EPI, C>(lg, acc, M, 0, n_t);
  }
}

// The output projection's split tiles finished together with the RMSNorm before the FFN for a row
// capacity of at most 64: one workgroup per row, each thread holding PER 8-column groups. A group
// comes from a (a whole tile) or is the residual plus the fixed-order sum of its tile's fp32 pieces
// (k_gemm_fixup's order); the pieces of all the thread's groups are loaded in rounds of four, the
// first round together with the residual and the gains. The sum of squares is reduced over the
// workgroup in a fixed order. With rows_done, also the per-sequence count of recomputed rows.
// the output projection's split plan for M rows on `slots` workgroups (as k_gemm made it)
template <class C>
__device__ __forceinline__ SplitPlan oproj_plan(const GemmArgs& g, int M, int slots) {
  const int MT = (M + C::BM - 1) / C::BM;
  const int NT = (g.Nout + C::BN - 1) / C::BN;
  return plan_split(MT * NT, slots, g.K / C::BK, split_mode_for<EPI_RESID, C>(MT * NT, slots));
}

template <int PER, class C>
__device__ __forceinline__ void resid_rmsnorm_row_body(const GemmArgs& g, int M,
                                                       const SplitPlan& sp,
                                                       const uint16_t* __restrict__ gain, float eps,
                                                       uint16_t* __restrict__ out, float* red) {
  const int d = g.d, groups = d / 8;
  const int MT = (M + C::BM - 1) / C::BM;
  constexpr int kTile = C::BM * C::BN;
  constexpr int kRound = 4;
  const int t = threadIdx.x, wid = t / kWave;
  for (int r = blockIdx.x; r < M; r += gridDim.x) {
    const int m_t = r / C::BM, rl = r - m_t * C::BM;
    const int64_t grow = int64_t(g.rowmap[r]);
    float* arow = g.a + int64_t(r) * d;
    float4 lo[PER], hi[PER];
    uint4 xr[PER], gg[PER];
    bool split[PER];
    const float* p0[PER];
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int gi = t + c * 256;
      split[c] = false;
      p0[c] = nullptr;
      lo[c] = hi[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      xr[c] = gg[c] = make_uint4(0u, 0u, 0u, 0u);
      if (gi >= groups) continue;
      const int col = gi * 8, n_t = col / C::BN;
      gg[c] = reinterpret_cast<const uint4*>(gain)[gi];
      if (n_t * MT + m_t < sp.full) {
        lo[c] = *reinterpret_cast<const float4*>(arow + col);
        hi[c] = *reinterpret_cast<const float4*>(arow + col + 4);
      } else {
        split[c] = true;
        p0[c] = g.part + int64_t(n_t * MT + m_t - sp.full) * sp.S * kTile + rl * C::BN +
                (col - n_t * C::BN);
        if (grow >= 0) xr[c] = *reinterpret_cast<const uint4*>(g.x + grow * d + col);
      }
    }
    for (int s0 = 0; s0 < sp.S; s0 += kRound) {
      float4 q0[PER][kRound], q1[PER][kRound];
#pragma unroll
      for (int c = 0; c < PER; ++c)
#pragma unroll
        for (int j = 0; j < kRound; ++j)
          if (split[c] && s0 + j < sp.S) {
            const float* q = p0[c] + int64_t(s0 + j) * kTile;
            q0[c][j] = *reinterpret_cast<const float4*>(q);
            q1[c][j] = *reinterpret_cast<const float4*>(q + 4);
          }
#pragma unroll
      for (int c = 0; c < PER; ++c)
#pragma unroll
        for (int j = 0; j < kRound; ++j)
          if (split[c] && s0 + j < sp.S) {
            if (s0 + j == 0) {
              lo[c] = q0[c][j];
              hi[c] = q1[c][j];
            } else {
              lo[c].x += q0[c][j].x; lo[c].y += q0[c][j].y; lo[c].z += q0[c][j].z; lo[c].w += q0[c][j].w;
              hi[c].x += q1[c][j].x; hi[c].y += q1[c][j].y; hi[c].z += q1[c][j].z; hi[c].w += q1[c][j].w;
            }
          }
    }
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      if (split[c]) {
        const int col = (t + c * 256) * 8;
        lo[c] = make_float4(bf_lo(xr[c].x) + lo[c].x, bf_hi(xr[c].x) + lo[c].y,
                            bf_lo(xr[c].y) + lo[c].z, bf_hi(xr[c].y) + lo[c].w);
        hi[c] = make_float4(bf_lo(xr[c].z) + hi[c].x, bf_hi(xr[c].z) + hi[c].y,
                            bf_lo(xr[c].w) + hi[c].z, bf_hi(xr[c].w) + hi[c].w);
        *reinterpret_cast<float4*>(arow + col) = lo[c];
        *reinterpret_cast<float4*>(arow + col + 4) = hi[c];
      }
      const float v[8] = {lo[c].x, lo[c].y, lo[c].z, lo[c].w, hi[c].x, hi[c].y, hi[c].z, hi[c].w};
#pragma unroll
      for (int k = 0; k < 8; k += 2) ss += v[k] * v[k] + v[k + 1] * v[k + 1];
    }
    ss = wave_sum(ss);
    if ((t & (kWave - 1)) == 0) red[wid] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float scale = 1.0f / sqrtf(tot / float(d) + eps);
    uint16_t* orow = out + int64_t(r) * d;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int gi = t + c * 256;
      if (gi >= groups) continue;
      uint4 o;
      o.x = pack_bf2(lo[c].x * scale * bf_lo(gg[c].x), lo[c].y * scale * bf_hi(gg[c].x));
      o.y = pack_bf2(lo[c].z * scale * bf_lo(gg[c].y), lo[c].w * scale * bf_hi(gg[c].y));
      o.z = pack_bf2(hi[c].x * scale * bf_lo(gg[c].z), hi[c].y * scale * bf_hi(gg[c].z));
      o.w = pack_bf2(hi[c].z * scale * bf_lo(gg[c].w), hi[c].w * scale * bf_hi(gg[c].w));
      reinterpret_cast<uint4*>(orow)[gi] = o;
    }
    __syncthreads();  // red is reused by the next row
  }
}

// slots: the output projection's grid (kStreamSlots for the weight-streaming kernel, else the
// persistent grid, whose tile shape follows the device row count as in k_gemm)
template <int PER>
__global__ __launch_bounds__(256) void k_resid_rmsnorm_row(GemmArgs g, int slots,
                                                           const uint16_t* __restrict__ gain,
                                                           float eps, uint16_t* __restrict__ out,
                                                           int32_t* __restrict__ rows_done, int B,
                                                           const int* __restrict__ seq_off) {
  __shared__ float red[4];
  const int M = g.hdr[kHdrM];
  if (rows_done && blockIdx.x == 0) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      int n = 0;
      for (int r = seq_off[b]; r < seq_off[b + 1]; ++r) n += g.rowmap[r] >= 0 ? 1 : 0;
      rows_done[b] = n;
    }
  }
  if (M <= 0) return;
  if (slots == kStreamSlots) {
    using C = StreamCfg<EPI_RESID>;
    resid_rmsnorm_row_body<PER, C>(g, M, oproj_plan<C>(g, M, slots), gain, eps, out, red);
  } else if (use_skinny(M)) {
    resid_rmsnorm_row_body<PER, CfgSkinny>(g, M, oproj_plan<CfgSkinny>(g, M, slots), gain, eps,
                                           out, red);
  } else {
    resid_rmsnorm_row_body<PER, CfgSmall>(g, M, oproj_plan<CfgSmall>(g, M, slots), gain, eps, out,
                                          red);
  }
}

// Sum of a split tail tile's partials in segment order, then the tile's epilogue; 4 columns per
// thread and item, kFixupU items per thread and round, with kFixupChunk partials of those items
// loaded before any is added (memory-level parallelism). Exits at once when the GEMM did not split.
constexpr int kFixupU = 1;
constexpr int kFixupChunk = 8;

template <int EPI, class C>
__device__ __forceinline__ void fixup_body(const GemmArgs& g, int M, int slots) {
  const int MT = (M + C::BM - 1) / C::BM;
  const int NT = EPI == EPI_SWIGLU ? g.Nout / (C::BN / 2) : (g.Nout + C::BN - 1) / C::BN;
  const SplitPlan sp = plan_split(MT * NT, slots, g.K / C::BK, split_mode_for<EPI, C>(MT * NT, slots));
  if (sp.rem == 0) return;
  // SwiGLU: an item is an output column group from its gate and up columns; rotary QKV: an item is
  // a column group of a 32-column group's first half together with its partner 16 columns on
  constexpr bool kPair = EPI == EPI_SWIGLU || EPI == EPI_QKV_ROPE;
  constexpr int OUTC = kPair ? C::BN / 2 : C::BN;  // items (x 4 columns) per tile row
  constexpr int Q = C::BM * OUTC / 4;              // float4 groups per tile
  constexpr int NV = kPair ? 2 : 1;                // float4 per item and partial
  const int64_t total = int64_t(sp.rem) * Q;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i0 < total;
       i0 += stride * kFixupU) {
    float4 v[kFixupU][NV];
    int m_u[kFixupU], col_u[kFixupU], nt_u[kFixupU], cols_u[kFixupU][NV];
    const float* pt_u[kFixupU];
    bool ok[kFixupU];
#pragma unroll
    for (int u = 0; u < kFixupU; ++u) {
      const int64_t i = i0 + u * stride;
      const int tt = int(i / Q), q = int(i % Q);
      const int r = q / (OUTC / 4), c4 = (q % (OUTC / 4)) * 4;
      const int tile = sp.full + tt;
      const int m_t = tile % MT, n_t = tile / MT;
      const int m = m_t * C::BM + r;
      int n = n_t * C::BN + c4;
      ok[u] = i < total && m < M && (EPI == EPI_SWIGLU || n < g.Nout);
      m_u[u] = m;
      col_u[u] = c4;
      nt_u[u] = n_t;
      // partial columns of this item: SwiGLU reads the gate and the up column of the same output
      int cols[NV];
      if constexpr (EPI == EPI_SWIGLU) {
        const int wn = c4 / (C::WN / 2), w = c4 % (C::WN / 2);
        cols[0] = wn * C::WN + w;
        cols[NV - 1] = cols[0] + C::WN / 2;
      } else if constexpr (EPI == EPI_QKV_ROPE) {
        cols[0] = (c4 >> 4) * 32 + (c4 & 15);
        cols[NV - 1] = cols[0] + 16;
        n = n_t * C::BN + cols[0];
        ok[u] = i < total && m < M && n < g.Nout;
      } else {
        cols[0] = c4;
      }
      pt_u[u] = g.part + int64_t(ok[u] ? tt : 0) * sp.S * (C::BM * C::BN) + r * C::BN;
      cols_u[u][0] = cols[0];
      cols_u[u][NV - 1] = cols[NV - 1];
    }
    // partials in segment order, kFixupChunk segments of every item loaded before they are added
    for (int s0 = 0; s0 < sp.S; s0 += kFixupChunk) {
      float4 p[kFixupU][kFixupChunk][NV];
#pragma unroll
      for (int u = 0; u < kFixupU; ++u)
#pragma unroll
        for (int j = 0; j < kFixupChunk; ++j)
#pragma unroll
          for (int e = 0; e < NV; ++e)
            if (ok[u] && s0 + j < sp.S)
              p[u][j][e] = *reinterpret_cast<const float4*>(
                  pt_u[u] + int64_t(s0 + j) * (C::BM * C::BN) + cols_u[u][e]);
#pragma unroll
      for (int u = 0; u < kFixupU; ++u)
#pragma unroll
        for (int j = 0; j < kFixupChunk; ++j)
#pragma unroll
          for (int e = 0; e < NV; ++e)
            if (s0 + j < sp.S) {
              if (s0 + j == 0) {
                v[u][e] = p[u][j][e];
              } else {
                v[u][e].x += p[u][j][e].x; v[u][e].y += p[u][j][e].y;
                v[u][e].z += p[u][j][e].z; v[u][e].w += p[u][j][e].w;
              }
            }
    }
#pragma unroll
    for (int u = 0; u < kFixupU; ++u) {
      if (!ok[u]) continue;
      const int m = m_u[u], c4 = col_u[u], n_t = nt_u[u];
      if constexpr (EPI == EPI_SWIGLU) {
        const float4 gt = v[u][0], up = v[u][NV - 1];
        const int j = n_t * (C::BN / 2) + c4;
        uint2 st;
        st.x = pack_bf2(gt.x / (1.0f + __expf(-gt.x)) * up.x, gt.y / (1.0f + __expf(-gt.y)) * up.y);
        st.y = pack_bf2(gt.z / (1.0f + __expf(-gt.z)) * up.z, gt.w / (1.0f + __expf(-gt.w)) * up.w);
        *reinterpret_cast<uint2*>(g.h + int64_t(m) * g.Nout + j) = st;
      } else {
        const float4 w = v[u][0];
        const int n = n_t * C::BN + c4;
        const int64_t grow = int64_t(g.rowmap[m]);
        if constexpr (EPI == EPI_QKV) {
          store_qkv(g, m, grow, n, w.x, w.y, w.z, w.w);
        } else if constexpr (EPI == EPI_QKV_ROPE) {
          const int np = n_t * C::BN + cols_u[u][0];
          store_qkv_rope(g, m, grow, np, w, v[u][NV - 1], rope_cs(g, m, np, 0),
                         rope_cs(g, m, np, 1));
        } else if constexpr (EPI == EPI_RESID) {
          const uint2 xr = grow >= 0 ? *reinterpret_cast<const uint2*>(g.x + grow * g.d + n)
                                     : make_uint2(0u, 0u);
          *reinterpret_cast<float4*>(g.a + int64_t(m) * g.d + n) =
              make_float4(bf_lo(xr.x) + w.x, bf_hi(xr.x) + w.y, bf_lo(xr.y) + w.z, bf_hi(xr.y) + w.w);
        } else if constexpr (EPI == EPI_VPROJ) {
          if (grow < 0) continue;
          uint2 st;
          st.x = pack_bf2(w.x, w.y);
          st.y = pack_bf2(w.z, w.w);
          *reinterpret_cast<uint2*>(g.y + grow * g.d + n) = st;
        } else {  // EPI_DOWN
          if (grow < 0) continue;  // a skipped position: the output keeps its row
          const float4 ar = *reinterpret_cast<const float4*>(g.a + int64_t(m) * g.d + n);
          uint2 st;
          st.x = pack_bf2(ar.x + w.x, ar.y + w.y);
          st.y = pack_bf2(ar.z + w.z, ar.w + w.w);
          *reinterpret_cast<uint2*>(g.y + grow * g.d + n) = st;
        }
      }
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_fixup(GemmArgs g, int slots) {
  const int M = g.hdr[kHdrM];
  if (M <= 0) return;
  if (slots == kStreamSlots)
    fixup_body<EPI, StreamCfg<EPI>>(g, M, slots);
  else if (use_skinny(M))
    fixup_body<EPI, CfgSkinny>(g, M, slots);
  else
    fixup_body<EPI, CfgSmall>(g, M, slots);
}

// The output projection's split tiles finished together with the RMSNorm before the FFN: one wave
// per row r takes each of its lane's 8-column groups either from a (a whole tile, stored by the
// GEMM's epilogue) or as the fixed-order sum of the tile's fp32 pieces plus the residual x (a split
// tile; the same order and residual as k_gemm_fixup's), stores that to a (the down projection's
// residual), then normalises the row held in registers -> an (bf16). This replaces the output
// projection's fixup launch. With rows_done, also the per-sequence count of recomputed rows.
template <int NC, class C>
__device__ __forceinline__ void resid_rms_rows(const GemmArgs& g, int M, const SplitPlan& sp,
                                               const uint16_t* __restrict__ gain, float eps,
                                               uint16_t* __restrict__ out) {
  const int d = g.d, groups = d / 8;
  const int MT = (M + C::BM - 1) / C::BM;
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kTile = C::BM * C::BN;
  for (int r = blockIdx.x * 4 + threadIdx.x / kWave; r < M; r += gridDim.x * 4) {
    const int m_t = r / C::BM, rl = r - m_t * C::BM;
    const int64_t grow = int64_t(g.rowmap[r]);
    float* arow = g.a + int64_t(r) * d;
    float4 lo[NC], hi[NC];
    uint4 xr[NC];
    bool split[NC];
    // piece 0 of a split group's 8 columns; piece s is kTile floats further
    auto piece0 = [&](int c) {
      const int col = (lane + c * kWave) * 8, n_t = col / C::BN;
      return g.part + int64_t(n_t * MT + m_t - sp.full) * sp.S * kTile + rl * C::BN +
             (col - n_t * C::BN);
    };
    // first round: a (whole tiles) or piece 0 (split tiles), the residual and the gains of every
    // group of the lane, all in flight together
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int gi = lane + c * kWave;
      split[c] = false;
      lo[c] = hi[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      xr[c] = make_uint4(0u, 0u, 0u, 0u);
      if (gi >= groups) continue;
      const int col = gi * 8, n_t = col / C::BN;
      if (n_t * MT + m_t < sp.full) {
        lo[c] = *reinterpret_cast<const float4*>(arow + col);
        hi[c] = *reinterpret_cast<const float4*>(arow + col + 4);
      } else {
        split[c] = true;
        const float* p0 = piece0(c);
        lo[c] = *reinterpret_cast<const float4*>(p0);
        hi[c] = *reinterpret_cast<const float4*>(p0 + 4);
        if (grow >= 0) xr[c] = *reinterpret_cast<const uint4*>(g.x + grow * d + col);
      }
    }
    // pieces 1 .. S-1 in order, each round loading the piece of every split group before adding
    for (int sg = 1; sg < sp.S; ++sg) {
      float4 t0[NC], t1[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (!split[c]) continue;
        const float* q = piece0(c) + int64_t(sg) * kTile;
        t0[c] = *reinterpret_cast<const float4*>(q);
        t1[c] = *reinterpret_cast<const float4*>(q + 4);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (!split[c]) continue;
        lo[c].x += t0[c].x; lo[c].y += t0[c].y; lo[c].z += t0[c].z; lo[c].w += t0[c].w;
        hi[c].x += t1[c].x; hi[c].y += t1[c].y; hi[c].z += t1[c].z; hi[c].w += t1[c].w;
      }
    }
    // a = residual + sum of the pieces (k_gemm_fixup's order), stored for the down projection
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!split[c]) continue;
      const int col = (lane + c * kWave) * 8;
      lo[c] = make_float4(bf_lo(xr[c].x) + lo[c].x, bf_hi(xr[c].x) + lo[c].y,
                          bf_lo(xr[c].y) + lo[c].z, bf_hi(xr[c].y) + lo[c].w);
      hi[c] = make_float4(bf_lo(xr[c].z) + hi[c].x, bf_hi(xr[c].z) + hi[c].y,
                          bf_lo(xr[c].w) + hi[c].z, bf_hi(xr[c].w) + hi[c].w);
      *reinterpret_cast<float4*>(arow + col) = lo[c];
      *reinterpret_cast<float4*>(arow + col + 4) = hi[c];
    }
    // the RMSNorm of rms_row, same per-lane order (the gains are loaded here, with the reduction)
    uint4 gg[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int gi = lane + c * kWave;
      gg[c] = gi < groups ? reinterpret_cast<const uint4*>(gain)[gi] : make_uint4(0u, 0u, 0u, 0u);
    }
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float v[8] = {lo[c].x, lo[c].y, lo[c].z, lo[c].w, hi[c].x, hi[c].y, hi[c].z, hi[c].w};
#pragma unroll
      for (int k = 0; k < 8; k += 2) ss += v[k] * v[k] + v[k + 1] * v[k + 1];
    }
    ss = wave_sum(ss);
    const float scale = 1.0f / sqrtf(ss / float(d) + eps);
    uint16_t* orow = out + int64_t(r) * d;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int gi = lane + c * kWave;
      if (gi >= groups) continue;
      uint4 o;
      o.x = pack_bf2(lo[c].x * scale * bf_lo(gg[c].x), lo[c].y * scale * bf_hi(gg[c].x));
      o.y = pack_bf2(lo[c].z * scale * bf_lo(gg[c].y), lo[c].w * scale * bf_hi(gg[c].y));
      o.z = pack_bf2(hi[c].x * scale * bf_lo(gg[c].z), hi[c].y * scale * bf_hi(gg[c].z));
      o.w = pack_bf2(hi[c].z * scale * bf_lo(gg[c].w), hi[c].w * scale * bf_hi(gg[c].w));
      reinterpret_cast<uint4*>(orow)[gi] = o;
    }
  }
}

template <int NC>
__global__ __launch_bounds__(256) void k_resid_rmsnorm(GemmArgs g, int slots,
                                                       const uint16_t* __restrict__ gain, float eps,
                                                       uint16_t* __restrict__ out,
                                                       int32_t* __restrict__ rows_done, int B,
                                                       const int* __restrict__ seq_off) {
  const int M = g.hdr[kHdrM];
  if (rows_done) {
    for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
      int n = 0;
      for (int r = seq_off[b]; r < seq_off[b + 1]; ++r) n += g.rowmap[r] >= 0 ? 1 : 0;
      rows_done[b] = n;
    }
  }
  if (M <= 0) return;
  // When the output projection split every tile (fewer tiles than workgroup slots: each group of a
  // row is a sum of pieces), a workgroup per row (grid-stride over the rows) keeps four times more
  // pieces in flight than a wave per row: closed-loop step (~500 rows, 4 pieces) 21.6 -> 15.9 us
  // per layer. With whole tiles (a plain read of a) the wave per row stays faster (~1.1k rows:
  // 15.1 against 17.7 us; ~2.2k rows: 16.5 against 25.1).
  constexpr int PER = NC >= 4 ? NC / 4 : 1;
  __shared__ float red[4];
  if (use_skinny(M)) {
    const SplitPlan sp = oproj_plan<CfgSkinny>(g, M, slots);
    if (sp.full == 0 && sp.rem > 0)
      resid_rmsnorm_row_body<PER, CfgSkinny>(g, M, sp, gain, eps, out, red);
    else
      resid_rms_rows<NC, CfgSkinny>(g, M, sp, gain, eps, out);
  } else {
    const SplitPlan sp = oproj_plan<CfgSmall>(g, M, slots);
    if (sp.full == 0 && sp.rem > 0)
      resid_rmsnorm_row_body<PER, CfgSmall>(g, M, sp, gain, eps, out, red);
    else
      resid_rms_rows<NC, CfgSmall>(g, M, sp, gain, eps, out);
  }
}

// ------------------------------------------------------------------------------ 4. attention
// Work item = (query tile of <= 64 selected rows of one sequence, head, key split). 4 waves, each
// owning 16 queries. S^T = K Q^T is computed with the key block as the MFMA A operand, so a lane
// holds 4 keys x 1 query per fragment; that register layout is exactly the B operand that
// O^T = V^T P^T needs (keys permuted consistently on both sides), so P never leaves registers.
// K and V blocks of 64 keys stream global -> LDS by DMA through kAttnStages distinct buffers in row
// layout with a 16-byte chunk swizzle. The V^T operand is read straight from the row-layout V block
// with the gfx950 transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4i + e receives element e of the 8-byte rows addressed by lanes i, i+4, i+8, i+12, so when those
// lanes address 4 consecutive head dims of 4 keys, every lane ends with 4 keys of one head dim.
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  uint16_t* o;
  float* opart;
  float* ml;
  const int* hdr;
  const int* seq_off;
  const int* tile_off;
  const int* tile_seq;
  int N, H, d, S_max;
  float scale_log2;  // log2(e) / sqrt(head_dim)
};

// 32-key blocks, two stages (32 KB of LDS at head_dim 128) and four workgroups per CU: measured
// 53.9 / 108.3 us per layer at batch 8, N = 1024 / 2048, against 59.3 / 115.3 for 64-key blocks at
// two workgroups per CU and 55.7 / 112.8 for 32-key blocks with three stages at three per CU
#ifndef DCU_ATTN_KB
#define DCU_ATTN_KB 32
#endif
#ifndef DCU_ATTN_STAGES
#define DCU_ATTN_STAGES 2
#endif
#ifndef DCU_ATTN_WGS
#define DCU_ATTN_WGS 4
#endif
constexpr int kKB = 64;                      // key-range granularity of split units
constexpr int kAttnKB = DCU_ATTN_KB;         // keys per block (32 or 64; 64 at head_dim 32)
constexpr int kAttnStages = DCU_ATTN_STAGES; // LDS stages of (K, V) blocks
constexpr int kAttnWgs = DCU_ATTN_WGS;       // workgroups per CU the registers are budgeted for
static_assert(kAttnKB == 32 || kAttnKB == 64, "key block");

// Work plan of the attention grid (G persistent workgroups, kAttnWgs per CU) for the device-side
// query-tile count. Items are (query tile, head) pairs. When there are fewer items than half the
// workgroups (e.g. one sequence or few selected rows) every item is split along the keys into S
// ranges so that the units use the idle workgroups; otherwise every item runs whole. (Splitting only the
// items of a partial last round was measured slower at batch 8: 65.6 vs 57.6 us per layer, since
// the short units and the merge cost more than the half-empty round, whose workgroups run alone
// on their CUs.) A split unit writes its unnormalised fp32 output and (max, sum) to a unit-indexed
// slot; k_attn_combine merges an item's S units in split order. Split units: items * S < G + items.
// (Closed-loop step, ~60 rows per sequence, 384 items: S = 2 in one round of units against S = 3
// with a partial second round.)
constexpr int kAttnMaxUnits = 2 * kAttnWgs * 256;  // 2 * (attention workgroups per CU * 256 CUs)

struct AttnPlan {
  int full, rem, S, kps;
};

// Most key ranges an item is split into: ranges of at least 64 keys (two 32-key blocks, so a
// unit's blocks are nearly all in flight at once), at most 16
constexpr int kAttnMaxSplit = 16;    // key ranges per item at most
constexpr int kAttnMinRange = 128;   // keys per range at least
// Ranges shorter than 128 keys cost more in the merge (one partial row per range) than they save:
// batch 1, N = 1024 (32 items), attention + merge 19.5 us with 16 ranges of 64 keys, 16.3-16.7 with
// 8 of 128, 17.4 with 4 of 256.
inline int attn_s_max(int N) {
  const int r = N / kAttnMinRange;
  return r > 1 ? (r < kAttnMaxSplit ? r : kAttnMaxSplit) : 1;
}

__device__ inline AttnPlan attn_plan(int items, int G, int N, int S_max) {
  const int whole = (N + kKB - 1) / kKB * kKB;
  AttnPlan p{items, 0, 1, whole};
  if (items <= 0) return p;
  if (2 * items >= G) return p;
  // Two candidates for S (both <= S_max): floor(G / items), whose units fit one round, and
  // ceil(G / items), which fills every workgroup but may need a partial second round (units
  // < G + items). The one that gives the busiest workgroup the fewest 64-key steps, rounds x steps
  // per unit, wins (ties to the smaller S: fewer partial rows to merge); a partial extra round of
  // units costs a whole unit's time. (Closed form, int32: every workgroup evaluates it.)
  int S_lo = G / items, S_hi = (G + items - 1) / items;
  S_lo = S_lo < S_max ? S_lo : S_max;
  S_hi = S_hi < S_max ? S_hi : S_max;
  int best_S = 1, best_kps = whole, best_cost = whole / kKB;
  for (int c = 0; c < 2; ++c) {
    const int S = c == 0 ? S_lo : S_hi;
    if (S <= 1 || (c == 1 && S == S_lo)) continue;
    const int kps = ((N + S - 1) / S + kKB - 1) / kKB * kKB;
    const int S_eff = (N + kps - 1) / kps;  // every range starts below N
    const int cost = (items * S_eff + G - 1) / G * (kps / kKB);
    if (cost < best_cost) {
      best_cost = cost;
      best_S = S_eff;
      best_kps = kps;
    }
  }
  if (best_S <= 1) return p;
  return AttnPlan{0, items, best_S, best_kps};
}

// Chunk swizzle of a key row: 8 consecutive keys land on distinct 16-byte bank groups (the K
// fragment reads), and the 8 keys x two adjacent chunks that 32 lanes of a transposing V read
// address land on distinct 8-byte bank pairs: with 16 chunks per row (head_dim 128), keys 0..7
// of a group XOR their chunk index with 0, 2, .., 14, so each key's chunk pair is its own
// (rocprofv3 LdsBankConflict 1.0 -> 0 conflict cycles per access cycle for the attention kernel
// against 0, 2, 4, 6, 1, 3, 5, 7, which gave keys k and k + 4 the same pair). Narrower rows keep
// the 8-key spread of the K reads.
template <int CH>
__device__ __forceinline__ int kvsw(int key) {
  return CH >= 16 ? (((key & 3) << 1) | (((key >> 2) & 1) << 3))
                  : ((((key & 3) << 1) | ((key >> 2) & 1))) & (CH - 1);
}
template <int CH>
__device__ __forceinline__ int kswz(int key, int c) { return key * CH + (c ^ kvsw<CH>(key)); }

// Pair exchange across 16 or 32 lanes with the gfx950 permlane swaps (VALU, no LDS round trip).
// Called with the same value twice they return, in every lane l, the values of lanes l & ~S and
// l | S, so a symmetric combine of the two equals the combine with lane l ^ S.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

template <int DH>
__global__ __launch_bounds__(256, kAttnWgs) void k_attn(AttnArgs g) {
  constexpr int KB = DH == 32 ? 64 : kAttnKB;  // keys per block
  constexpr int kKF = KB / 16;                // 16-key fragments per block
  constexpr int CH = DH / 8;            // 16-byte chunks per head row
  constexpr int BLK = KB * CH;         // chunks per K (or V) block
  constexpr int NQ = BLK / 64 / 4;      // DMA instructions per wave per block, per operand
  constexpr int ST = kAttnStages;
  static_assert(NQ >= 1, "block size");
  static_assert(ST == 2 || ST == 3, "stages");
  __shared__ u32x4 k0[BLK], k1[BLK], k2[ST > 2 ? BLK : 1];
  __shared__ u32x4 v0[BLK], v1[BLK], v2[ST > 2 ? BLK : 1];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6, grp = lane >> 4, col = lane & 15;
  const int wid_s = __builtin_amdgcn_readfirstlane(wid);
  const int Tq = g.hdr[kHdrTq];
  const AttnPlan ap = attn_plan(Tq * g.H, gridDim.x, g.N, g.S_max);
  const int units = ap.full + ap.rem * ap.S;
  // per-lane (row, logical chunk) of this wave's DMA instructions
  int drow[NQ], dcol[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int p = (i * 4 + wid) * 64 + lane;
    drow[i] = p / CH;
    dcol[i] = (p % CH) ^ kvsw<CH>(drow[i]);
  }
  // per-lane halfword offsets of the transposing V reads: this lane addresses key 4*grp + j
  // (j = (lane >> 2) & 3) and head dims 16*df + 4*(lane & 3) .. +3 of the block
  int vto[DH / 16];
  {
    const int i = lane & 3, key = 4 * grp + ((lane >> 2) & 3);
#pragma unroll
    for (int df = 0; df < DH / 16; ++df) {
      const int dc = 2 * df + (i >> 1);
      vto[df] = key * DH + ((dc ^ kvsw<CH>(key)) * 8) + 4 * (i & 1);
    }
  }
  for (int w = blockIdx.x; w < units; w += gridDim.x) {
    // whole item, or split unit v of item full + v / S covering key range v mod S
    const int v = w - ap.full;
    const int item = w < ap.full ? w : ap.full + v / ap.S;
    const int split = w < ap.full ? 0 : v % ap.S;
    const int h = item % g.H;
    const int tile = item / g.H;
    const int b = g.tile_seq[tile];
    const int r0 = g.seq_off[b] + (tile - g.tile_off[b]) * kQTile;
    const int rend = g.seq_off[b + 1];
    // whole items cover every key; split units their range
    const int kbeg = split * ap.kps;
    const int kend = w < ap.full ? g.N : min(g.N, kbeg + ap.kps);
    const int nblk = (kend - kbeg + KB - 1) / KB;
    // this wave's 16 queries; lane column `col` is its query. A wave whose 16 rows all lie past
    // the sequence's last row (the ragged last tile) still issues its share of every block's DMA
    // and takes part in the barriers, but skips the scores, softmax and products: its SIMD issue
    // slots go to the co-resident workgroups
    const bool wave_live = r0 + wid_s * 16 < rend;
    int qr = r0 + wid * 16 + col;
    const bool qvalid = qr < rend;
    qr = qvalid ? qr : rend - 1;
    u32x4 qf[DH / 32];
#pragma unroll
    for (int kk = 0; kk < DH / 32; ++kk)
      qf[kk] = ld16(g.q + int64_t(qr) * g.d + h * DH + kk * 32 + grp * 8);

    f32x4 acc_o[DH / 16];
#pragma unroll
    for (int i = 0; i < DH / 16; ++i) acc_o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_part = 0.0f;
    // per-lane source offsets of block 0 (elements from the sequence/head base); full blocks
    // advance by 64 rows, the ragged last block clamps its rows to the last valid key
    const int64_t head_base = int64_t(b) * g.N * g.d + h * DH;
    int64_t doff[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) doff[i] = int64_t(kbeg + drow[i]) * g.d + dcol[i] * 8;
    const int64_t blk_step = int64_t(KB) * g.d;

    auto issue = [&](auto sidx, int j) {
      constexpr int S = decltype(sidx)::value;
      u32x4* kb = S == 0 ? k0 : (S == 1 ? k1 : k2);
      u32x4* vb = S == 0 ? v0 : (S == 1 ? v1 : v2);
      const int jj = j < nblk ? j : nblk - 1;
      const bool full = kbeg + (jj + 1) * KB <= kend;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        int64_t off;
        if (full) {
          off = head_base + doff[i] + jj * blk_step;
        } else {
          int key = kbeg + jj * KB + drow[i];
          key = key < kend ? key : kend - 1;
          off = head_base + int64_t(key) * g.d + dcol[i] * 8;
        }
        const uint32_t lo = uint32_t(reinterpret_cast<uintptr_t>(DCU_LDS_PTR(kb + (i * 4 + wid_s) * 64)));
        const uint32_t lv = uint32_t(reinterpret_cast<uintptr_t>(DCU_LDS_PTR(vb + (i * 4 + wid_s) * 64)));
        gemm::dma16(g.kc + off, lo);
        gemm::dma16(g.vc + off, lv);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    auto compute = [&](auto sidx, int j) {
      constexpr int S = decltype(sidx)::value;
      if (!wave_live) return;
      const u32x4* kb = S == 0 ? k0 : (S == 1 ? k1 : k2);
      const uint16_t* vh = reinterpret_cast<const uint16_t*>(S == 0 ? v0 : (S == 1 ? v1 : v2));
      const int kb0 = kbeg + j * KB;
      // S^T for 64 keys x 16 queries: 4 fragments (keys 16f + 4*grp + i)
      f32x4 s[kKF];
#pragma unroll
      for (int f = 0; f < kKF; ++f) {
        s[f] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int key = f * 16 + col;
#pragma unroll
        for (int kk = 0; kk < DH / 32; ++kk)
          s[f] = mfma16x16x32(kb[kswz<CH>(key, kk * 4 + grp)], qf[kk], s[f]);
      }
      // raw scores; the scale log2(e)/sqrt(dh) > 0 is applied inside exp2 (fma), and only the
      // ragged last block masks keys past the end
      if (kb0 + KB > kend) {
#pragma unroll
        for (int f = 0; f < kKF; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb0 + f * 16 + grp * 4 + i >= kend) s[f][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int f = 0; f < kKF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[f][i]);
      mx = max_xor32(max_xor16(mx));
      mx *= g.scale_log2;
      // lazy rescaling: the reference max only moves when a score exceeds it by more than 2^8, so
      // exp2(score - m_ref) <= 256 and the accumulators are rescaled rarely (exact after the final
      // division by the same-referenced sum)
      const bool grow = mx > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mx : m_run;
        const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int df = 0; df < DH / 16; ++df) acc_o[df] *= alpha;
      }
      float psum = 0.0f;
      uint32_t pk[kKF][2];
#pragma unroll
      for (int f = 0; f < kKF; ++f) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(s[f][i], g.scale_log2, -m_run));
          psum += p[i];
        }
        pk[f][0] = pack_bf2(p[0], p[1]);
        pk[f][1] = pack_bf2(p[2], p[3]);
      }
      l_part += psum;
      // O^T += V^T P^T over two 32-key chunks; MFMA k index 8*grp + j maps to key
      // 32c + 4*grp + j (j < 4) and 32c + 16 + 4*grp + (j - 4) (j >= 4)
#pragma unroll
      for (int c = 0; c < KB / 32; ++c) {
        const u32x4 pb = u32x4{pk[2 * c][0], pk[2 * c][1], pk[2 * c + 1][0], pk[2 * c + 1][1]};
#pragma unroll
        for (int df = 0; df < DH / 16; ++df) {
          const u32x2 lo = lds_read_tr16(vh + vto[df] + (32 * c) * DH);
          const u32x2 hi = lds_read_tr16(vh + vto[df] + (32 * c + 16) * DH);
          acc_o[df] = mfma16x16x32(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, acc_o[df]);
        }
      }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    auto iter = [&](auto cur, int j) {
      constexpr int S = decltype(cur)::value;
      constexpr int NXT = (S + ST - 1) % ST;
      gemm::wait_vm_lgkm0<(ST - 2) * 2 * NQ>();
      __builtin_amdgcn_s_barrier();  // block j has landed; the previous block is fully consumed
      issue(std::integral_constant<int, NXT>{}, j + ST - 1);
      compute(cur, j);
    };
    if (nblk > 0 && nblk <= ST) {
      // a short unit (split ranges of few blocks): all its blocks are issued at once, one buffer
      // each, and consumed in order without refills (one DMA latency instead of one per block)
      issue(I0{}, 0);
      if (nblk > 1) issue(I1{}, 1);
      if constexpr (ST == 3) { if (nblk > 2) issue(I2{}, 2); }
      auto consume = [&](auto cur, int j) {
        // blocks j+1 .. nblk-1 may still be in flight
        if (nblk - 1 - j >= 2) gemm::wait_vm_lgkm0<2 * 2 * NQ>();
        else if (nblk - 1 - j == 1) gemm::wait_vm_lgkm0<2 * NQ>();
        else gemm::wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        compute(cur, j);
      };
      consume(I0{}, 0);
      if (nblk > 1) consume(I1{}, 1);
      if constexpr (ST == 3) { if (nblk > 2) consume(I2{}, 2); }
      __builtin_amdgcn_s_barrier();  // every wave is done with the buffers before the next unit
    } else if (nblk > 0) {
      issue(I0{}, 0);
      if constexpr (ST == 3) issue(I1{}, 1);
      for (int j = 0; j < nblk; j += ST) {
        iter(I0{}, j);
        if (j + 1 < nblk) iter(I1{}, j + 1); else break;
        if constexpr (ST == 3) {
          if (j + 2 < nblk) iter(I2{}, j + 2); else break;
        }
      }
      gemm::wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
    }

    const float l_tot = sum_xor32(sum_xor16(l_part));
    if (qvalid) {
      if (w < ap.full) {
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int df = 0; df < DH / 16; ++df) {
          uint2 st;
          st.x = pack_bf2(acc_o[df][0] * inv, acc_o[df][1] * inv);
          st.y = pack_bf2(acc_o[df][2] * inv, acc_o[df][3] * inv);
          *reinterpret_cast<uint2*>(g.o + int64_t(qr) * g.d + h * DH + df * 16 + grp * 4) = st;
        }
      } else {
        // unit slot v: [kQTile query rows][DH] fp32 and [kQTile][2] (max, sum)
        const int qi = wid * 16 + col;
        float* op = g.opart + (int64_t(v) * kQTile + qi) * DH;
#pragma unroll
        for (int df = 0; df < DH / 16; ++df)
          *reinterpret_cast<float4*>(op + df * 16 + grp * 4) =
              make_float4(acc_o[df][0], acc_o[df][1], acc_o[df][2], acc_o[df][3]);
        if (grp == 0) {
          float* mlp = g.ml + (int64_t(v) * kQTile + qi) * 2;
          mlp[0] = m_run;
          mlp[1] = l_tot;
        }
      }
    }
  }
}

// merge the S (<= kAttnMaxSplit) units of every split item, one wave per (item, query row), in
// split order; exits at once when the plan split nothing. The (max, sum) pairs (lane s holds unit
// s's) and all S partial rows are loaded together, before the row's sequence lookup, which only
// gates the store: their slots follow from the unit index alone (a row past its sequence's end
// has slots that were never written; they are loaded and merged but not stored).
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs g, int DH, int attn_grid) {
  const AttnPlan ap = attn_plan(g.hdr[kHdrTq] * g.H, attn_grid, g.N, g.S_max);
  if (ap.rem == 0) return;
  const int lane = threadIdx.x & 63;
  const int S = ap.S;
  const int64_t pairs = int64_t(ap.rem) * kQTile;
  for (int64_t p = int64_t(blockIdx.x) * 4 + threadIdx.x / 64; p < pairs;
       p += int64_t(gridDim.x) * 4) {
    const int k = int(p / kQTile), j = int(p % kQTile);
    const int item = ap.full + k;
    const int h = item % g.H, tile = item / g.H;
    const int64_t slot0 = int64_t(k) * S * kQTile + j;  // unit s of this row: slot0 + s * kQTile
    float m_s = -INFINITY, l_s = 0.0f;
    if (lane < S) {
      const float2 v = *reinterpret_cast<const float2*>(g.ml + (slot0 + int64_t(lane) * kQTile) * 2);
      m_s = v.x;
      l_s = v.y;
    }
    float o0[kAttnMaxSplit], o1[kAttnMaxSplit];
#pragma unroll
    for (int u = 0; u < kAttnMaxSplit; ++u) {
      o0[u] = o1[u] = 0.0f;
      if (u < S) {
        const float* op = g.opart + (slot0 + int64_t(u) * kQTile) * DH;
        if (lane < DH) o0[u] = op[lane];
        if (lane + 64 < DH) o1[u] = op[lane + 64];
      }
    }
    const int b = g.tile_seq[tile];
    const int r = g.seq_off[b] + (tile - g.tile_off[b]) * kQTile + j;
    const int rend = g.seq_off[b + 1];
    const float mx = wave_max(m_s);
    float l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int u = 0; u < kAttnMaxSplit; ++u) {
      if (u >= S) break;
      const float w = __builtin_amdgcn_exp2f(__shfl(m_s, u, kWave) - mx);
      l += __shfl(l_s, u, kWave) * w;
      acc0 += o0[u] * w;
      acc1 += o1[u] * w;
    }
    if (r >= rend) continue;
    const float inv = 1.0f / l;
    uint16_t* dst = g.o + int64_t(r) * g.d + h * DH;
    if (lane < DH) dst[lane] = uint16_t(f_to_bf_bits(acc0 * inv));
    if (lane + 64 < DH) dst[lane + 64] = uint16_t(f_to_bf_bits(acc1 * inv));
  }
}

// ------------------------------------------------------------------------------ host side
constexpr int kCUs = 256;

// Attention of the device-side query tiles over the caches, then the merge of split units (it exits
// at once unless the device-side plan split the items).
int launch_attention(const AttnArgs& aa, int DH, hipStream_t s) {
  const int attn_blocks = kAttnWgs * kCUs;  // persistent; the plan depends on the device row count
  static_assert(2 * (kAttnWgs * kCUs) <= kAttnMaxUnits, "attention split slots");
  if (DH == 128)
    hipLaunchKernelGGL(k_attn<128>, dim3(attn_blocks), dim3(256), 0, s, aa);
  else if (DH == 64)
    hipLaunchKernelGGL(k_attn<64>, dim3(attn_blocks), dim3(256), 0, s, aa);
  else
    hipLaunchKernelGGL(k_attn<32>, dim3(attn_blocks), dim3(256), 0, s, aa);
  DCU_LAUNCH_CHECK();
  // the merge is a chain of dependent loads per (item, row): as many workgroups as the attention
  // grid keep four times more rows in flight than one per CU (closed-loop step: 79 -> 57 us)
  hipLaunchKernelGGL(k_attn_combine, dim3(attn_blocks), dim3(256), 0, s, aa, DH, attn_blocks);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}

struct Layout {
  int M_cap, Tq_max;
  size_t hdr, seq_off, tile_off, tile_seq, rowmap, xn, q, o, a, h, part, opart, ml, rope, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(const dcu_layer* w, int B, int N, int max_rows) {
  Layout L{};
  const int64_t BN = int64_t(B) * N;
  L.M_cap = int(max_rows <= 0 || max_rows > BN ? BN : max_rows);
  // query tiles: sum over sequences of ceil(rows_b / kQTile) <= ceil(M / kQTile) + B - 1
  L.Tq_max = (L.M_cap + kQTile - 1) / kQTile + B - 1;
  const size_t d = size_t(w->d), F = size_t(w->ffn), M = size_t(L.M_cap);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.hdr = take(64);
  L.seq_off = take(sizeof(int) * (B + 1));
  L.tile_off = take(sizeof(int) * (B + 1));
  L.tile_seq = take(sizeof(int) * L.Tq_max);
  L.rowmap = take(sizeof(int) * M);
  L.xn = take(2 * M * d);
  L.q = take(2 * M * d);
  L.o = take(2 * M * d);
  L.a = take(4 * M * d);
  L.h = take(2 * M * F);
  // split tail partials: at most 2 * (resident workgroups) tile segments of 128 x 128 fp32; with a
  // row capacity of at most 64 every device row count takes the 64 x 64 tiles, whose weight-streaming
  // split keeps at most one segment per resident workgroup
  L.part = L.M_cap <= CfgSkinny::BM
               ? take(size_t(4) * (2 * kCUs) * CfgSkinny::BM * CfgSkinny::BN)
               : take(size_t(4) * 2 * (2 * kCUs) * CfgSmall::BM * CfgSmall::BN);
  // attention split units: [units][kQTile][head_dim] fp32 and [units][kQTile][2]. A split plan
  // cuts each of at most Tq_max * n_heads items into at most S_max key ranges, and never makes
  // more than kAttnMaxUnits units
  const int64_t plan_units = int64_t(L.Tq_max) * w->n_heads * attn_s_max(N);
  const size_t units = size_t(plan_units < kAttnMaxUnits ? plan_units : kAttnMaxUnits);
  L.opart = take(size_t(4) * units * kQTile * w->head_dim);
  L.ml = take(size_t(4) * units * kQTile * 2);
  // rotary (cos, sin) per row and head-dim pair
  L.rope = take(w->weight_layout == DCU_WEIGHTS_BLOCKED_ROPE ? size_t(4) * M * w->head_dim : 0);
  L.total = off;
  return L;
}

int validate(const dcu_layer* w, int B, int N) {
  if (!w || B <= 0 || N <= 0) return DCU_EINVAL;
  if (!w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down || !w->g_attn || !w->g_ffn)
    return DCU_EINVAL;
  if (w->d <= 0 || w->n_heads <= 0 || w->head_dim <= 0 || w->ffn <= 0) return DCU_EINVAL;
  if (w->weight_layout == DCU_WEIGHTS_BLOCKED) {
    if (w->rope_theta != 0.0f) return DCU_EINVAL;
  } else if (w->weight_layout == DCU_WEIGHTS_BLOCKED_ROPE) {
    if (!(w->rope_theta > 0.0f) || w->rope_theta - w->rope_theta != 0.0f) return DCU_EINVAL;
  } else {
    return DCU_EUNSUPPORTED;
  }
  if (int64_t(w->n_heads) * w->head_dim != w->d) return DCU_EINVAL;
  if (!(w->rms_eps >= 0.0f)) return DCU_EINVAL;
  if (w->head_dim != 32 && w->head_dim != 64 && w->head_dim != 128) return DCU_EUNSUPPORTED;
  if (w->d % 64 != 0 || w->ffn % 64 != 0) return DCU_EUNSUPPORTED;
  if (N > 65536 || int64_t(B) * N > (int64_t(1) << 28) || B > kMaxSeqs) return DCU_EUNSUPPORTED;
  const void* ps[] = {w->w_qkv, w->w_o, w->w_gate_up, w->w_down, w->g_attn, w->g_ffn};
  for (const void* p : ps)
    if (!dcu_aligned16(p)) return DCU_EUNSUPPORTED;
  return DCU_OK;
}


// The persistent projection grids always hold the resident workgroup count, so that the tail of a
// tile walk can be split over idle slots (the split plan is a function of the device row count).
int gemm_slots() {
  return 2 * kCUs;  // two workgroups per CU (64-72 KB of LDS each)
}

// A row capacity of at most 64 takes the weight-streaming kernel (its grid is one workgroup per
// CU); otherwise the persistent two-per-CU kernel, which picks its tile shape on the device.
template <int EPI>
void launch_gemm(const GemmArgs& ga, hipStream_t s, int M_cap) {
  if (M_cap <= CfgStream::BM)
    hipLaunchKernelGGL((k_gemm_stream<EPI>), dim3(kStreamSlots), dim3(256), 0, s, ga);
  else
    hipLaunchKernelGGL((k_gemm<EPI>), dim3(gemm_slots()), dim3(256), 0, s, ga);
}

// The fixup is launched unless the host can tell that the projection will not split: with a row
// capacity of at most 64, every device row count takes the streaming kernel's 64 x 128 tiles with
// one row tile, so the split plan is the same for all of them.
template <int EPI>
void launch_fixup(const GemmArgs& ga, hipStream_t s, int M_cap) {
  if (M_cap <= CfgStream::BM) {
    using C = StreamCfg<EPI>;
    const int NT = EPI == EPI_SWIGLU ? ga.Nout / (C::BN / 2) : (ga.Nout + C::BN - 1) / C::BN;
    const SplitPlan sp = plan_split(NT, kStreamSlots, ga.K / C::BK, split_mode<EPI, C>());
    if (sp.rem == 0) return;
    hipLaunchKernelGGL((k_gemm_fixup<EPI>), dim3(2048), dim3(256), 0, s, ga, kStreamSlots);
    return;
  }
  hipLaunchKernelGGL((k_gemm_fixup<EPI>), dim3(2048), dim3(256), 0, s, ga, gemm_slots());
}

// Row-major [rows, cols] -> blocked layout (gemm.h): one 16-byte chunk per thread, reads coalesced
// along the rows. With a second source b (the up matrix), the 16-row groups of a and b alternate
// in the output (a's group g -> group 2g, b's group g -> group 2g + 1). With rope_rows > 0 (the Q
// and K rows of W_qkv) the rows below rope_rows are reordered inside each head of dh rows: head dim
// j < dh/2 becomes row 32(j/16) + j%16 of the head, j >= dh/2 row 32((j-dh/2)/16) + 16 + j%16.
__global__ __launch_bounds__(256) void k_pack_weights(const u32x4* __restrict__ a,
                                                      const u32x4* __restrict__ b, int64_t rows,
                                                      int64_t cols, int64_t rope_rows, int dh,
                                                      u32x4* __restrict__ out) {
  const int64_t cpr = cols / 8;  // chunks per row
  const int64_t n = rows * cpr;  // chunks per source
  const int64_t kt_n = cols / 64;
  const int nsrc = b ? 2 : 1;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n * nsrc;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int m = i < n ? 0 : 1;
    const int64_t k = i - m * n;
    const int64_t r0 = k / cpr, ch = k - r0 * cpr;
    int64_t r = r0;
    if (r0 < rope_rows) {
      const int64_t j = r0 % dh, h = dh / 2;
      const int64_t jj = j < h ? j : j - h;
      r = r0 - j + (jj >> 4) * 32 + (j < h ? 0 : 16) + (jj & 15);
    }
    const int64_t g = (r >> 4) * nsrc + m, kt = ch >> 3;
    const int rr = int(r & 15), c = int(ch & 7);
    out[(g * kt_n + kt) * 128 + c * 16 + rr] = (m ? b : a)[k];
  }
}

int launch_pack(const void* a, const void* b, int64_t rows, int64_t cols, int64_t rope_rows,
                int dh, void* out, void* stream) {
  const int64_t chunks = rows * cols / 8 * (b ? 2 : 1);
  const int64_t want = (chunks + 255) / 256;
  const unsigned grid = unsigned(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(k_pack_weights, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(a), static_cast<const u32x4*>(b), rows, cols,
                     rope_rows, dh, static_cast<u32x4*>(out));
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}

}  // namespace
}  // namespace dcu

extern "C" int dcu_pack_weights(const void* w, int32_t rows, int32_t cols, void* out,
                                void* stream) {
  if (!w || !out || rows <= 0 || cols <= 0) return DCU_EINVAL;
  if (rows % 16 != 0 || cols % 64 != 0) return DCU_EUNSUPPORTED;
  if (int64_t(rows) * cols >= (int64_t(1) << 40)) return DCU_EUNSUPPORTED;
  if (!dcu_aligned16(w) || !dcu_aligned16(out)) return DCU_EUNSUPPORTED;
  return dcu::launch_pack(w, nullptr, rows, cols, 0, 1, out, stream);
}

extern "C" int dcu_pack_qkv(const void* w_qkv, int32_t d, int32_t head_dim, void* out,
                            void* stream) {
  if (!w_qkv || !out || d <= 0 || head_dim <= 0) return DCU_EINVAL;
  if (d % head_dim != 0) return DCU_EINVAL;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return DCU_EUNSUPPORTED;
  if (d % 64 != 0 || 3 * int64_t(d) * d >= (int64_t(1) << 40)) return DCU_EUNSUPPORTED;
  if (!dcu_aligned16(w_qkv) || !dcu_aligned16(out)) return DCU_EUNSUPPORTED;
  return dcu::launch_pack(w_qkv, nullptr, 3 * int64_t(d), d, 2 * int64_t(d), head_dim, out,
                          stream);
}

extern "C" int dcu_pack_gate_up(const void* w_gate, const void* w_up, int32_t F, int32_t d,
                                void* out, void* stream) {
  if (!w_gate || !w_up || !out || F <= 0 || d <= 0) return DCU_EINVAL;
  if (F % 16 != 0 || d % 64 != 0) return DCU_EUNSUPPORTED;
  if (2 * int64_t(F) * d >= (int64_t(1) << 40)) return DCU_EUNSUPPORTED;
  if (!dcu_aligned16(w_gate) || !dcu_aligned16(w_up) || !dcu_aligned16(out))
    return DCU_EUNSUPPORTED;
  return dcu::launch_pack(w_gate, w_up, F, d, 0, 1, out, stream);
}

extern "C" size_t dcu_selective_layer_workspace(const dcu_layer* w, int32_t B, int32_t N,
                                                int32_t max_rows) {
  if (dcu::validate(w, B, N) != DCU_OK) return 0;
  return dcu::make_layout(w, B, N, max_rows).total;
}

extern "C" int dcu_selective_layer_staged(const dcu_layer* w, const void* x_in,
                                          const int32_t* sel_idx, const int32_t* sel_count,
                                          int32_t B, int32_t N, int32_t max_rows, void* k_cache,
                                          void* v_cache, void* y_out, void* workspace,
                                          size_t workspace_bytes, int32_t* rows_done,
                                          void* stream, void* const* events, int32_t n_events) {
  using namespace dcu;
  if (events != nullptr && n_events < DCU_LAYER_STAGES + 1) return DCU_EINVAL;
  int st = validate(w, B, N);
  if (st != DCU_OK) return st;
  if (!x_in || !k_cache || !v_cache || !y_out) return DCU_EINVAL;
  if ((sel_idx == nullptr) != (sel_count == nullptr)) return DCU_EINVAL;
  if (!dcu_aligned16(x_in) || !dcu_aligned16(k_cache) || !dcu_aligned16(v_cache) ||
      !dcu_aligned16(y_out))
    return DCU_EUNSUPPORTED;
  const Layout L = make_layout(w, B, N, max_rows);
  if (!workspace || workspace_bytes < L.total) return DCU_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DCU_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Ptrs P;
  P.hdr = reinterpret_cast<int*>(ws + L.hdr);
  P.seq_off = reinterpret_cast<int*>(ws + L.seq_off);
  P.tile_off = reinterpret_cast<int*>(ws + L.tile_off);
  P.tile_seq = reinterpret_cast<int*>(ws + L.tile_seq);
  P.rowmap = reinterpret_cast<int*>(ws + L.rowmap);
  P.xn = reinterpret_cast<uint16_t*>(ws + L.xn);
  P.q = reinterpret_cast<uint16_t*>(ws + L.q);
  P.o = reinterpret_cast<uint16_t*>(ws + L.o);
  P.a = reinterpret_cast<float*>(ws + L.a);
  P.h = reinterpret_cast<uint16_t*>(ws + L.h);
  P.opart = reinterpret_cast<float*>(ws + L.opart);
  P.ml = reinterpret_cast<float*>(ws + L.ml);
  P.rope = reinterpret_cast<float2*>(ws + L.rope);
  P.rope_dh = w->weight_layout == DCU_WEIGHTS_BLOCKED_ROPE ? w->head_dim : 0;
  P.rope_l2t = P.rope_dh > 0 ? float(log2(double(w->rope_theta))) : 0.0f;
  const int d = w->d, F = w->ffn, H = w->n_heads, DH = w->head_dim;
  const uint16_t* x = static_cast<const uint16_t*>(x_in);
  int stage = 0;
  auto mark = [&]() -> bool {
    if (!events) return true;
    void* e = events[stage++];  // a NULL entry skips that mark
    return !e || hipEventRecord(static_cast<hipEvent_t>(e), s) == hipSuccess;
  };
  if (!mark()) return DCU_EHIP;

  const int norm_blocks = (L.M_cap + 3) / 4 < 2048 ? (L.M_cap + 3) / 4 : 2048;
  const uint16_t* ga_ = static_cast<const uint16_t*>(w->g_attn);
  // A row capacity of at most 64: the gather and the RMSNorm run inside the QKV weight stream
  // (stage 1 and the QKV fixup stage are then empty)
  const bool fused_qkv = L.M_cap <= CfgSkinny::BM && d <= kFusedMaxD &&
                         (P.rope_dh == 0 || P.rope_dh <= kFusedMaxRopeDh);
  if (!fused_qkv) {
#define DCU_GATHER(NC)                                                                        \
  hipLaunchKernelGGL(k_gather_rmsnorm<NC>, dim3(norm_blocks), dim3(256), 0, s, x, sel_idx,    \
                     sel_count, int(B), int(N), L.M_cap, ga_, d, w->rms_eps, P.xn, P)
    switch (rms_nc(d, false)) {
      case 1: DCU_GATHER(1); break;
      case 2: DCU_GATHER(2); break;
      case 4: DCU_GATHER(4); break;
      case 8: DCU_GATHER(8); break;
      case 16: DCU_GATHER(16); break;
      default: DCU_GATHER(0); break;
    }
#undef DCU_GATHER
    DCU_LAUNCH_CHECK();
  }
  if (!mark()) return DCU_EHIP;

  GemmArgs ga{};
  ga.part = reinterpret_cast<float*>(ws + L.part);
  ga.hdr = P.hdr;
  ga.rowmap = P.rowmap;
  ga.d = d;
  // QKV projection, k/v scattered into the caches
  ga.A = P.xn;
  ga.W = static_cast<const uint16_t*>(w->w_qkv);
  ga.K = d;
  ga.Nout = 3 * d;
  ga.q = P.q;
  ga.kc = static_cast<uint16_t*>(k_cache);
  ga.vc = static_cast<uint16_t*>(v_cache);
  ga.rope_dh = P.rope_dh;
  ga.rope = P.rope;
  if (fused_qkv) {
    const int qkv_tiles = (3 * d + CfgSkinny::BN - 1) / CfgSkinny::BN;
    const dim3 grid(unsigned(qkv_tiles < kStreamSlots ? qkv_tiles : kStreamSlots));
    if (P.rope_dh > 0)
      hipLaunchKernelGGL(k_qkv_fused<EPI_QKV_ROPE>, grid, dim3(256), 0, s, ga, P, x, sel_idx,
                         sel_count, int(B), int(N), L.M_cap, ga_, w->rms_eps);
    else
      hipLaunchKernelGGL(k_qkv_fused<EPI_QKV>, grid, dim3(256), 0, s, ga, P, x, sel_idx,
                         sel_count, int(B), int(N), L.M_cap, ga_, w->rms_eps);
  } else if (P.rope_dh > 0) {
    launch_gemm<EPI_QKV_ROPE>(ga, s, L.M_cap);
  } else {
    launch_gemm<EPI_QKV>(ga, s, L.M_cap);
  }
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;
  if (!fused_qkv) {
    if (P.rope_dh > 0)
      launch_fixup<EPI_QKV_ROPE>(ga, s, L.M_cap);
    else
      launch_fixup<EPI_QKV>(ga, s, L.M_cap);
    DCU_LAUNCH_CHECK();
  }
  if (!mark()) return DCU_EHIP;

  // attention over the updated caches
  AttnArgs aa{};
  aa.q = P.q;
  aa.kc = static_cast<const uint16_t*>(k_cache);
  aa.vc = static_cast<const uint16_t*>(v_cache);
  aa.o = P.o;
  aa.opart = P.opart;
  aa.ml = P.ml;
  aa.hdr = P.hdr;
  aa.seq_off = P.seq_off;
  aa.tile_off = P.tile_off;
  aa.tile_seq = P.tile_seq;
  aa.N = N;
  aa.H = H;
  aa.d = d;
  aa.S_max = attn_s_max(N);  // at most 16 key ranges of >= 128 keys
  aa.scale_log2 = float(1.4426950408889634 / sqrt(double(DH)));
  st = launch_attention(aa, DH, s);
  if (st != DCU_OK) return st;
  if (!mark()) return DCU_EHIP;

  // output projection + residual -> a (fp32)
  ga.A = P.o;
  ga.W = static_cast<const uint16_t*>(w->w_o);
  ga.K = d;
  ga.Nout = d;
  ga.x = x;
  ga.a = P.a;

  launch_gemm<EPI_RESID>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;
  // RMSNorm before the FFN -> an (reuses the xn buffer). Rows of up to 4096 values and a row
  // capacity above 64: the output projection's split tiles are finished inside the RMSNorm kernel
  // (no fixup launch; stage 6 is then empty). At most 64 rows (a wave per row for a few dozen
  // rows, each group summing all its tiles' pieces: 17.2 us against 7.1 + 7.7 us for the fixup's
  // 2048 workgroups and the plain RMSNorm at batch 1) and wider rows take the two launches.
  const uint16_t* gf_ = static_cast<const uint16_t*>(w->g_ffn);
  // at most 64 rows and rows of up to 8192 values: a workgroup per row finishes the split tiles and
  // normalises (stage 6 empty)
  const int row_per = L.M_cap <= CfgStream::BM ? (d / 8 + 255) / 256 : 0;
  const bool row_rms = row_per >= 1 && row_per <= 4;
  const int rnc = L.M_cap <= CfgStream::BM ? 0 : rms_nc(d, true);
  const int o_slots = gemm_slots();
  if (rnc == 0 && !row_rms) launch_fixup<EPI_RESID>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;
  if (row_rms) {
#define DCU_ROW_RMS(PER)                                                                      \
  hipLaunchKernelGGL(k_resid_rmsnorm_row<PER>, dim3(unsigned(L.M_cap)), dim3(256), 0, s, ga,      \
                     L.M_cap <= CfgStream::BM ? kStreamSlots : o_slots, gf_, w->rms_eps, P.xn,   \
                     rows_done, int(B), P.seq_off)
    switch (row_per) {
      case 1: DCU_ROW_RMS(1); break;
      case 2: DCU_ROW_RMS(2); break;
      case 3: DCU_ROW_RMS(3); break;
      default: DCU_ROW_RMS(4); break;
    }
#undef DCU_ROW_RMS
  } else {
#define DCU_RMS(NC)                                                                        \
  hipLaunchKernelGGL(k_rmsnorm_f32<NC>, dim3(norm_blocks), dim3(256), 0, s, P.a, P.hdr, gf_, d, \
                     w->rms_eps, P.xn, rows_done, int(B), P.seq_off, P.rowmap)
#define DCU_RESID_RMS(NC)                                                                  \
  hipLaunchKernelGGL(k_resid_rmsnorm<NC>, dim3(norm_blocks), dim3(256), 0, s, ga, o_slots, gf_, \
                     w->rms_eps, P.xn, rows_done, int(B), P.seq_off)
    switch (rnc) {
      case 1: DCU_RESID_RMS(1); break;
      case 2: DCU_RESID_RMS(2); break;
      case 4: DCU_RESID_RMS(4); break;
      case 8: DCU_RESID_RMS(8); break;
      default:
        switch (rms_nc(d, true)) {
          case 1: DCU_RMS(1); break;
          case 2: DCU_RMS(2); break;
          case 4: DCU_RMS(4); break;
          case 8: DCU_RMS(8); break;
          default: DCU_RMS(0); break;
        }
        break;
    }
#undef DCU_RESID_RMS
#undef DCU_RMS
  }
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;

  // gate and up together, SwiGLU epilogue -> h
  ga.A = P.xn;
  ga.W = static_cast<const uint16_t*>(w->w_gate_up);
  ga.K = d;
  ga.Nout = F;
  ga.h = P.h;
  launch_gemm<EPI_SWIGLU>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;
  launch_fixup<EPI_SWIGLU>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;

  // down projection + residual, scattered back into y_out
  ga.A = P.h;
  ga.W = static_cast<const uint16_t*>(w->w_down);
  ga.K = F;
  ga.Nout = d;
  ga.y = static_cast<uint16_t*>(y_out);
  launch_gemm<EPI_DOWN>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;
  launch_fixup<EPI_DOWN>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  if (!mark()) return DCU_EHIP;
  return DCU_OK;
}

extern "C" int dcu_v_features(const dcu_layer* w, const void* x_in, int32_t B, int32_t N,
                              void* v_out, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dcu;
  int st = validate(w, B, N);
  if (st != DCU_OK) return st;
  if (!x_in || !v_out) return DCU_EINVAL;
  if (!dcu_aligned16(x_in) || !dcu_aligned16(v_out)) return DCU_EUNSUPPORTED;
  const Layout L = make_layout(w, B, N, 0);
  if (!workspace || workspace_bytes < L.total) return DCU_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DCU_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Ptrs P{};
  P.hdr = reinterpret_cast<int*>(ws + L.hdr);
  P.seq_off = reinterpret_cast<int*>(ws + L.seq_off);
  P.tile_off = reinterpret_cast<int*>(ws + L.tile_off);
  P.tile_seq = reinterpret_cast<int*>(ws + L.tile_seq);
  P.rowmap = reinterpret_cast<int*>(ws + L.rowmap);
  P.xn = reinterpret_cast<uint16_t*>(ws + L.xn);
  const int d = w->d;
  // every row: RMSNorm with the attention gain (the projection input of the layer)
  const int norm_blocks = (L.M_cap + 3) / 4 < 2048 ? (L.M_cap + 3) / 4 : 2048;
  {
    const uint16_t* x = static_cast<const uint16_t*>(x_in);
    const uint16_t* ga_ = static_cast<const uint16_t*>(w->g_attn);
#define DCU_GATHER(NC)                                                                        \
  hipLaunchKernelGGL(k_gather_rmsnorm<NC>, dim3(norm_blocks), dim3(256), 0, s, x, nullptr,    \
                     nullptr, int(B), int(N), L.M_cap, ga_, d, w->rms_eps, P.xn, P)
    switch (rms_nc(d, false)) {
      case 1: DCU_GATHER(1); break;
      case 2: DCU_GATHER(2); break;
      case 4: DCU_GATHER(4); break;
      case 8: DCU_GATHER(8); break;
      case 16: DCU_GATHER(16); break;
      default: DCU_GATHER(0); break;
    }
#undef DCU_GATHER
  }
  DCU_LAUNCH_CHECK();
  // V = xn W_v^T: the W_v rows (2d .. 3d-1) of the blocked W_qkv are its row groups from 2d/16 on
  GemmArgs ga{};
  ga.part = reinterpret_cast<float*>(ws + L.part);
  ga.hdr = P.hdr;
  ga.rowmap = P.rowmap;
  ga.d = d;
  ga.A = P.xn;
  ga.W = static_cast<const uint16_t*>(w->w_qkv) + int64_t(2 * d / 16) * (d / 64) * gemm::kBlockElems;
  ga.K = d;
  ga.Nout = d;
  ga.y = static_cast<uint16_t*>(v_out);
  launch_gemm<EPI_VPROJ>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  launch_fixup<EPI_VPROJ>(ga, s, L.M_cap);
  DCU_LAUNCH_CHECK();
  return DCU_OK;
}

extern "C" int dcu_attention_context(const dcu_layer* w, const void* x_in, int32_t B, int32_t N,
                                     const void* k_cache, const void* v_cache, void* ctx_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  using namespace dcu;
  int st = validate(w, B, N);
  if (st != DCU_OK) return st;
  if (!x_in || !k_cache || !v_cache || !ctx_out) return DCU_EINVAL;
  if (!dcu_aligned16(x_in) || !dcu_aligned16(k_cache) || !dcu_aligned16(v_cache) ||
      !dcu_aligned16(ctx_out))
    return DCU_EUNSUPPORTED;
  const Layout L = make_layout(w, B, N, 0);
  if (!workspace || workspace_bytes < L.total) return DCU_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DCU_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Ptrs P{};
  P.hdr = reinterpret_cast<int*>(ws + L.hdr);
  P.seq_off = reinterpret_cast<int*>(ws + L.seq_off);
  P.tile_off = reinterpret_cast<int*>(ws + L.tile_off);
  P.tile_seq = reinterpret_cast<int*>(ws + L.tile_seq);
  P.rowmap = reinterpret_cast<int*>(ws + L.rowmap);
  P.xn = reinterpret_cast<uint16_t*>(ws + L.xn);
  P.q = reinterpret_cast<uint16_t*>(ws + L.q);
  P.opart = reinterpret_cast<float*>(ws + L.opart);
  P.ml = reinterpret_cast<float*>(ws + L.ml);
  P.rope = reinterpret_cast<float2*>(ws + L.rope);
  P.rope_dh = w->weight_layout == DCU_WEIGHTS_BLOCKED_ROPE ? w->head_dim : 0;
  P.rope_l2t = P.rope_dh > 0 ? float(log2(double(w->rope_theta))) : 0.0f;
  const int d = w->d, DH = w->head_dim;
  // every row (dense plan): RMSNorm with the attention gain, row map, query tiles, rotary table
  const int norm_blocks = (L.M_cap + 3) / 4 < 2048 ? (L.M_cap + 3) / 4 : 2048;
  {
    const uint16_t* x = static_cast<const uint16_t*>(x_in);
    const uint16_t* ga_ = static_cast<const uint16_t*>(w->g_attn);
#define DCU_GATHER(NC)                                                                        \
  hipLaunchKernelGGL(k_gather_rmsnorm<NC>, dim3(norm_blocks), dim3(256), 0, s, x, nullptr,    \
                     nullptr, int(B), int(N), L.M_cap, ga_, d, w->rms_eps, P.xn, P)
    switch (rms_nc(d, false)) {
      case 1: DCU_GATHER(1); break;
      case 2: DCU_GATHER(2); break;
      case 4: DCU_GATHER(4); break;
      case 8: DCU_GATHER(8); break;
      case 16: DCU_GATHER(16); break;
      default: DCU_GATHER(0); break;
    }
#undef DCU_GATHER
  }
  DCU_LAUNCH_CHECK();
  // q = xn W_q^T: the first d rows of the blocked W_qkv (every output column is a Q column, so
  // the QKV epilogue only writes q rows; the caches are not touched)
  GemmArgs ga{};
  ga.part = reinterpret_cast<float*>(ws + L.part);
  ga.hdr = P.hdr;
  ga.rowmap = P.rowmap;
  ga.d = d;
  ga.A = P.xn;
  ga.W = static_cast<const uint16_t*>(w->w_qkv);
  ga.K = d;
  ga.Nout = d;
  ga.q = P.q;
  ga.rope_dh = P.rope_dh;
  ga.rope = P.rope;
  if (P.rope_dh > 0) {
    launch_gemm<EPI_QKV_ROPE>(ga, s, L.M_cap);
    DCU_LAUNCH_CHECK();
    launch_fixup<EPI_QKV_ROPE>(ga, s, L.M_cap);
  } else {
    launch_gemm<EPI_QKV>(ga, s, L.M_cap);
    DCU_LAUNCH_CHECK();
    launch_fixup<EPI_QKV>(ga, s, L.M_cap);
  }
  DCU_LAUNCH_CHECK();
  // attention of every row over the caches as given; in the dense plan compacted row r is global
  // row r, so the context rows land in place
  AttnArgs aa{};
  aa.q = P.q;
  aa.kc = static_cast<const uint16_t*>(k_cache);
  aa.vc = static_cast<const uint16_t*>(v_cache);
  aa.o = static_cast<uint16_t*>(ctx_out);
  aa.opart = P.opart;
  aa.ml = P.ml;
  aa.hdr = P.hdr;
  aa.seq_off = P.seq_off;
  aa.tile_off = P.tile_off;
  aa.tile_seq = P.tile_seq;
  aa.N = N;
  aa.H = w->n_heads;
  aa.d = d;
  aa.S_max = attn_s_max(N);
  aa.scale_log2 = float(1.4426950408889634 / sqrt(double(DH)));
  return launch_attention(aa, DH, s);
}

// ------------------------------------------------------------------------------ allocation-free call
// The scratch of dcu_selective_layer_noalloc: a library-owned device array (every GPU the library
// runs on holds its own copy until the process ends). In host code `scratch` names a host-side
// stand-in, not the device address: the device address comes from hipGetSymbolAddress, once per
// device, and only that address is passed to the kernels.
static __device__ __align__(256) unsigned char scratch[DCU_NOALLOC_SCRATCH_BYTES];

namespace dcu {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of the scratch array on the device that runs `stream`, looked up on the first call
// for that device with the device current.
int noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return DCU_EHIP;
  if (stream == nullptr) {
    dev = cur;
  } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    return DCU_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return DCU_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DCU_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return DCU_EHIP;
    if (e != hipSuccess || p == nullptr) return DCU_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DCU_OK;
}
}  // namespace
}  // namespace dcu

extern "C" int dcu_selective_layer_noalloc(const dcu_layer* w, const void* x_in,
                                           const int32_t* sel_idx, const int32_t* sel_count,
                                           int32_t B, int32_t N, int32_t max_rows, void* k_cache,
                                           void* v_cache, void* y_out, int32_t* rows_done,
                                           void* stream) {
  using namespace dcu;
  const int st = validate(w, B, N);
  if (st != DCU_OK) return st;
  if (make_layout(w, B, N, max_rows).total > size_t(DCU_NOALLOC_SCRATCH_BYTES)) return DCU_EWORKSPACE;
  void* ws = nullptr;
  const int sst = noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
  if (sst != DCU_OK) return sst;
  return dcu_selective_layer_staged(w, x_in, sel_idx, sel_count, B, N, max_rows, k_cache, v_cache,
                                    y_out, ws, size_t(DCU_NOALLOC_SCRATCH_BYTES), rows_done, stream,
                                    nullptr, 0);
}

extern "C" int dcu_selective_layer(const dcu_layer* w, const void* x_in, const int32_t* sel_idx,
                                   const int32_t* sel_count, int32_t B, int32_t N,
                                   int32_t max_rows, void* k_cache, void* v_cache, void* y_out,
                                   void* workspace, size_t workspace_bytes, int32_t* rows_done,
                                   void* stream) {
  return dcu_selective_layer_staged(w, x_in, sel_idx, sel_count, B, N, max_rows, k_cache, v_cache,
                                    y_out, workspace, workspace_bytes, rows_done, stream, nullptr,
                                    0);
}
