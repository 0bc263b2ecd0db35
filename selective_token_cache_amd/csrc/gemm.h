// Persistent bf16 MFMA GEMM core for gfx950: Y[M, Nout] = A[M, K] * W[Nout, K]^T, fp32 accumulation.
// A is row-major (K-contiguous activations); W comes in the blocked layout below.
//
// * One 256-thread workgroup (4 waves in a WGM x WGN grid) computes a BM x BN tile; each wave owns
//   WM x WN as (WM/16) x (WN/16) fragments of v_mfma_f32_16x16x32_bf16. The weight fragment is the
//   MFMA A operand and the activation fragment the B operand, so each lane ends with 4 consecutive
//   output columns of one output row.
// * K advances in tiles of 64. Tiles stream global -> LDS with global_load_lds_dwordx4 (no VGPR
//   staging) through STAGES distinct LDS buffers: while the MFMAs consume tile kt, the loads of tiles
//   kt+1 .. kt+STAGES-1 are in flight. Each buffer is a separate __shared__ array and the stage index
//   is a compile-time constant, so the compiler only waits on the DMA group that is actually consumed
//   (a raw s_barrier is used: __syncthreads would drain every outstanding load).
// * Blocked weights: W is stored as [Nout/16][K/64] blocks of 16 rows x 64 columns (2 KB); inside a
//   block, 16-byte chunk c (columns 8c .. 8c+7) of row r sits at chunk position 16 c + r. A block is
//   the 16 x 64 slice one weight fragment needs for one K-tile, in exactly the order its 64 lanes read
//   it (lane l of the fragment for the k-half ks takes chunk 64 ks + l), so the weight DMA copies
//   whole 1 KB runs and the fragment reads are linear (no bank conflicts, no swizzle), and each
//   fragment's weight stream over K is one contiguous range. (Measured against row-major weights:
//   the same results bit for bit, 7-8% faster at 64, 1122 and 2048 rows.)
// * A tile rows are BK bf16 in LDS; chunk c of row r is stored at c ^ (r & 7), which spreads the 16
//   rows read by one MFMA operand load over the banks. The DMA writes 64 consecutive chunks per
//   instruction, so the swizzle is applied by choosing which global chunk each lane fetches.
// * Rows of A beyond M are clamped to row M-1 (valid memory; their results are never stored); the
//   prefetch of K-tiles past the end is clamped to the last tile (its buffer is never consumed), which
//   keeps the number of DMA groups in flight uniform.
// * Tiles are walked persistently; tile ids are remapped so that consecutive M-tiles sharing one
//   weight tile run on the same XCD (workgroup i runs on XCD i % 8) and share its L2.
#pragma once

#include <type_traits>
#include <utility>

#include "common.h"

namespace dcu {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define DCU_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One wave-wide 16-byte-per-lane DMA: lane i copies 16 bytes from gptr to LDS byte address
// lds_addr + 16 i. Written as asm so that the compiler does not add its own (conservative) waits
// for the LDS writes: completion is tracked explicitly with s_waitcnt vmcnt before each barrier.
// No output registers; "memory" keeps other memory accesses from moving across it.
// M0 (the DMA's LDS base) is a register the compiler reserves, hence its -Winline-asm note that a
// clobbered M0 is not preserved: nothing here needs it preserved. The compiler itself uses M0 only
// for LDS DMA, GWS, message and indirect register-index instructions, and the kernels that call
// this function contain none of those: the build lists their gfx950 assembly and fails unless every
// M0 write there is this asm's, directly followed by its DMA, and nothing else reads M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with vmcnt = n (0..63) and lgkmcnt = 0; expcnt left at its maximum
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8));
}

// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N - 1>{}), in order
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait for every memory access the compiler tracks (the previous tile's epilogue loads and stores)
// before a main loop starts. The DMAs are asm the compiler does not count; if a tracked access were
// still pending at the loop head, the compiler's own wait for it (vmcnt 0, which also drains the
// DMAs in flight) would land inside the K loop and serialise the stages.
__device__ __forceinline__ void wait_tracked_memory() { wait_vm_lgkm0<0>(); }

// chunk c of activation row r in a stage buffer (8 16-byte chunks per row)
__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int NW_ = 4>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, NW = NW_;
  static constexpr int BK = 64, RC = 8;               // K-tile; 16-byte chunks per LDS row
  static constexpr int ROWS_PER_DMA = 8;              // rows written by one wave-wide 16-byte DMA
  static constexpr int THREADS = 64 * NW;
  static constexpr int WGM = BM / WM, WGN = BN / WN;
  static_assert(WGM * WGN == NW, "wave grid");
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int ROWS = BM + BN;                 // LDS rows per stage
  static constexpr int CHUNKS = ROWS * RC;             // 16-byte chunks per stage
  static constexpr int NQ = ROWS / (ROWS_PER_DMA * NW);  // DMA instructions per wave per stage
  static constexpr int NQA = BM / (ROWS_PER_DMA * NW);   // ... of which load activation rows
  static_assert(ROWS % (ROWS_PER_DMA * NW) == 0, "rows per stage");
  static_assert(BM % (ROWS_PER_DMA * NW) == 0, "activation / weight DMA split by instruction");
  static_assert(BN % 16 == 0 && WN % 16 == 0, "whole 16-row weight blocks");
  static_assert(STAGES >= 2 && STAGES <= 8, "stages");
  static_assert((STAGES - 2) * NQ < 64, "vmcnt range");
  using acc_t = f32x4;
};

// Elements of one blocked-weight block (16 rows x 64 columns)
constexpr int kBlockElems = 16 * 64;

// Block source of the weight operand: block(n_t, jb) is the first K-tile's block of tile rows
// 16 jb .. 16 jb + 15 of weight tile n_t; the next K-tiles follow at kBlockElems steps.
// The default maps tile row tr to weight row n_t*BN + tr (blocks past the end clamped to the last).
struct PlainBlocks {
  const uint16_t* W;
  int Nout;
  int KT;  // K / 64 of the matrix
  template <int BN>
  __device__ __forceinline__ const uint16_t* block(int n_t, int jb) const {
    const int G = Nout / 16;
    int g = n_t * (BN / 16) + jb;
    g = g < G ? g : G - 1;
    return W + int64_t(g) * KT * kBlockElems;
  }
  template <int BN>
  __device__ __forceinline__ int tiles() const { return (Nout + BN - 1) / BN; }
};

// Gate/up interleave: each wave's WN tile rows are WN/2 gate rows followed by the WN/2 up rows of
// the same output columns, so matching gate and up accumulators land in the same lane. W is the
// fused gate/up matrix: its 16-row groups alternate gate group g (group 2g) and up group g (2g+1).
template <int WN>
struct GateUpBlocks {
  static_assert((WN / 2) % 16 == 0, "gate and up halves of whole blocks");
  const uint16_t* W;
  int F;
  int KT;
  template <int BN>
  __device__ __forceinline__ const uint16_t* block(int n_t, int jb) const {
    const int tr = jb * 16, wn = tr / WN, within = tr % WN;
    const int j = n_t * (BN / 2) + wn * (WN / 2) + (within % (WN / 2));
    const int grp = 2 * (j / 16) + (within < WN / 2 ? 0 : 1);
    return W + int64_t(grp) * KT * kBlockElems;
  }
  template <int BN>
  __device__ __forceinline__ int tiles() const { return F / (BN / 2); }
};

// Per-lane global sources of a wave's NQ DMA instructions for K-tile kt0 of the range; instruction i
// advances by dma_step<C>(i) elements per K-tile. Instructions i < NQA load 8 activation rows
// (row-major, swizzled chunks; arow(r) is the first element of tile row r); the others load half a
// weight block (1 KB, linear).
template <class C, class WB, class AR>
__device__ __forceinline__ void dma_sources_rows(const uint16_t* (&src)[C::NQ], const AR& arow,
                                                 int n_t, const WB& wb, int kt0) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < C::NQ; ++i) {
    const int q = i * C::NW + wid;
    if (i < C::NQA) {
      const int row = q * C::ROWS_PER_DMA + lane / C::RC;
      const int c = (lane % C::RC) ^ (row & 7);
      src[i] = arow(row) + c * 8 + kt0 * C::BK;
    } else {
      const int qb = q - C::BM / C::ROWS_PER_DMA;  // weight half-block: block qb / 2, half qb % 2
      src[i] = wb.template block<C::BN>(n_t, qb >> 1) + int64_t(kt0) * kBlockElems +
               (qb & 1) * (kBlockElems / 2) + lane * 8;
    }
  }
}

// The same for a row-major A of M rows from row m0 (rows past M clamped to row M-1)
template <class C, class WB>
__device__ __forceinline__ void dma_sources(const uint16_t* (&src)[C::NQ], const uint16_t* A, int M,
                                            int K, int m0, int n_t, const WB& wb, int kt0) {
  dma_sources_rows<C>(
      src,
      [&](int row) {
        const int ar = m0 + row < M ? m0 + row : M - 1;
        return A + int64_t(ar) * K;
      },
      n_t, wb, kt0);
}

template <class C>
__host__ __device__ constexpr int dma_step(int i) {
  return i < C::NQA ? C::BK : kBlockElems;
}

// weight fragment f (0 <= f < FN) of wave column wn, k-half ks, as the lane's chunk index in a stage
template <class C>
__device__ __forceinline__ int wfrag(int wn, int f, int ks, int lane) {
  return C::BM * C::RC + (wn * (C::WN / 16) + f) * 128 + ks * 64 + lane;
}

// Main loop over one tile. acc is [FM][FN] f32x4. Buffers b0..b3 are the stage arrays.
// K-tiles [kt0, kt1) of the tile (all of K when kt1 < 0).
template <class C, class WB>
__device__ __forceinline__ void tile_mainloop(f32x4 (&acc)[C::FM][C::FN], const uint16_t* A, int M,
                                              int K, int m0, int n_t, const WB& wb, u32x4* b0,
                                              u32x4* b1, u32x4* b2, u32x4* b3, int kt0 = 0,
                                              int kt1 = -1) {
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int wm = wid / C::WGN, wn = wid % C::WGN;
  const int KT = (kt1 < 0 ? K / C::BK : kt1) - kt0;
  const uint16_t* src[C::NQ];
  dma_sources<C>(src, A, M, K, m0, n_t, wb, kt0);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{};
  wait_tracked_memory();

  // the wave index as a scalar, so every DMA's LDS base (M0) is computed without readfirstlane
  const int wid_s = __builtin_amdgcn_readfirstlane(wid);
  // all DMA instructions of a stage are issued back to back and kept together by a scheduling
  // barrier: interleaving them with LDS reads would make every M0 write wait for those reads
  auto issue = [&](auto sidx, int kt) {
    constexpr int S = decltype(sidx)::value;
    u32x4* buf = S == 0 ? b0 : (S == 1 ? b1 : (S == 2 ? b2 : b3));
    const int kc = kt < KT ? kt : KT - 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      const int q = i * C::NW + wid_s;
      dma16(static_cast<const void*>(src[i] + int64_t(kc) * dma_step<C>(i)),
            uint32_t(reinterpret_cast<uintptr_t>(DCU_LDS_PTR(buf + q * 64))));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](auto sidx) {
    constexpr int S = decltype(sidx)::value;
    const u32x4* buf = S == 0 ? b0 : (S == 1 ? b1 : (S == 2 ? b2 : b3));
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const int c = ks * 4 + (lane >> 4);
      u32x4 fw[C::FN], fx[C::FM];
#pragma unroll
      for (int f = 0; f < C::FN; ++f) fw[f] = buf[wfrag<C>(wn, f, ks, lane)];
#pragma unroll
      for (int f = 0; f < C::FM; ++f) fx[f] = buf[swz(wm * C::WM + f * 16 + (lane & 15), c)];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma(fw[j], fx[i], acc[i][j]);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // prologue: tiles 0 .. STAGES-2
  issue(I0{}, 0);
  if constexpr (C::STAGES > 2) issue(I1{}, 1);
  if constexpr (C::STAGES > 3) issue(I2{}, 2);
  // steady state, unrolled by STAGES so that every buffer index is a constant
  auto iter = [&](auto cur, int kt) {
    constexpr int S = decltype(cur)::value;
    constexpr int NXT = (S + C::STAGES - 1) % C::STAGES;
    wait_vm_lgkm0<(C::STAGES - 2) * C::NQ>();
    __builtin_amdgcn_s_barrier();
    issue(std::integral_constant<int, NXT>{}, kt + C::STAGES - 1);
    compute(cur);
  };
  for (int kt = 0; kt < KT; kt += C::STAGES) {
    iter(I0{}, kt);
    if (kt + 1 < KT) iter(I1{}, kt + 1); else break;
    if constexpr (C::STAGES > 2) { if (kt + 2 < KT) iter(I2{}, kt + 2); else break; }
    if constexpr (C::STAGES > 3) { if (kt + 3 < KT) iter(I3{}, kt + 3); else break; }
  }
  // drain the clamped prefetches before the buffers are reused by the next tile
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
}

// The same main loop for any stage count (2..8): the STAGES buffers sit at compile-time offsets of
// one LDS array; the DMA sources come from dma_sources / dma_sources_rows for K-tile kt0. Used by
// the weight stream of a few rows (one workgroup per CU). ap(f, k, frag) is applied to every
// activation fragment after its LDS read: fragment f (0 <= f < FM) of the lane's row, whose 8
// elements are columns k .. k+7 of A.
template <class C, class AP>
__device__ __forceinline__ void tile_mainloop_deep(f32x4 (&acc)[C::FM][C::FN],
                                                   const uint16_t* const (&src0)[C::NQ],
                                                   u32x4* smem, int kt0, int kt1, AP& ap) {
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int wm = wid / C::WGN, wn = wid % C::WGN;
  const int KT = kt1 - kt0;
  const uint16_t* src[C::NQ];
#pragma unroll
  for (int i = 0; i < C::NQ; ++i) src[i] = src0[i];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{};
  wait_tracked_memory();
  const int wid_s = __builtin_amdgcn_readfirstlane(wid);
  auto issue = [&](auto sidx, int kt) {
    u32x4* buf = smem + decltype(sidx)::value * C::CHUNKS;
    const int kc = kt < KT ? kt : KT - 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      const int q = i * C::NW + wid_s;
      dma16(static_cast<const void*>(src[i] + int64_t(kc) * dma_step<C>(i)),
            uint32_t(reinterpret_cast<uintptr_t>(DCU_LDS_PTR(buf + q * 64))));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](auto sidx, int kt) {
    const u32x4* buf = smem + decltype(sidx)::value * C::CHUNKS;
#pragma unroll
    for (int ks = 0; ks < C::BK / 32; ++ks) {
      const int c = ks * 4 + (lane >> 4);
      u32x4 fw[C::FN], fx[C::FM];
#pragma unroll
      for (int f = 0; f < C::FN; ++f) fw[f] = buf[wfrag<C>(wn, f, ks, lane)];
#pragma unroll
      for (int f = 0; f < C::FM; ++f) fx[f] = buf[swz(wm * C::WM + f * 16 + (lane & 15), c)];
#pragma unroll
      for (int f = 0; f < C::FM; ++f) ap(f, (kt0 + kt) * C::BK + c * 8, fx[f]);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma(fw[j], fx[i], acc[i][j]);
    }
  };
  // prologue: K-tiles 0 .. STAGES-2
  static_for<C::STAGES - 1>([&](auto s) { issue(s, decltype(s)::value); });
  for (int kt = 0; kt < KT; kt += C::STAGES) {
    bool live = true;
    static_for<C::STAGES>([&](auto cur) {
      constexpr int S = decltype(cur)::value;
      if (!live || kt + S >= KT) {
        live = false;
        return;
      }
      wait_vm_lgkm0<(C::STAGES - 2) * C::NQ>();
      __builtin_amdgcn_s_barrier();
      issue(std::integral_constant<int, (S + C::STAGES - 1) % C::STAGES>{}, kt + S + C::STAGES - 1);
      compute(cur, kt + S);
    });
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
}

// Two-buffer main loop with early refill. A K-tile's fragments are all read into registers right
// after the barrier that makes the tile visible; a second barrier (after lgkmcnt(0)) then frees its
// buffer, which is refilled at once with K-tile kt+2 while the MFMAs run. Each DMA thus has two
// K-tiles of compute to land instead of one, with the same two buffers.
template <class C, class WB>
__device__ __forceinline__ void tile_mainloop_er(f32x4 (&acc)[C::FM][C::FN], const uint16_t* A,
                                                 int M, int K, int m0, int n_t, const WB& wb,
                                                 u32x4* b0, u32x4* b1, int kt0 = 0, int kt1 = -1) {
  static_assert(C::STAGES == 2, "two buffers");
  static_assert(C::NQ < 64, "vmcnt range");
  constexpr int KS = C::BK / 32;
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int wm = wid / C::WGN, wn = wid % C::WGN;
  const int KT = (kt1 < 0 ? K / C::BK : kt1) - kt0;
  const uint16_t* src[C::NQ];
  dma_sources<C>(src, A, M, K, m0, n_t, wb, kt0);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{};
  wait_tracked_memory();
  const int wid_s = __builtin_amdgcn_readfirstlane(wid);
  auto issue = [&](auto sidx, int kt) {
    constexpr int S = decltype(sidx)::value;
    u32x4* buf = S == 0 ? b0 : b1;
    const int kc = kt < KT ? kt : KT - 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < C::NQ; ++i) {
      const int q = i * C::NW + wid_s;
      dma16(static_cast<const void*>(src[i] + int64_t(kc) * dma_step<C>(i)),
            uint32_t(reinterpret_cast<uintptr_t>(DCU_LDS_PTR(buf + q * 64))));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto iter = [&](auto sidx, int kt) {
    constexpr int S = decltype(sidx)::value;
    const u32x4* buf = S == 0 ? b0 : b1;
    wait_vm_lgkm0<C::NQ>();         // K-tile kt landed (kt+1 may still be in flight)
    __builtin_amdgcn_s_barrier();   // ... for every wave
    asm volatile("" ::: "memory");  // the LDS reads below stay after the barrier
    u32x4 fw[KS][C::FN], fx[KS][C::FM];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks * 4 + (lane >> 4);
#pragma unroll
      for (int f = 0; f < C::FN; ++f) fw[ks][f] = buf[wfrag<C>(wn, f, ks, lane)];
#pragma unroll
      for (int f = 0; f < C::FM; ++f) fx[ks][f] = buf[swz(wm * C::WM + f * 16 + (lane & 15), c)];
    }
    wait_vm_lgkm0<C::NQ>();         // this wave's reads of the buffer are done
    __builtin_amdgcn_s_barrier();   // ... every wave's: refill it with K-tile kt+2
    issue(sidx, kt + 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma(fw[ks][j], fx[ks][i], acc[i][j]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  issue(I0{}, 0);
  issue(I1{}, 1);
  for (int kt = 0; kt < KT; kt += 2) {
    iter(I0{}, kt);
    if (kt + 1 < KT) iter(I1{}, kt + 1); else break;
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
}

// Persistent tile walk: the round-th tile of this workgroup, remapped XCD-major (workgroup i runs
// on XCD i mod 8; each XCD takes a contiguous run of tiles, so the M-tiles that share a weight tile
// share that XCD's L2). A partial last round is spread evenly over the 8 XCDs (XCD x takes
// rem/8 tiles, one more for x < rem mod 8) instead of filling the first XCDs and idling the rest.
__device__ __forceinline__ bool next_tile(int round, int total, int MT, int* m_t, int* n_t) {
  const int G = gridDim.x, per_xcd = G >> 3;
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int base = round * G;
  if (base >= total) return false;
  const int rem = total - base;
  int tile;
  if (rem >= G) {
    tile = base + x * per_xcd + j;
  } else {
    const int q = rem >> 3, r = rem & 7;
    if (j >= q + (x < r ? 1 : 0)) return false;
    tile = base + x * q + (x < r ? x : r) + j;
  }
  *m_t = tile % MT;
  *n_t = tile / MT;
  return true;
}

}  // namespace gemm
}  // namespace dcu
