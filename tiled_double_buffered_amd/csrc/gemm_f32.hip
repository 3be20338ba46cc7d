// gemmf32: FP32 GEMM C = A.B for gfx950 (MI355X), tiled through LDS, with a
// single-buffered and a double-buffered K-loop, an FP32 matrix-core micro-kernel,
// a guarded path for ragged or misaligned operands, and a per-shape dispatcher.
//
// What the K-loop does comes from two pages on the technique:
//   "Double Buffering" (metalworking glossary), code figure: two staging buffers per
//     operand; each iteration opens with one barrier, loads tile l+1 into the idle
//     buffer when there is one, computes on the current buffer and swaps.
//   "Case Study: The Double-Buffered GEMM", code figure: a prologue loads tile 0 into
//     buffer 0 before the loop; its second paragraph: the sibling (single-buffered)
//     kernel has one buffer set and two barriers per iteration.
//   Same case study, paragraph after the figure: the one barrier serves both as "the
//     prefetch has landed" and as "every wave is done reading the buffer about to be
//     overwritten", because the buffers alternate.
// The pages' own kernels target Apple GPUs; everything below is written for CDNA4:
// 64-lane waves, v_mfma_f32_32x32x2_f32 on the matrix cores, LDS with padded rows,
// 16-byte global loads, and an XCD-aware ordering of workgroups.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "gemmf32.h"

namespace gemmf32 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------------------------
// Tile configuration.
//   BM x BN : output tile of one workgroup        BK : K depth of one LDS tile
//   WAVES_M x WAVES_N waves per workgroup; each wave owns a TM x TN sub-tile made of
//   FM x FN blocks of 32 x 32, one 16-register accumulator per block.
// LDS layout of one slot (FP32):
//   As[BM][AS]  A tile with k contiguous, row stride AS = BK + 4 (the pad of 4 words
//               makes the 16-byte reads of 8 or 16 consecutive rows hit distinct banks)
//   Bs[BK][BS]  B tile with n contiguous, row stride BS = BN + 8 (so the two half-waves,
//               which read rows 4 apart, land on opposite halves of the 64 banks)
// ------------------------------------------------------------------------------------
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int AS = BK + 4;
  static constexpr int BS = BN + 8;
  static constexpr int A_SLOT = BM * AS;
  static constexpr int B_SLOT = BK * BS;
  static constexpr int SLOT = A_SLOT + B_SLOT;  // floats per LDS slot
  // Global -> LDS copy: 16-byte groups of 4 consecutive floats along a row.
  static constexpr int A_GROUPS_PER_ROW = BK / 4;
  static constexpr int B_GROUPS_PER_ROW = BN / 4;
  static constexpr int A_PER_T = BM * BK / 4 / NT;  // groups per thread per tile
  static constexpr int B_PER_T = BK * BN / 4 / NT;
  static constexpr int A_ROWS_PER_PASS = NT / A_GROUPS_PER_ROW;
  static constexpr int B_ROWS_PER_PASS = NT / B_GROUPS_PER_ROW;
  // Unroll the double-buffered loop by two (fixed slot addresses) unless the wave's
  // register budget is too tight for it: with eight waves per workgroup a wave has 256
  // registers, and a 128-accumulator wave tile plus two tiles' worth of copy and fragment
  // registers would spill.
  static constexpr bool DB_UNROLL = NT <= 256 || FM * FN * 16 <= 64;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(BK % 8 == 0, "BK must be a multiple of 8");
  static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "copy must divide");
  static_assert(NT % A_GROUPS_PER_ROW == 0 && NT % B_GROUPS_PER_ROW == 0, "copy rows");
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "copy work per thread");
};

// Flags passed to the kernel.
enum : int {
  kVecA = 1,  // A 16-byte aligned and lda % 4 == 0: rows can be read 16 bytes at a time
  kVecB = 2,  // same for B
};

// ------------------------------------------------------------------------------------
// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin; renumber
// them so that consecutive ids run on one XCD (which has its own L2), then walk the
// tiles in column-major groups of `group_m` tile rows so that workgroups close in id
// share panels of A and B.  Both choices can be changed per launch for measurement (flags
// bits 8..15: group_m, 0 = the default 8; bit 16: keep the hardware order of ids).
// ------------------------------------------------------------------------------------
enum : int { kRasterGroupShift = 8, kRasterNoXcdRemap = 1 << 16 };

__device__ inline void tile_coords(int tiles_m, int tiles_n, int flags, int& tm, int& tn) {
  constexpr int kXcds = 8;
  const int gm_flag = (flags >> kRasterGroupShift) & 0xff;
  const int group_m = gm_flag ? gm_flag : 8;
  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  if (!(flags & kRasterNoXcdRemap) && nwg % kXcds == 0)
    bid = (bid % kXcds) * (nwg / kXcds) + bid / kXcds;
  const int per_group = group_m * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * group_m;
  const int rows = min(tiles_m - first_m, group_m);
  const int in_group = bid - group * per_group;
  tm = first_m + in_group % rows;
  tn = in_group / rows;
}

// ------------------------------------------------------------------------------------
// The workgroup's copy of one K tile: global memory -> registers -> LDS.
// Thread t moves groups g = t + p * NT (p = 0 .. PER_T-1); group g of A is row
// g / (BK/4), columns 4 * (g % (BK/4)) .. +3 of the tile; likewise for B with BN/4.
// ------------------------------------------------------------------------------------
template <class C>
struct TileCopy {
  floatx4 ra[C::A_PER_T];
  floatx4 rb[C::B_PER_T];

  // Per-thread coordinates inside the tile.
  int a_row, a_col, b_row, b_col;

  __device__ inline void init(int tid) {
    a_row = tid / C::A_GROUPS_PER_ROW;
    a_col = 4 * (tid % C::A_GROUPS_PER_ROW);
    b_row = tid / C::B_GROUPS_PER_ROW;
    b_col = 4 * (tid % C::B_GROUPS_PER_ROW);
  }

  // Fast path: the whole tile lies inside the matrices and rows are 16-byte aligned.
  __device__ inline void load_a_fast(const float* __restrict__ A, int64_t lda, int m0,
                                     int k0) {
    const float* p = A + (int64_t)(m0 + a_row) * lda + (k0 + a_col);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      ra[i] = *reinterpret_cast<const floatx4*>(p + (int64_t)(i * C::A_ROWS_PER_PASS) * lda);
  }
  __device__ inline void load_b_fast(const float* __restrict__ B, int64_t ldb, int n0,
                                     int k0) {
    const float* p = B + (int64_t)(k0 + b_row) * ldb + (n0 + b_col);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      rb[i] = *reinterpret_cast<const floatx4*>(p + (int64_t)(i * C::B_ROWS_PER_PASS) * ldb);
  }

  // Guarded path: element by element; anything outside M x K (A) or K x N (B) reads as
  // +0, so a partial K tile adds exact zeros and edge rows/columns stay finite.
  __device__ inline void load_a_guarded(const float* __restrict__ A, int64_t lda, int M,
                                        int K, int m0, int k0) {
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int r = m0 + a_row + i * C::A_ROWS_PER_PASS;
      const int c = k0 + a_col;
      const float* p = A + (int64_t)r * lda + c;
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (r < M && c + e < K) ? p[e] : 0.0f;
      ra[i] = v;
    }
  }
  __device__ inline void load_b_guarded(const float* __restrict__ B, int64_t ldb, int N,
                                        int K, int n0, int k0) {
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int r = k0 + b_row + i * C::B_ROWS_PER_PASS;
      const int c = n0 + b_col;
      const float* p = B + (int64_t)r * ldb + c;
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (r < K && c + e < N) ? p[e] : 0.0f;
      rb[i] = v;
    }
  }

  __device__ inline void store_a(float* slot) {
    float* As = slot;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      *reinterpret_cast<floatx4*>(As + (a_row + i * C::A_ROWS_PER_PASS) * C::AS + a_col) = ra[i];
  }
  __device__ inline void store_b(float* slot) {
    float* Bs = slot + C::A_SLOT;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      *reinterpret_cast<floatx4*>(Bs + (b_row + i * C::B_ROWS_PER_PASS) * C::BS + b_col) = rb[i];
  }
  __device__ inline void store(float* slot) {
    store_a(slot);
    store_b(slot);
  }
};

// ------------------------------------------------------------------------------------
// Matrix-core micro-kernel.
// v_mfma_f32_32x32x2_f32: lane L supplies A[L%32][L/32] and B[L/32][L%32] of a
// 32x2 by 2x32 step and accumulates a 32x32 block, of which lane L holds column L%32,
// rows 8*(r/4) + 4*(L/32) + r%4 in accumulator register r (r = 0..15).
// A K tile is consumed in BK/8 rounds of eight k values.  In round q lane L reads
// A[row][8q+4h .. 8q+4h+3] (h = L/32) with one 16-byte LDS read and B[8q+4h+t][col] for
// t = 0..3; the MFMA for t then sums k = 8q+t and 8q+4+t.  The four MFMAs of a round
// cover its eight k values once each, so the product is unchanged; only the order of the
// k sum differs from the textbook loop.
// ------------------------------------------------------------------------------------
template <class C>
struct Frag {
  floatx4 a[C::FM];
  float b[C::FN][4];
};

// This lane's fragment offsets (in floats) inside an LDS slot.
template <class C>
struct LaneView {
  int a_off, b_off;
  __device__ inline void init(int wm, int wn, int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    a_off = (wm * C::TM + l32) * C::AS + 4 * h;
    b_off = C::A_SLOT + (4 * h) * C::BS + wn * C::TN + l32;
  }
};

template <class C>
__device__ inline void read_frag(const float* slot, const LaneView<C>& lv, int q, Frag<C>& f) {
  const float* a_ptr = slot + lv.a_off + 8 * q;
  const float* b_ptr = slot + lv.b_off + 8 * q * C::BS;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
    f.a[fm] = *reinterpret_cast<const floatx4*>(a_ptr + fm * 32 * C::AS);
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int t = 0; t < 4; ++t) f.b[fn][t] = b_ptr[t * C::BS + fn * 32];
}

// The MFMAs of one round; PART 0 = all four k pairs, 1 = the first two, 2 = the last two.
template <class C, int PART>
__device__ inline void mfma_round(const Frag<C>& f, floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int t0 = PART == 2 ? 2 : 0;
  constexpr int t1 = PART == 1 ? 2 : 4;
#pragma unroll
  for (int t = t0; t < t1; ++t)
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] =
            __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[fm][t], f.b[fn][t], acc[fm][fn], 0, 0, 0);
}

// ------------------------------------------------------------------------------------
// Instruction interleaving for the unguarded loops.  The compiler's scheduler, left
// alone, sinks the global prefetch loads to just before their LDS stores, which exposes
// their whole latency.  These hints (sched_group_barrier, applied to the scheduling
// region they close) ask for each other memory instruction to be followed by a share of
// the MFMAs, so that the matrix pipe keeps issuing while loads and stores are in flight.
// ------------------------------------------------------------------------------------
enum : int { kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100,
             kSchedDsWrite = 0x200 };

template <int MASK, int SIZE>
__device__ __forceinline__ void sched_group() {
  if constexpr (SIZE > 0) __builtin_amdgcn_sched_group_barrier(MASK, SIZE, 0);
}

// NOTHER instructions of class OMASK spread evenly over NMFMA MFMAs.
template <int OMASK, int NOTHER, int NMFMA, int I = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (NOTHER == 0) {
    sched_group<kSchedMfma, NMFMA>();
  } else if constexpr (I < NOTHER) {
    constexpr int lo = I * NMFMA / NOTHER, hi = (I + 1) * NMFMA / NOTHER;
    sched_group<OMASK, 1>();
    sched_group<kSchedMfma, hi - lo>();
    sched_interleave<OMASK, NOTHER, NMFMA, I + 1>();
  }
}

template <class C>
struct Sched {
  static constexpr int R = C::BK / 8;                  // rounds per K tile
  static constexpr int MQ = 4 * C::FM * C::FN;         // MFMAs per round
  static constexpr int G = C::A_PER_T + C::B_PER_T;    // 16-byte global loads per tile
  static constexpr int W = C::A_PER_T + C::B_PER_T;    // 16-byte LDS stores per tile
  static constexpr int D = C::FM + 2 * C::FN;          // LDS read instructions per round

  // Double-buffered, from the top of an iteration up to the barrier: round 0 carries the
  // global loads of tile l+1 and the LDS reads of round 1; middle rounds carry the reads
  // of the next round; the first half of the last round carries the LDS stores of tile
  // l+1 into the idle slot.
  template <int Q = 0>
  static __device__ __forceinline__ void db_before_barrier() {
    if constexpr (Q == 0) {
      sched_interleave<kSchedVmemRead, G, MQ / 2>();
      if constexpr (R > 1) sched_interleave<kSchedDsRead, D, MQ - MQ / 2>();
      else sched_group<kSchedMfma, MQ - MQ / 2>();
      db_before_barrier<1>();
    } else if constexpr (Q < R - 1) {
      sched_interleave<kSchedDsRead, D, MQ>();
      db_before_barrier<Q + 1>();
    } else {
      sched_interleave<kSchedDsWrite, W, MQ / 2>();
    }
  }
  // After the barrier: the first reads of tile l+1, then the rest of tile l's last round.
  static __device__ __forceinline__ void db_after_barrier() {
    sched_group<kSchedDsRead, D>();
    sched_group<kSchedMfma, MQ - MQ / 2>();
  }
  // Rounds whose MFMAs each carry the LDS reads of the following round.
  template <int Q = 0>
  static __device__ __forceinline__ void rounds_with_reads() {
    if constexpr (Q < R - 1) {
      sched_interleave<kSchedDsRead, D, MQ>();
      rounds_with_reads<Q + 1>();
    }
  }
};

// ------------------------------------------------------------------------------------
// The K-loop.  GUARD = false is taken by workgroups whose whole tile lies inside the
// matrices, with 16-byte-aligned rows and K a multiple of BK: every copy is unguarded.
// GUARD = true picks per K tile between the unguarded and the element-guarded copy.
// ------------------------------------------------------------------------------------
template <class C>
struct LoopArgs {
  const float* A;
  const float* B;
  int64_t lda, ldb;
  int M, N, K, m0, n0;
  bool vec_a, vec_b;
};

template <class C, bool GUARD>
__device__ inline void load_tile_a(TileCopy<C>& cp, const LoopArgs<C>& g, int kt) {
  const int k0 = kt * C::BK;
  if (!GUARD || (g.vec_a && k0 + C::BK <= g.K))
    cp.load_a_fast(g.A, g.lda, g.m0, k0);
  else
    cp.load_a_guarded(g.A, g.lda, g.M, g.K, g.m0, k0);
}

template <class C, bool GUARD>
__device__ inline void load_tile_b(TileCopy<C>& cp, const LoopArgs<C>& g, int kt) {
  const int k0 = kt * C::BK;
  if (!GUARD || (g.vec_b && k0 + C::BK <= g.K))
    cp.load_b_fast(g.B, g.ldb, g.n0, k0);
  else
    cp.load_b_guarded(g.B, g.ldb, g.N, g.K, g.n0, k0);
}

template <class C, bool GUARD>
__device__ inline void load_tile(TileCopy<C>& cp, const LoopArgs<C>& g, int kt) {
  load_tile_a<C, GUARD>(cp, g, kt);
  load_tile_b<C, GUARD>(cp, g, kt);
}

// Double-buffered: two LDS slots, tile l+1 copied into the idle slot while tile l is
// multiplied, ONE barrier per K tile.  The loop is rotated so that the barrier sits at
// the hand-off between slots: after this wave has written tile l+1 into the idle slot and
// before anybody reads it.  That single barrier is at once "tile l+1 has landed" and
// "nobody still reads the slot that tile l+2 will overwrite" (all reads of tile l are
// already in registers by then).  LDS fragments are read one round ahead of the MFMAs,
// and the second half of tile l's last round runs after the barrier, covering the
// latency of the first reads of tile l+1.  Barriers per product: 1 (prologue) +
// (k_tiles - 1) = k_tiles, the same count as a barrier at the top of every iteration.
// One steady-state step of the double-buffered loop: copy tile l+1 towards the idle slot
// `nxt` while multiplying the tile in `cur`, one barrier at the hand-off.  On entry f[0]
// holds round 0 of the current tile; on exit it holds round 0 of tile l+1.
template <class C, bool GUARD>
__device__ __forceinline__ void db_step(const float* cur, float* nxt, TileCopy<C>& cp,
                                        const LaneView<C>& lv, const LoopArgs<C>& g, int l,
                                        Frag<C> (&f)[2], floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  load_tile<C, GUARD>(cp, g, l + 1);  // in flight during the MFMAs below
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 1>(f[1], acc);
  cp.store(nxt);
  if constexpr (!GUARD) Sched<C>::template db_before_barrier<0>();
  __syncthreads();
  read_frag(nxt, lv, 0, f[0]);
  mfma_round<C, 2>(f[1], acc);
  if constexpr (!GUARD) Sched<C>::db_after_barrier();
}

// Double-buffered: two LDS slots, tile l+1 copied into the idle slot while tile l is
// multiplied, ONE barrier per K tile.  The loop is rotated so that the barrier sits at
// the hand-off between slots: after this wave has written tile l+1 into the idle slot and
// before anybody reads it.  That single barrier is at once "tile l+1 has landed" and
// "nobody still reads the slot that tile l+2 will overwrite" (all reads of tile l are
// already in registers by then).  LDS fragments are read one round ahead of the MFMAs,
// and the second half of tile l's last round runs after the barrier, covering the
// latency of the first reads of tile l+1.  Barriers per product: 1 (prologue) +
// (k_tiles - 1) = k_tiles, the same count as a barrier at the top of every iteration.
// Where registers allow (DB_UNROLL) the loop body holds two steps (slot 0 -> 1, then slot
// 1 -> 0), so both slot addresses are fixed in each step instead of being recomputed from
// the tile parity.
template <class C, bool GUARD>
__device__ inline void k_loop_db(float* smem, TileCopy<C>& cp, const LaneView<C>& lv,
                                 const LoopArgs<C>& g, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  Frag<C> f[2];
  float* const s0 = smem;
  float* const s1 = smem + C::SLOT;
  load_tile<C, GUARD>(cp, g, 0);  // prologue: tile 0 into slot 0
  cp.store(s0);
  __syncthreads();
  read_frag(s0, lv, 0, f[0]);
  int l = 0;
  if constexpr (C::DB_UNROLL) {
    for (; l + 2 < k_tiles; l += 2) {
      db_step<C, GUARD>(s0, s1, cp, lv, g, l, f, acc);
      db_step<C, GUARD>(s1, s0, cp, lv, g, l + 1, f, acc);
    }
  }
  for (; l + 1 < k_tiles; ++l)
    db_step<C, GUARD>((l & 1) ? s1 : s0, (l & 1) ? s0 : s1, cp, lv, g, l, f, acc);
  // Last tile (l == k_tiles - 1): nothing left to prefetch.
  const float* cur = (l & 1) ? s1 : s0;
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 0>(f[1], acc);
}

// Single-buffered: one LDS slot; per K tile: copy -> barrier -> multiply -> barrier.
// The second barrier comes as soon as this wave's last LDS read of the tile has returned
// (the last round's MFMAs run after it on registers).
// SPLIT = true is the same loop with the A and B copies published by separate barriers,
// copy A -> barrier -> copy B -> barrier -> multiply -> barrier: three barriers per K tile,
// the arrangement the LuisaCompute note measured before it coalesced the two copy fences
// ("Dependence-aware group synchronization on M1 Max", section "Transformation and safety
// boundary").  It exists to measure what one barrier per K tile costs on this hardware.
template <class C, bool GUARD, bool SPLIT = false>
__device__ inline void k_loop_sb(float* smem, TileCopy<C>& cp, const LaneView<C>& lv,
                                 const LoopArgs<C>& g, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  Frag<C> f[2];
  for (int l = 0; l < k_tiles; ++l) {
    if constexpr (SPLIT) {
      load_tile_a<C, GUARD>(cp, g, l);
      cp.store_a(smem);
      __syncthreads();  // the A tile is in LDS
      load_tile_b<C, GUARD>(cp, g, l);
      cp.store_b(smem);
    } else {
      load_tile<C, GUARD>(cp, g, l);
      cp.store(smem);
    }
    __syncthreads();  // tile l is in LDS
    read_frag(smem, lv, 0, f[0]);
#pragma unroll
    for (int q = 0; q + 1 < R; ++q) {
      read_frag(smem, lv, q + 1, f[(q + 1) & 1]);
      mfma_round<C, 0>(f[q & 1], acc);
    }
    if constexpr (!GUARD) {
      sched_group<kSchedDsRead, Sched<C>::D>();
      Sched<C>::template rounds_with_reads<0>();
    }
    __syncthreads();  // every wave has read tile l: the slot may be overwritten
    mfma_round<C, 0>(f[1], acc);
  }
}

// ------------------------------------------------------------------------------------
// The kernel with register-staged copies.  LOOP (the variant id of the C ABI):
//   1 single-buffered: one slot, two barriers per K tile
//   2 double-buffered: two slots, one barrier per K tile
//   4 single-buffered with split copy barriers: one slot, three barriers per K tile
// ------------------------------------------------------------------------------------
enum : int { kLoopSB = 1, kLoopDB = 2, kLoopSB3 = 4 };

template <class C, int LOOP>
__global__ void __launch_bounds__(C::NT)
gemm_f32_tile_kernel(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                     const float* __restrict__ B, int64_t ldb, float* __restrict__ Cmat,
                     int64_t ldc, int flags, int k_chunk, int64_t c_split_stride) {
  // Split-K: workgroup row y of the grid multiplies K range [y*k_chunk, y*k_chunk + k_chunk)
  // into its own M x N partial product at Cmat + y*c_split_stride.
  if (gridDim.y > 1) {
    const int kb = blockIdx.y * k_chunk;
    K = min(K - kb, k_chunk);
    A += kb;
    B += (int64_t)kb * ldb;
    Cmat += (int64_t)blockIdx.y * c_split_stride;
  }
  static_assert((C::BK / 8) % 2 == 0, "BK/8 rounds must be even for the fragment ping-pong");
  static_assert(LOOP == kLoopSB || LOOP == kLoopDB || LOOP == kLoopSB3, "loop kind");
  constexpr bool DB = LOOP == kLoopDB;
  constexpr bool SPLIT = LOOP == kLoopSB3;
  __shared__ __attribute__((aligned(16))) float smem[(DB ? 2 : 1) * C::SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;

  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, flags, tm, tn);
  LoopArgs<C> g;
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.m0 = tm * C::BM;
  g.n0 = tn * C::BN;
  const bool m_full = g.m0 + C::BM <= M;
  const bool n_full = g.n0 + C::BN <= N;
  g.vec_a = (flags & kVecA) && m_full;
  g.vec_b = (flags & kVecB) && n_full;

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

  TileCopy<C> cp;
  cp.init(tid);
  LaneView<C> lv;
  lv.init(wm, wn, lane);
  const int k_tiles = (K + C::BK - 1) / C::BK;
  if (k_tiles > 0) {
    const bool unguarded = g.vec_a && g.vec_b && (K % C::BK) == 0;
    if constexpr (DB) {
      if (unguarded)
        k_loop_db<C, false>(smem, cp, lv, g, k_tiles, acc);
      else
        k_loop_db<C, true>(smem, cp, lv, g, k_tiles, acc);
    } else {
      if (unguarded)
        k_loop_sb<C, false, SPLIT>(smem, cp, lv, g, k_tiles, acc);
      else
        k_loop_sb<C, true, SPLIT>(smem, cp, lv, g, k_tiles, acc);
    }
  }

  // Epilogue: C is written once, never read.  Lanes 0-31 of a store cover 32 consecutive
  // columns of one row and lanes 32-63 the same columns four rows further down.
  const int row0 = g.m0 + wm * C::TM + 4 * (lane >> 5);
  const int col0 = g.n0 + wn * C::TN + (lane & 31);
  if (m_full && n_full) {
    float* cbase = Cmat + (int64_t)row0 * ldc + col0;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cbase[(int64_t)(fm * 32 + 8 * (r >> 2) + (r & 3)) * ldc + fn * 32] = acc[fm][fn][r];
  } else {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + fm * 32 + 8 * (r >> 2) + (r & 3);
          const int col = col0 + fn * 32;
          if (row < M && col < N) Cmat[(int64_t)row * ldc + col] = acc[fm][fn][r];
        }
  }
}

// ------------------------------------------------------------------------------------
// Multi-stage variant (MS): S LDS stages filled by gfx950 direct-to-LDS loads.
//
// The glossary page ("Double Buffering", second paragraph and the figure caption) notes
// that its platform lost its asynchronous copy engine, so its double buffering overlaps
// copies and math only through instruction-level parallelism, and it names the CUDA
// analogue: a multi-stage asynchronous-copy pipeline.  gfx950 has the asynchronous copy:
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight into LDS
// (lane L's bytes land at M0 + 16*L), with no registers in between and completion
// tracked by vmcnt.  Tiles l+1 .. l+S-1 are in flight while tile l is multiplied.
//
// LDS layout of a stage (no padding; XOR swizzle at 16-byte-chunk granularity):
//   A part: BM rows of BK floats;  chunk c of row r is stored at chunk c ^ swz_a(r)
//   B part: BK rows of BN floats;  chunk c of row k is stored at chunk c ^ swz_b(k)
// A wave's copy instruction always fills 1 KiB of consecutive LDS; each lane chooses the
// global chunk that belongs at its position, so the swizzle costs nothing on the copy
// side and makes the fragment reads conflict-free: the 16 lanes of a 16-byte read (16
// consecutive rows, one logical chunk) hit 16 distinct bank groups, and the two
// half-waves of a B read (rows k and k+4) fall on opposite halves of the 64 banks.
//
// The compiler's own wait insertion cannot tell one stage from another and would wait
// for every outstanding copy before any LDS read, so the copies are issued from inline
// assembly and their completion is waited for explicitly, per tile.
// ------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) float lds_float;

template <class C, int S>
struct MsCfg {
  static constexpr int STAGES = S;
  static constexpr int A_FLOATS = C::BM * C::BK;
  static constexpr int B_FLOATS = C::BK * C::BN;
  static constexpr int STAGE = A_FLOATS + B_FLOATS;  // floats per stage
  static constexpr int A_CHUNKS = A_FLOATS / 256;    // 1 KiB copy instructions, A part
  static constexpr int B_CHUNKS = B_FLOATS / 256;
  static constexpr int WAVES = C::NT / 64;
  static constexpr int D = (A_CHUNKS + B_CHUNKS) / WAVES;  // copies per wave per tile
  static constexpr int CPR_A = C::BK / 4;            // 16-byte chunks per A row
  static constexpr int RPC_A = 256 / C::BK;          // A rows per 1 KiB
  static constexpr int CPR_B = C::BN / 4;
  static constexpr int RPC_B = 256 / C::BN;
  // LDS floats: the stages, or the two padded slots of the guarded fallback loop.
  static constexpr int LDS_FLOATS = S * STAGE > 2 * C::SLOT ? S * STAGE : 2 * C::SLOT;
  static_assert(S >= 2, "at least two stages");
  static_assert(C::BK == 16 || C::BK == 32 || C::BK == 64, "swizzle period");
  static_assert(C::BN % 64 == 0, "B swizzle flips chunk bit 3 inside 16-chunk groups");
  static_assert(A_FLOATS % 256 == 0 && B_FLOATS % 256 == 0, "whole 1 KiB copies");
  static_assert((A_CHUNKS + B_CHUNKS) % WAVES == 0, "copies divide among waves");
  static_assert(D * (S - 2) <= 63, "vmcnt range");
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS of one CU");
};

template <class C>
__device__ __forceinline__ int swz_a(int row) {
  return (row / (64 / C::BK)) % (C::BK / 4);
}
__device__ __forceinline__ int swz_b(int k) { return ((k >> 2) & 1) << 3; }

template <class C, int S>
struct MsCopy {
  using MC = MsCfg<C, S>;
  const float* ptr[MC::D];  // this lane's source for tile 0
  int64_t step[MC::D];      // floats between consecutive K tiles
  uint32_t lds_off[MC::D];  // byte offset of the wave's 1 KiB inside a stage
  uint32_t lds_base;        // LDS byte address of stage 0

  __device__ inline void init(const float* smem, int wave, int lane, const float* A,
                              int64_t lda, const float* B, int64_t ldb, int m0, int n0) {
    lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_float*)smem);
#pragma unroll
    for (int i = 0; i < MC::D; ++i) {
      const int j = wave + i * MC::WAVES;  // which 1 KiB of the stage this copy fills
      if (j < MC::A_CHUNKS) {
        const int row = j * MC::RPC_A + lane / MC::CPR_A;
        const int c = (lane % MC::CPR_A) ^ swz_a<C>(row);
        ptr[i] = A + (int64_t)(m0 + row) * lda + 4 * c;
        step[i] = C::BK;
        lds_off[i] = (uint32_t)j * 1024u;
      } else {
        const int jb = j - MC::A_CHUNKS;
        const int k = jb * MC::RPC_B + lane / MC::CPR_B;
        const int c = (lane % MC::CPR_B) ^ swz_b(k);
        ptr[i] = B + (int64_t)k * ldb + n0 + 4 * c;
        step[i] = (int64_t)C::BK * ldb;
        lds_off[i] = (uint32_t)(MC::A_FLOATS * 4 + jb * 1024);
      }
    }
  }

  // Start the copy of K tile kt into stage st (asynchronous; counted by vmcnt).
  __device__ inline void issue(int kt, int st) const {
    const uint32_t stage_base = lds_base + (uint32_t)st * (uint32_t)(MC::STAGE * 4);
#pragma unroll
    for (int i = 0; i < MC::D; ++i) {
      const float* src = ptr[i] + (int64_t)kt * step[i];
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(stage_base + lds_off[i]);
      // M0 is reserved by the compiler, which warns about clobbering it.  Nothing else in
      // these kernels uses M0 (a structural test checks that every M0 write is one of these
      // copies, immediately followed by its load), so the clobber is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :
                   : "v"(src), "s"(m0v)
                   : "memory", "m0");
#pragma clang diagnostic pop
    }
  }
};

// Wait until at most N copies of this wave are outstanding and this wave's LDS reads have
// returned.
template <int N>
__device__ __forceinline__ void ms_wait() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" : : "n"(N) : "memory");
}

// Wait until tile l+1 has landed in this wave's copies (the S-2 tiles issued after it may
// stay in flight) and this wave's LDS reads have returned, then barrier.
template <class C, int S>
__device__ __forceinline__ void ms_wait_tile_barrier() {
  ms_wait<MsCfg<C, S>::D * (S - 2)>();
  asm volatile("s_barrier" : : : "memory");
}

template <class C, int S>
struct LaneViewMs {
  int a_off;          // float offset of this lane's A row (fm = 0) inside a stage
  int a_x;            // h ^ swz_a(row): logical chunk 2q+h of the row is at (2q) ^ a_x
  int b_off[C::FN];   // float offset of B[4h][col(fn)] inside a stage (swizzled)

  __device__ inline void init(int wm, int wn, int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    const int row = wm * C::TM + l32;
    a_off = row * C::BK;
    a_x = h ^ swz_a<C>(row);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int col = wn * C::TN + fn * 32 + l32;
      const int k = 4 * h;
      b_off[fn] = MsCfg<C, S>::A_FLOATS + k * C::BN + 4 * ((col >> 2) ^ swz_b(k)) + (col & 3);
    }
  }
};

template <class C, int S>
__device__ inline void read_frag_ms(const float* stage, const LaneViewMs<C, S>& lv, int q,
                                    Frag<C>& f) {
  const float* a_ptr = stage + lv.a_off + 4 * ((2 * q) ^ lv.a_x);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
    f.a[fm] = *reinterpret_cast<const floatx4*>(a_ptr + fm * 32 * C::BK);
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
    for (int t = 0; t < 4; ++t) f.b[fn][t] = stage[lv.b_off[fn] + (8 * q + t) * C::BN];
}

// One steady-state step of the MS loop for tile l held in stage `st`: start the copy of
// tile l+S-1 into the stage that tile l-1 used, multiply tile l, and -- at the hand-off,
// before the second half of tile l's last round -- wait for tile l+1 and pass ONE
// barrier.  That barrier makes tile l+1 visible to every wave and certifies that every
// wave has finished reading tile l, whose stage the copy issued in the next step
// overwrites.  Near the end the copy index is clamped to the last tile (a harmless
// duplicate into a stage no later tile uses), so every wait keeps S-2 tiles in flight.
template <class C, int S>
__device__ __forceinline__ void ms_step(const float* smem, const MsCopy<C, S>& cp,
                                        const LaneViewMs<C, S>& lv, int l, int k_tiles,
                                        int st, Frag<C> (&f)[2],
                                        floatx16 (&acc)[C::FM][C::FN]) {
  using MC = MsCfg<C, S>;
  constexpr int R = C::BK / 8;
  cp.issue(min(l + S - 1, k_tiles - 1), st == 0 ? S - 1 : st - 1);
  const float* cur = smem + st * MC::STAGE;
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag_ms(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 1>(f[1], acc);
  Sched<C>::template rounds_with_reads<0>();
  sched_group<kSchedMfma, Sched<C>::MQ / 2>();
  ms_wait_tile_barrier<C, S>();
  read_frag_ms(smem + (st + 1 == S ? 0 : st + 1) * MC::STAGE, lv, 0, f[0]);
  mfma_round<C, 2>(f[1], acc);
  Sched<C>::db_after_barrier();
}

// The MS K-loop: prologue (tiles 0 .. S-2 in flight, tile 0 landed), steps unrolled S at a
// time so that every stage address is fixed, the remaining steps one by one, and the
// last tile (nothing left to copy) peeled off.
template <class C, int S>
__device__ inline void k_loop_ms(float* smem, const MsCopy<C, S>& cp,
                                 const LaneViewMs<C, S>& lv, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN]) {
  using MC = MsCfg<C, S>;
  constexpr int R = C::BK / 8;
#pragma unroll
  for (int t = 0; t < S - 1; ++t) cp.issue(min(t, k_tiles - 1), t);
  ms_wait_tile_barrier<C, S>();
  Frag<C> f[2];
  read_frag_ms(smem, lv, 0, f[0]);
  int l = 0;
  for (; l + S < k_tiles; l += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) ms_step<C, S>(smem, cp, lv, l + u, k_tiles, u, f, acc);
  }
  for (; l + 1 < k_tiles; ++l) ms_step<C, S>(smem, cp, lv, l, k_tiles, l % S, f, acc);
  const float* cur = smem + (l % S) * MC::STAGE;  // last tile: nothing left to copy
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag_ms(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 0>(f[1], acc);
}

template <class C, int S>
__global__ void __launch_bounds__(C::NT)
gemm_f32_ms_kernel(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                   const float* __restrict__ B, int64_t ldb, float* __restrict__ Cmat,
                   int64_t ldc, int flags, int k_chunk, int64_t c_split_stride) {
  // Split-K: workgroup row y of the grid multiplies K range [y*k_chunk, y*k_chunk + k_chunk)
  // into its own M x N partial product at Cmat + y*c_split_stride.
  if (gridDim.y > 1) {
    const int kb = blockIdx.y * k_chunk;
    K = min(K - kb, k_chunk);
    A += kb;
    B += (int64_t)kb * ldb;
    Cmat += (int64_t)blockIdx.y * c_split_stride;
  }
  using MC = MsCfg<C, S>;
  __shared__ __attribute__((aligned(1024))) float smem[MC::LDS_FLOATS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N;
  const int wn = wave % C::WAVES_N;
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, flags, tm, tn);
  LoopArgs<C> g;
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.m0 = tm * C::BM;
  g.n0 = tn * C::BN;
  const bool m_full = g.m0 + C::BM <= M;
  const bool n_full = g.n0 + C::BN <= N;
  g.vec_a = (flags & kVecA) && m_full;
  g.vec_b = (flags & kVecB) && n_full;

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

  const int k_tiles = (K + C::BK - 1) / C::BK;
  if (k_tiles > 0) {
    if (g.vec_a && g.vec_b && (K % C::BK) == 0) {
      MsCopy<C, S> cp;
      cp.init(smem, wave, lane, A, lda, B, ldb, g.m0, g.n0);
      LaneViewMs<C, S> lv;
      lv.init(wm, wn, lane);
      k_loop_ms<C, S>(smem, cp, lv, k_tiles, acc);
    } else {
      // Edge, misaligned or K-ragged tiles: the guarded double-buffered loop.
      TileCopy<C> cp;
      cp.init(tid);
      LaneView<C> lv;
      lv.init(wm, wn, lane);
      k_loop_db<C, true>(smem, cp, lv, g, k_tiles, acc);
    }
  }

  const int row0 = g.m0 + wm * C::TM + 4 * (lane >> 5);
  const int col0 = g.n0 + wn * C::TN + (lane & 31);
  if (m_full && n_full) {
    float* cbase = Cmat + (int64_t)row0 * ldc + col0;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          cbase[(int64_t)(fm * 32 + 8 * (r >> 2) + (r & 3)) * ldc + fn * 32] = acc[fm][fn][r];
  } else {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + fm * 32 + 8 * (r >> 2) + (r & 3);
          const int col = col0 + fn * 32;
          if (row < M && col < N) Cmat[(int64_t)row * ldc + col] = acc[fm][fn][r];
        }
  }
}

// Stage count per configuration: as many as fit (at most 4) in the 160 KiB of a CU.
template <class C>
constexpr int ms_stages() {
  constexpr int stage_bytes = 4 * (C::BM * C::BK + C::BK * C::BN);
  return (160 * 1024) / stage_bytes >= 4 ? 4 : (160 * 1024) / stage_bytes;
}

// ------------------------------------------------------------------------------------
// Split-K reduction: C[i][j] = P[0][i][j] + P[1][i][j] + ... + P[S-1][i][j], summed in
// that fixed order, so a split product is deterministic.  P holds S partial products of
// M x N floats each, rows of N.  A streaming kernel bounded by HBM bandwidth:
// (S + 1) * 4 * M * N bytes per launch.  VEC: rows of P and C are 16-byte aligned and
// N % 4 == 0, so each thread moves 4 consecutive columns.
// ------------------------------------------------------------------------------------
template <bool VEC>
__global__ void __launch_bounds__(256)
gemm_f32_splitk_reduce(int M, int N, int S, const float* __restrict__ P,
                       float* __restrict__ C, int64_t ldc) {
  const int64_t mn = (int64_t)M * N;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if constexpr (VEC) {
    const int n4 = N / 4;
    const int64_t total = (int64_t)M * n4;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += stride) {
      const int64_t i = t / n4;
      const int64_t j = 4 * (t - i * n4);
      const int64_t e = i * N + j;
      floatx4 acc = *reinterpret_cast<const floatx4*>(P + e);
      for (int sp = 1; sp < S; ++sp) acc += *reinterpret_cast<const floatx4*>(P + sp * mn + e);
      *reinterpret_cast<floatx4*>(C + i * ldc + j) = acc;
    }
  } else {
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < mn; e += stride) {
      const int64_t i = e / N;
      const int64_t j = e - i * N;
      float acc = P[e];
      for (int sp = 1; sp < S; ++sp) acc += P[sp * mn + e];
      C[i * ldc + j] = acc;
    }
  }
}

// ------------------------------------------------------------------------------------
// Configuration table.  Ids are part of the ABI (gemm_f32_ex, gemm_f32_config_info).
// ------------------------------------------------------------------------------------
using Cfg0 = TileCfg<256, 256, 16, 2, 2>;  // wave 128x128 (16 blocks)
using Cfg1 = TileCfg<256, 256, 32, 2, 2>;  // wave 128x128, deeper K tile
using Cfg2 = TileCfg<256, 128, 16, 2, 2>;  // wave 128x64
using Cfg3 = TileCfg<128, 128, 16, 2, 2>;  // wave 64x64
using Cfg4 = TileCfg<128, 128, 32, 2, 2>;  // wave 64x64, deeper K tile
using Cfg5 = TileCfg<128, 64, 32, 2, 2>;   // wave 64x32
using Cfg6 = TileCfg<64, 64, 32, 2, 2>;    // wave 32x32
using Cfg7 = TileCfg<64, 64, 64, 2, 2>;    // wave 32x32, deeper K tile
using Cfg8 = TileCfg<256, 256, 32, 2, 4>;  // 8 waves of 128x64: two waves per SIMD
using Cfg9 = TileCfg<128, 256, 32, 2, 4>;  // 8 waves of 64x64
using Cfg10 = TileCfg<32, 128, 32, 1, 4>;  // 4 waves of 32x32 side by side: skinny M

typedef void (*KernelFn)(int, int, int, const float*, int64_t, const float*, int64_t, float*,
                         int64_t, int, int, int64_t);

struct CfgEntry {
  int bm, bn, bk, nt;
  int lds_sb, lds_db;
  int ms_stages, lds_ms;
  KernelFn sb, db, ms, sb3;
};

template <class C>
constexpr CfgEntry make_entry() {
  constexpr int S = ms_stages<C>();
  return CfgEntry{C::BM,
                  C::BN,
                  C::BK,
                  C::NT,
                  (int)(C::SLOT * sizeof(float)),
                  (int)(2 * C::SLOT * sizeof(float)),
                  S,
                  (int)(MsCfg<C, S>::LDS_FLOATS * sizeof(float)),
                  &gemm_f32_tile_kernel<C, kLoopSB>,
                  &gemm_f32_tile_kernel<C, kLoopDB>,
                  &gemm_f32_ms_kernel<C, S>,
                  &gemm_f32_tile_kernel<C, kLoopSB3>};
}

static const CfgEntry kConfigs[] = {
    make_entry<Cfg0>(), make_entry<Cfg1>(), make_entry<Cfg2>(), make_entry<Cfg3>(),
    make_entry<Cfg4>(), make_entry<Cfg5>(), make_entry<Cfg6>(), make_entry<Cfg7>(),
    make_entry<Cfg8>(), make_entry<Cfg9>(), make_entry<Cfg10>(),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

}  // namespace gemmf32

#include "dispatch_table.h"

namespace gemmf32 {

// ------------------------------------------------------------------------------------
// Host side: validation, dispatch, launch.
// ------------------------------------------------------------------------------------
static thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = 2147483647LL - 1024;  // keeps tile-end arithmetic in int32

static int validate(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                    const float* B, int64_t ldb, const float* C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  const int64_t min_lda = K > 1 ? K : 1;
  const int64_t min_ldb = N > 1 ? N : 1;
  if (lda < min_lda || ldb < min_ldb || ldc < min_ldb) return GEMMF32_ERR_BAD_LD;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMMF32_ERR_TOO_LARGE;
  if (lda > kMaxDim * 64 || ldb > kMaxDim * 64 || ldc > kMaxDim * 64)
    return GEMMF32_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return GEMMF32_OK;
  if (C == nullptr) return GEMMF32_ERR_NULL_PTR;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMMF32_ERR_NULL_PTR;
  if (((uintptr_t)C & 3u) != 0) return GEMMF32_ERR_MISALIGNED;
  if (K > 0 && ((((uintptr_t)A) & 3u) != 0 || (((uintptr_t)B) & 3u) != 0))
    return GEMMF32_ERR_MISALIGNED;
  // Byte extents [begin, end) of the three operands; C must be disjoint from A and B.
  const uintptr_t c0 = (uintptr_t)C;
  const uintptr_t c1 = c0 + (uintptr_t)(((M - 1) * ldc + N) * 4);
  if (K > 0) {
    const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)(((M - 1) * lda + K) * 4);
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)(((K - 1) * ldb + N) * 4);
    if (c0 < a1 && a0 < c1) return GEMMF32_ERR_ALIAS;
    if (c0 < b1 && b0 < c1) return GEMMF32_ERR_ALIAS;
  }
  return GEMMF32_OK;
}

// GEMMF32_RASTER=<group_m>[,noxcd] changes the workgroup order of every launch (for
// measurement); group_m in 1..255.
static int env_raster_flags() {
  const char* v = std::getenv("GEMMF32_RASTER");
  if (v == nullptr || *v == 0) return 0;
  char* end = nullptr;
  long gm = std::strtol(v, &end, 10);
  int flags = 0;
  if (gm >= 1 && gm <= 255) flags |= (int)gm << kRasterGroupShift;
  if (end && std::strstr(end, "noxcd")) flags |= kRasterNoXcdRemap;
  return flags;
}

// One launch of a GEMM kernel.  splits > 1: grid rows y = 0..splits-1 each multiply the
// K range [y*k_chunk, ...) into C + y*c_split_stride (the split-K partial products).
static int launch(int variant, int cfg_id, int64_t M, int64_t N, int64_t K, const float* A,
                  int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                  void* stream, int splits = 1, int k_chunk = 0, int64_t c_split_stride = 0) {
  const CfgEntry& e = kConfigs[cfg_id];
  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
  if (tiles * e.nt > 0xFFFFFFFFLL) return GEMMF32_ERR_TOO_LARGE;
  int flags = 0;
  if (K > 0 && (((uintptr_t)A) & 15u) == 0 && (lda & 3) == 0) flags |= kVecA;
  if (K > 0 && (((uintptr_t)B) & 15u) == 0 && (ldb & 3) == 0) flags |= kVecB;
  flags |= env_raster_flags();
  int m = (int)M, n = (int)N, k = (int)K;
  int kc = splits > 1 ? k_chunk : k;
  void* args[] = {&m,   &n,     &k,  (void*)&A, &lda, (void*)&B,
                  &ldb, &C,     &ldc, &flags,   &kc,  &c_split_stride};
  KernelFn fn = variant == GEMMF32_VARIANT_SB    ? e.sb
                : variant == GEMMF32_VARIANT_MS  ? e.ms
                : variant == GEMMF32_VARIANT_SB3 ? e.sb3
                                                 : e.db;
  hipError_t err = hipLaunchKernel((const void*)fn, dim3((unsigned)tiles, (unsigned)splits),
                                   dim3(e.nt), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return GEMMF32_ERR_HIP;
  }
  return GEMMF32_OK;
}

static int env_variant() {
  const char* v = std::getenv("GEMMF32_VARIANT");
  if (v == nullptr) return GEMMF32_VARIANT_AUTO;
  if (std::strcmp(v, "sb") == 0) return GEMMF32_VARIANT_SB;
  if (std::strcmp(v, "db") == 0) return GEMMF32_VARIANT_DB;
  if (std::strcmp(v, "ms") == 0) return GEMMF32_VARIANT_MS;
  return GEMMF32_VARIANT_AUTO;
}

static int run(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
               int64_t ldb, float* C, int64_t ldc, int variant, int cfg_id, void* stream) {
  if (variant != GEMMF32_VARIANT_AUTO && variant != GEMMF32_VARIANT_SB &&
      variant != GEMMF32_VARIANT_DB && variant != GEMMF32_VARIANT_MS &&
      variant != GEMMF32_VARIANT_SB3)
    return GEMMF32_ERR_BAD_CONFIG;
  if (cfg_id < -1 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  int rc = validate(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != GEMMF32_OK) return rc;
  if (M == 0 || N == 0) return GEMMF32_OK;
  if (variant == GEMMF32_VARIANT_AUTO) {
    int v = 0, c = 0;
    select_shape(M, N, K, &v, &c);
    variant = v;
    if (cfg_id < 0) cfg_id = c;
  } else if (cfg_id < 0) {
    cfg_id = select_for_variant(M, N, K, variant == GEMMF32_VARIANT_SB3 ? GEMMF32_VARIANT_SB
                                                                        : variant);
  }
  return launch(variant, cfg_id, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

constexpr int kMaxSplits = 64;
constexpr int kSplitGranule = 64;  // K chunks are whole K tiles of every configuration

// K chunk of one split and the number of splits actually used.
static void splitk_plan(int64_t K, int splits, int64_t* k_chunk, int* used) {
  int64_t kc = (K + splits - 1) / splits;
  kc = (kc + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  if (kc < kSplitGranule) kc = kSplitGranule;
  *k_chunk = kc;
  *used = (int)((K + kc - 1) / kc);
}

static int run_splitk(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                      const float* B, int64_t ldb, float* C, int64_t ldc, int splits,
                      float* ws, int64_t ws_floats, void* stream) {
  if (splits == 0 && M >= 0 && N >= 0 && K >= 0) splits = select_splits(M, N, K);
  if (splits < 1 || splits > kMaxSplits) return GEMMF32_ERR_BAD_CONFIG;
  int rc = validate(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != GEMMF32_OK) return rc;
  if (M == 0 || N == 0) return GEMMF32_OK;
  int64_t kc = 0;
  int used = 1;
  if (K > 0) splitk_plan(K, splits, &kc, &used);
  if (used <= 1) return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_AUTO, -1, stream);
  const int64_t need = (int64_t)used * M * N;
  if (ws == nullptr) return GEMMF32_ERR_NULL_PTR;
  if (((uintptr_t)ws & 3u) != 0) return GEMMF32_ERR_MISALIGNED;
  if (ws_floats < need) return GEMMF32_ERR_BAD_LD;
  // The workspace must not overlap A, B or C.
  const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + (uintptr_t)(need * 4);
  const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)(((M - 1) * lda + K) * 4);
  const uintptr_t b0 = (uintptr_t)B, b1 = b0 + (uintptr_t)(((K - 1) * ldb + N) * 4);
  const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)(((M - 1) * ldc + N) * 4);
  if ((w0 < a1 && a0 < w1) || (w0 < b1 && b0 < w1) || (w0 < c1 && c0 < w1))
    return GEMMF32_ERR_ALIAS;
  int v = 0, cfg = 0;
  select_shape(M, N, kc, &v, &cfg);
  rc = launch(v, cfg, M, N, K, A, lda, B, ldb, ws, N, stream, used, (int)kc, M * N);
  if (rc != GEMMF32_OK) return rc;
  const bool vec = (N % 4) == 0 && (ldc % 4) == 0 && ((uintptr_t)ws & 15u) == 0 &&
                   ((uintptr_t)C & 15u) == 0;
  const int64_t items = vec ? M * (N / 4) : M * N;
  const int64_t blocks64 = (items + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 4096 ? blocks64 : 4096);
  int m = (int)M, n = (int)N;
  const float* p = ws;
  void* args[] = {&m, &n, &used, (void*)&p, &C, &ldc};
  const void* fn = vec ? (const void*)&gemm_f32_splitk_reduce<true>
                       : (const void*)&gemm_f32_splitk_reduce<false>;
  hipError_t err = hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return GEMMF32_ERR_HIP;
  }
  return GEMMF32_OK;
}

}  // namespace gemmf32

using namespace gemmf32;

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
             int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, env_variant(), -1, stream);
}

int gemm_f32_sb(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_SB, -1, stream);
}

int gemm_f32_db(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_DB, -1, stream);
}

int gemm_f32_ms(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_MS, -1, stream);
}

int gemm_f32_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, int variant, int cfg_id, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, variant, cfg_id, stream);
}

int gemm_f32_splitk(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                    const float* B, int64_t ldb, float* C, int64_t ldc, int splits,
                    float* workspace, int64_t workspace_floats, void* stream) {
  return run_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_floats,
                    stream);
}

int gemm_f32_splitk_select(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  return select_splits(M, N, K);
}

int64_t gemm_f32_splitk_workspace(int64_t M, int64_t N, int64_t K, int splits) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  if (splits == 0) splits = select_splits(M, N, K);
  if (splits < 1 || splits > kMaxSplits) return GEMMF32_ERR_BAD_CONFIG;
  if (M == 0 || N == 0 || K == 0) return 0;
  int64_t kc = 0;
  int used = 1;
  splitk_plan(K, splits, &kc, &used);
  return used <= 1 ? 0 : (int64_t)used * M * N;
}

int gemm_f32_select(int64_t M, int64_t N, int64_t K, int* variant, int* cfg_id) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  int v = 0, c = 0;
  select_shape(M, N, K, &v, &c);
  if (variant) *variant = v;
  if (cfg_id) *cfg_id = c;
  return GEMMF32_OK;
}

int gemm_f32_select_cfg(int64_t M, int64_t N, int64_t K, int variant) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  if (variant != GEMMF32_VARIANT_SB && variant != GEMMF32_VARIANT_DB &&
      variant != GEMMF32_VARIANT_MS)
    return GEMMF32_ERR_BAD_CONFIG;
  return select_for_variant(M, N, K, variant);
}

int gemm_f32_num_configs(void) { return kNumConfigs; }

int gemm_f32_config_info(int cfg_id, int* BM, int* BN, int* BK, int* threads, int* lds_sb,
                         int* lds_db) {
  if (cfg_id < 0 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  const CfgEntry& e = kConfigs[cfg_id];
  if (BM) *BM = e.bm;
  if (BN) *BN = e.bn;
  if (BK) *BK = e.bk;
  if (threads) *threads = e.nt;
  if (lds_sb) *lds_sb = e.lds_sb;
  if (lds_db) *lds_db = e.lds_db;
  return GEMMF32_OK;
}

int gemm_f32_config_ms(int cfg_id, int* stages, int* lds_bytes) {
  if (cfg_id < 0 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  const CfgEntry& e = kConfigs[cfg_id];
  if (stages) *stages = e.ms_stages;
  if (lds_bytes) *lds_bytes = e.lds_ms;
  return GEMMF32_OK;
}

int gemm_f32_last_hip_error(void) { return g_last_hip_error; }

const char* gemm_f32_strerror(int code) {
  switch (code) {
    case GEMMF32_OK: return "success";
    case GEMMF32_ERR_NEGATIVE_DIM: return "negative matrix dimension";
    case GEMMF32_ERR_BAD_LD: return "leading dimension smaller than the row length";
    case GEMMF32_ERR_NULL_PTR: return "null pointer for a non-empty operand";
    case GEMMF32_ERR_MISALIGNED: return "operand pointer not 4-byte aligned";
    case GEMMF32_ERR_ALIAS: return "C overlaps A or B";
    case GEMMF32_ERR_TOO_LARGE: return "dimension or grid too large for one launch";
    case GEMMF32_ERR_BAD_CONFIG: return "unknown variant or tile configuration";
    case GEMMF32_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

const char* gemm_f32_version(void) { return "gemmf32 0.1.0 gfx950"; }

}  // extern "C"
