// The register-staged K-loops of gemmf32 and their kernel: double-buffered (two LDS
// slots, one barrier per K tile), single-buffered (one slot, two barriers) and the
// single-buffered baseline with split copy barriers (three).
#pragma once

#include "gemm_common.h"

namespace gemmf32 {

// One steady-state step of the double-buffered loop: copy tile l+1 towards the idle slot
// `nxt` while multiplying the tile in `cur`, one barrier at the hand-off.  On entry f[0]
// holds round 0 of the current tile; on exit it holds round 0 of tile l+1.  MASKED: tile
// l+1 is the last one (it may end past K).
template <class C, bool GUARD, bool MASKED = false, bool EDGE = true>
__device__ __forceinline__ void db_step(const float* cur, float* nxt, TileCopy<C>& cp,
                                        const LaneView<C>& lv, const LoopArgs<C>& g, int l,
                                        Frag<C> (&f)[2], floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  load_tile<C, GUARD, MASKED, EDGE>(cp, g, l + 1);  // in flight during the MFMAs below
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 1>(f[1], acc);
  cp.store(nxt);
  // The scheduling hints describe the two sides of the barrier separately; the fences
  // (sched_barrier) keep the compiler from moving register-only MFMAs across it, which
  // would undo the tail of MFMAs placed after the LDS stores.
  if constexpr (!GUARD) {
    Sched<C>::template db_before_barrier<0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if constexpr (!GUARD) __builtin_amdgcn_sched_barrier(0);
  cp.poison(const_cast<float*>(cur));  // debug builds: tile l's slot is free from here on
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
// the tile parity.  The step that copies the last tile (and the prologue, when there is
// only one) is peeled: that tile may end past K, and its A columns >= K are zeroed.
template <class C, bool GUARD, bool EDGE = true>
__device__ inline void k_loop_db(float* smem, TileCopy<C>& cp, const LaneView<C>& lv,
                                 const LoopArgs<C>& g, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  Frag<C> f[2];
  float* const s0 = smem;
  float* const s1 = smem + C::SLOT;
  cp.poison(s0);  // debug builds: nothing is valid in either slot yet
  cp.poison(s1);
  if (k_tiles == 1)  // prologue: tile 0 into slot 0
    load_tile<C, GUARD, true>(cp, g, 0);
  else
    load_tile<C, GUARD, false, EDGE>(cp, g, 0);
  cp.store(s0);
  __syncthreads();
  read_frag(s0, lv, 0, f[0]);
  int l = 0;
  if constexpr (C::DB_UNROLL) {
    for (; l + 3 < k_tiles; l += 2) {
      db_step<C, GUARD, false, EDGE>(s0, s1, cp, lv, g, l, f, acc);
      db_step<C, GUARD, false, EDGE>(s1, s0, cp, lv, g, l + 1, f, acc);
    }
  }
  for (; l + 2 < k_tiles; ++l)
    db_step<C, GUARD, false, EDGE>((l & 1) ? s1 : s0, (l & 1) ? s0 : s1, cp, lv, g, l, f, acc);
  if (l + 1 < k_tiles) {  // the copy of the last tile
    db_step<C, GUARD, true>((l & 1) ? s1 : s0, (l & 1) ? s0 : s1, cp, lv, g, l, f, acc);
    ++l;
  }
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
template <class C, bool GUARD, bool SPLIT, bool MASKED, bool EDGE>
__device__ __forceinline__ void sb_step(float* smem, TileCopy<C>& cp, const LaneView<C>& lv,
                                        const LoopArgs<C>& g, int l,
                                        floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  Frag<C> f[2];
  if constexpr (SPLIT) {
    load_tile_a<C, GUARD, MASKED, EDGE>(cp, g, l);
    cp.store_a(smem);
    __syncthreads();  // the A tile is in LDS
    load_tile_b<C, GUARD, MASKED, EDGE>(cp, g, l);
    cp.store_b(smem);
  } else {
    load_tile<C, GUARD, MASKED, EDGE>(cp, g, l);
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
  cp.poison(smem);  // debug builds: from here on nobody may read tile l
  mfma_round<C, 0>(f[1], acc);
}

template <class C, bool GUARD, bool SPLIT = false, bool EDGE = true>
__device__ inline void k_loop_sb(float* smem, TileCopy<C>& cp, const LaneView<C>& lv,
                                 const LoopArgs<C>& g, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN]) {
  cp.poison(smem);  // debug builds: nothing is valid in the slot yet
  for (int l = 0; l + 1 < k_tiles; ++l)
    sb_step<C, GUARD, SPLIT, false, EDGE>(smem, cp, lv, g, l, acc);
  // the last tile may end past K: its A columns >= K are zeroed
  if (k_tiles > 0) sb_step<C, GUARD, SPLIT, true, EDGE>(smem, cp, lv, g, k_tiles - 1, acc);
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
                     int64_t ldc, int flags, SplitArgs sp) {
  static_assert((C::BK / 8) % 2 == 0, "BK/8 rounds must be even for the fragment ping-pong");
  static_assert(LOOP == kLoopSB || LOOP == kLoopDB || LOOP == kLoopSB3, "loop kind");
  constexpr bool DB = LOOP == kLoopDB;
  constexpr bool SPLIT = LOOP == kLoopSB3;
  __shared__ __attribute__((aligned(16))) float smem[(DB ? 2 : 1) * C::SLOT];

  const SplitWork w = split_work(sp, K, A, B, ldb);
  TilePos<C> t;
  t.init(M, N, K, A, lda, B, ldb, flags, w.bid, sp.tiles);
  split_output(sp, w, N, t, Cmat, ldc);
  floatx16 acc[C::FM][C::FN];
  zero_acc<C>(acc);
  TileCopy<C> cp;
  cp.init(t.tid, lda, ldb);
  LaneView<C> lv;
  lv.init(t.wm, t.wn, t.lane);
  const int k_tiles = (K + C::BK - 1) / C::BK;
  if (k_tiles > 0) {
    // Interior tiles copy every K tile but the last with the widest buffer range; edge
    // tiles need exact ranges throughout; the element-guarded loop handles the rest.
    const bool interior = t.m_full && t.n_full;
    if constexpr (DB) {
      if (t.unguarded() && interior)
        k_loop_db<C, false, false>(smem, cp, lv, t.g, k_tiles, acc);
      else if (t.unguarded())
        k_loop_db<C, false, true>(smem, cp, lv, t.g, k_tiles, acc);
      else
        k_loop_db<C, true>(smem, cp, lv, t.g, k_tiles, acc);
    } else {
      if (t.unguarded() && interior)
        k_loop_sb<C, false, SPLIT, false>(smem, cp, lv, t.g, k_tiles, acc);
      else if (t.unguarded())
        k_loop_sb<C, false, SPLIT, true>(smem, cp, lv, t.g, k_tiles, acc);
      else
        k_loop_sb<C, true, SPLIT>(smem, cp, lv, t.g, k_tiles, acc);
    }
  }
  store_c<C>(acc, Cmat, ldc, t);
}

}  // namespace gemmf32
