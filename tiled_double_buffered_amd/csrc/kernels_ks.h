// The K-split (KS) kernel of gemmf32: the K range of one output tile divided among the
// wave groups of one workgroup, whose partial sums meet in LDS.
#pragma once

#include "gemm_common.h"
#include "kernels_sb_db.h"

namespace gemmf32 {

// ------------------------------------------------------------------------------------
// Few output rows against a long K (the skinny regime the case study places LLM decode
// in: "Case Study: The Double-Buffered GEMM", paragraph on the three regimes) leave most
// of a CU idle: a 32 x 32 output tile is one wave's MFMA chain, on one of the four SIMDs,
// and wider tiles cut the number of workgroups instead.  Here KS groups of the
// configuration's waves share one output tile.  Group g walks the g-th contiguous chunk
// of the K tiles with a double-buffered loop (k_loop_ks below) in its own two LDS slots;
// then groups
// 1 .. KS-1 hand their sums to group 0 through LDS, and group 0 adds them in that fixed
// order and stores the tile.  Deterministic; the result differs from the one-group loop
// only in the order of the FP32 additions.  No workspace: everything stays on chip.
//
// Barriers are per workgroup, so every wave must pass the same number: the group loop
// passes one per K tile, and a group with fewer K tiles (the last chunk, or none when K is
// short) passes the missing ones after its loop.
// ------------------------------------------------------------------------------------
// A one-wave configuration gets four groups, one wave per SIMD of the CU (when their slots
// fit in LDS); any other configuration has no KS kernel (1).
template <class C>
constexpr int ks_groups() {
  constexpr int ks = 4;
  constexpr int slots = ks * 2 * C::SLOT * 4;
  constexpr int red = (ks - 1) * C::NT * C::FM * C::FN * 16 * 4;
  return C::NT == 64 && slots <= 160 * 1024 && red <= 160 * 1024 ? ks : 1;
}

template <class C, int KS>
struct KsCfg {
  static constexpr int RED = (KS - 1) * C::NT * C::FM * C::FN * 16;  // hand-off floats
  static constexpr int SLOTS = KS * 2 * C::SLOT;
  static constexpr int LDS_FLOATS = SLOTS > RED ? SLOTS : RED;
  static_assert(KS >= 2, "at least two groups");
  static_assert(C::NT * KS <= 1024, "threads of one workgroup");
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS of one CU");
};

// ------------------------------------------------------------------------------------
// The loop of one group: double-buffered LDS slots as in k_loop_db (one barrier per K
// tile), but the global loads run two tiles ahead, into two register sets used in turn.
// A group is one wave per SIMD with a short MFMA chain per tile, so one tile of lookahead
// leaves most of the load latency exposed.  In step l tile l is multiplied from slot
// l % 2, tile l+1 (loaded during step l-1) goes to the idle slot before the barrier, and
// tile l+2 is loaded into the register set that held tile l.
// ------------------------------------------------------------------------------------
template <class C, bool GUARD, bool EDGE>
__device__ __forceinline__ void ks_load(TileCopy<C>& cp, const LoopArgs<C>& g, int kt,
                                        int k_tiles) {
  if (kt + 1 == k_tiles)  // the last tile: its A columns >= K are zeroed
    load_tile<C, GUARD, true>(cp, g, kt);
  else
    load_tile<C, GUARD, false, EDGE>(cp, g, kt);
}

template <class C, bool GUARD, bool EDGE>
__device__ __forceinline__ void ks_step(const float* cur, float* nxt, TileCopy<C>& have,
                                        TileCopy<C>& next, const LaneView<C>& lv,
                                        const LoopArgs<C>& g, int l, int k_tiles,
                                        Frag<C> (&f)[2], floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  if (l + 2 < k_tiles) ks_load<C, GUARD, EDGE>(next, g, l + 2, k_tiles);
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 1>(f[1], acc);
  have.store(nxt);
  if constexpr (!GUARD) {
    Sched<C>::template db_before_barrier<0>();
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if constexpr (!GUARD) __builtin_amdgcn_sched_barrier(0);
  have.poison(const_cast<float*>(cur));  // debug builds: tile l's slot is free from here on
  read_frag(nxt, lv, 0, f[0]);
  mfma_round<C, 2>(f[1], acc);
  if constexpr (!GUARD) Sched<C>::db_after_barrier();
}

// Barriers: 1 (prologue) + (k_tiles - 1), one per K tile as in k_loop_db.
template <class C, bool GUARD, bool EDGE = true>
__device__ inline void k_loop_ks(float* smem, TileCopy<C>& cp0, TileCopy<C>& cp1,
                                 const LaneView<C>& lv, const LoopArgs<C>& g, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN]) {
  constexpr int R = C::BK / 8;
  Frag<C> f[2];
  float* const s0 = smem;
  float* const s1 = smem + C::SLOT;
  cp0.poison(s0);  // debug builds: nothing is valid in either slot yet
  cp0.poison(s1);
  ks_load<C, GUARD, EDGE>(cp0, g, 0, k_tiles);
  cp0.store(s0);
  if (k_tiles > 1) ks_load<C, GUARD, EDGE>(cp1, g, 1, k_tiles);
  __syncthreads();
  read_frag(s0, lv, 0, f[0]);
  int l = 0;
  for (; l + 3 < k_tiles; l += 2) {
    ks_step<C, GUARD, EDGE>(s0, s1, cp1, cp0, lv, g, l, k_tiles, f, acc);
    ks_step<C, GUARD, EDGE>(s1, s0, cp0, cp1, lv, g, l + 1, k_tiles, f, acc);
  }
  for (; l + 1 < k_tiles; ++l) {
    if (l & 1)
      ks_step<C, GUARD, EDGE>(s1, s0, cp0, cp1, lv, g, l, k_tiles, f, acc);
    else
      ks_step<C, GUARD, EDGE>(s0, s1, cp1, cp0, lv, g, l, k_tiles, f, acc);
  }
  // Last tile (l == k_tiles - 1): nothing left to load.
  const float* cur = (l & 1) ? s1 : s0;
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  mfma_round<C, 0>(f[1], acc);
}

template <class C, int KS>
__global__ void __launch_bounds__(C::NT * KS)
gemm_f32_ks_kernel(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                   const float* __restrict__ B, int64_t ldb, float* __restrict__ Cmat,
                   int64_t ldc, int flags, SplitArgs sp) {
  using KC = KsCfg<C, KS>;
  __shared__ __attribute__((aligned(16))) float smem[KC::LDS_FLOATS];

  const SplitWork w = split_work(sp, K, A, B, ldb);  // a plain launch: the tile only
  const int grp = __builtin_amdgcn_readfirstlane((int)threadIdx.x / C::NT);
  // This group's chunk: K tiles [grp * n, grp * n + n) of k_tiles, cut at K.
  const int k_tiles = (K + C::BK - 1) / C::BK;
  const int n = (k_tiles + KS - 1) / KS;
  const int kb = grp * n * C::BK;
  const int kg = max(0, min(K - kb, n * C::BK));
  const int my_tiles = (kg + C::BK - 1) / C::BK;
  TilePos<C> t;
  t.init(M, N, kg, A + kb, lda, B + (int64_t)kb * ldb, ldb, flags, w.bid, sp.tiles);
  // the group's own thread, wave and lane numbers
  t.tid = (int)threadIdx.x - grp * C::NT;
  t.lane = t.tid & 63;
  t.wave = __builtin_amdgcn_readfirstlane(t.tid >> 6);
  t.wm = t.wave / C::WAVES_N;
  t.wn = t.wave % C::WAVES_N;
  floatx16 acc[C::FM][C::FN];
  zero_acc<C>(acc);
  TileCopy<C> cp0, cp1;
  cp0.init(t.tid, lda, ldb);
  cp1.init(t.tid, lda, ldb);
  LaneView<C> lv;
  lv.init(t.wm, t.wn, t.lane);
  float* const slots = smem + grp * 2 * C::SLOT;
  if (my_tiles > 0) {
    if (t.unguarded() && t.m_full && t.n_full)
      k_loop_ks<C, false, false>(slots, cp0, cp1, lv, t.g, my_tiles, acc);
    else if (t.unguarded())
      k_loop_ks<C, false, true>(slots, cp0, cp1, lv, t.g, my_tiles, acc);
    else
      k_loop_ks<C, true>(slots, cp0, cp1, lv, t.g, my_tiles, acc);
  }
  for (int i = my_tiles; i < n; ++i) __syncthreads();  // the barriers of missing K tiles

  // Hand-off: group g (g >= 1) writes its sums to region g-1, lane-contiguous per
  // (wave, block, accumulator register); group 0 adds regions 0 .. KS-2 in order.
  __syncthreads();  // every group is done reading its slots
  constexpr int kRegion = C::NT * C::FM * C::FN * 16;
  if (grp > 0) {
    float* red = smem + (grp - 1) * kRegion;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[((t.wave * C::FM * C::FN + fm * C::FN + fn) * 16 + r) * 64 + t.lane] =
              acc[fm][fn][r];
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g + 1 < KS; ++g) {
      const float* red = smem + g * kRegion;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[fm][fn][r] +=
                red[((t.wave * C::FM * C::FN + fm * C::FN + fn) * 16 + r) * 64 + t.lane];
    }
    store_c<C>(acc, Cmat, ldc, t);
  }
}

}  // namespace gemmf32
