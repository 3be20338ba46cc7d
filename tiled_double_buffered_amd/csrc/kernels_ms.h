// The multi-stage (MS) K-loop of gemmf32 and its kernel: S LDS stages filled by gfx950
// direct-to-LDS copies.
#pragma once

#include "gemm_common.h"
#include "kernels_sb_db.h"

namespace gemmf32 {

// ------------------------------------------------------------------------------------
// Multi-stage variant (MS): S LDS stages filled by gfx950 direct-to-LDS loads.
//
// The glossary page ("Double Buffering", second paragraph and the figure caption) notes
// that its platform lost its asynchronous copy engine, so its double buffering overlaps
// copies and math only through instruction-level parallelism, and it names the CUDA
// analogue: a multi-stage asynchronous-copy pipeline.  gfx950 has the asynchronous copy:
// buffer_load_dwordx4 with the lds flag moves 16 bytes per lane from global memory
// straight into LDS (lane L's bytes land at M0 + 16*L), with no registers in between and
// completion tracked by vmcnt.  Tiles l+1 .. l+S-1 are in flight while tile l is multiplied.
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
  static constexpr int RPC_B = 256 / C::BN;          // (when whole rows fit in 1 KiB)
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

__device__ __forceinline__ int swz_b(int k) { return ((k >> 2) & 1) << 3; }

// The four descriptor words of a raw buffer starting at `base` and `range` bytes long
// (flags as for the register-staged copies), for the inline-assembly copies below.
typedef int int32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int32x4 buffer_words(const float* base, uint32_t range) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  int32x4 r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)(uint32_t)(b >> 32);
  r[2] = (int)range;
  r[3] = kBufferFlags;
  return r;
}

template <class C, int S>
struct MsCopy {
  using MC = MsCfg<C, S>;
  uint32_t off[MC::D];      // this lane's byte offset from its operand's tile origin
  bool from_a[MC::D];       // copy i fills part of the A tile (uniform per wave)
  uint32_t lds_off[MC::D];  // byte offset of the wave's 1 KiB inside a stage
  uint32_t lds_base;        // LDS byte address of stage 0
  const float* a_org;       // A + m0 * lda
  const float* b_org;       // B + n0
  int64_t ldb;
  int64_t a_bytes, b_bytes;  // byte extents of A and B left from a_org and b_org

  __device__ inline void init(const float* smem, int wave, int lane, const float* A,
                              int64_t lda, const float* B, int64_t ldb_, int m0, int n0,
                              int64_t a_bytes_, int64_t b_bytes_) {
    // The wave index is below WAVES; saying so lets the compiler resolve at compile time
    // which operand each copy reads wherever the split of A and B chunks allows.
    __builtin_assume(wave >= 0 && wave < MC::WAVES);
    lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_float*)smem);
    a_org = A + (int64_t)m0 * lda;
    b_org = B + n0;
    ldb = ldb_;
    a_bytes = a_bytes_ - (int64_t)m0 * lda * 4;
    b_bytes = b_bytes_ - (int64_t)n0 * 4;
#pragma unroll
    for (int i = 0; i < MC::D; ++i) {
      const int j = wave + i * MC::WAVES;  // which 1 KiB of the stage this copy fills
      from_a[i] = j < MC::A_CHUNKS;
      if (j < MC::A_CHUNKS) {
        const int row = j * MC::RPC_A + lane / MC::CPR_A;
        const int c = (lane % MC::CPR_A) ^ swz_a<C::BK>(row);
        off[i] = (uint32_t)(((int64_t)row * lda + 4 * c) * 4);
        lds_off[i] = (uint32_t)j * 1024u;
      } else {
        const int jb = j - MC::A_CHUNKS;
        int k, c;
        if constexpr (256 % C::BN == 0) {  // whole B rows per 1 KiB
          k = jb * MC::RPC_B + lane / MC::CPR_B;
          c = (lane % MC::CPR_B) ^ swz_b(k);
        } else {  // a 1 KiB copy spans row boundaries (192-wide tiles)
          const int p = jb * 256 + 4 * lane;  // float index in the stage's B part
          k = p / C::BN;
          c = ((p % C::BN) / 4) ^ swz_b(k);
        }
        off[i] = (uint32_t)(((int64_t)k * ldb + 4 * c) * 4);
        lds_off[i] = (uint32_t)(MC::A_FLOATS * 4 + jb * 1024);
      }
    }
  }

  // Start the copy of K tile kt into stage st (asynchronous; counted by vmcnt).  The
  // sources are buffer loads: a descriptor per operand and K tile, built from the tile's
  // origin in scalar registers, plus this lane's fixed 32-bit offset, so no vector address
  // arithmetic runs per copy.  (The host takes this path only when every offset inside a
  // tile fits in 32 bits.)
  template <bool EXACT>
  __device__ inline void issue(int kt, int st) const {
    const uint32_t stage_base = lds_base + (uint32_t)st * (uint32_t)(MC::STAGE * 4);
    // Ranges end where A and B end: rows of A past M read as 0, and columns of B past N
    // read the next row or 0, which reach only C elements the epilogue does not store.
    // (EXACT: edge tiles; interior tiles lie inside A and B, and the widest range saves
    // the scalar arithmetic.)
    const int32x4 ra = buffer_words(
        a_org + (int64_t)kt * C::BK,
        EXACT ? TileCopy<C>::range_from(a_bytes, (int64_t)kt * C::BK) : kBufferRange);
    const int32x4 rb = buffer_words(
        b_org + (int64_t)kt * C::BK * ldb,
        EXACT ? TileCopy<C>::range_from(b_bytes, (int64_t)kt * C::BK * ldb) : kBufferRange);
#pragma unroll
    for (int i = 0; i < MC::D; ++i) {
      const int32x4 r = from_a[i] ? ra : rb;
      const uint32_t m0v = __builtin_amdgcn_readfirstlane(stage_base + lds_off[i]);
      // M0 is reserved by the compiler, which warns about clobbering it.  Nothing else in
      // these kernels uses M0 (a structural test checks that every M0 write is one of these
      // copies, followed by its load), so the clobber is safe here.  A scalar write of M0
      // needs one wait state before a direct-to-LDS load reads it; the compiler inserts that
      // for its own code but cannot see inside this statement, hence the s_nop.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(off[i]), "s"(r), "s"(m0v)
                   : "memory", "m0");
#pragma clang diagnostic pop
    }
  }
};

// LDS-poison debug mode: overwrite with NaN the 16 bytes this lane's copies write into
// stage st (lane L of a copy fills bytes 16 L .. 16 L + 15 of the copy's 1 KiB), after the
// barrier that frees the stage and before the copy that refills it.  The wait makes these
// stores land before that copy can write the same bytes.
template <class C, int S>
__device__ __forceinline__ void ms_poison(float* smem, const MsCopy<C, S>& cp, int lane,
                                          int st) {
  if constexpr (kLdsPoison) {
    using MC = MsCfg<C, S>;
#pragma unroll
    for (int i = 0; i < MC::D; ++i)
      *reinterpret_cast<floatx4*>(smem + st * MC::STAGE + (cp.lds_off[i] + 16 * lane) / 4) =
          nan4();
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  }
}

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
    a_x = h ^ swz_a<C::BK>(row);
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
// With one wave per SIMD and one 32 x 32 block per wave (four MFMAs per round), the whole
// last round runs after the barrier, from registers already loaded: its four MFMAs cover
// the LDS latency of the next tile's first fragments, which half a round left partly
// exposed (64 x 64 tiles: 1.5-3% faster).  Where two waves share a SIMD the other wave
// covers it, and the half-round split measured as fast or faster.
template <class C, int S, bool EDGE>
__device__ __forceinline__ void ms_step(float* smem, const MsCopy<C, S>& cp,
                                        const LaneViewMs<C, S>& lv, int l, int k_tiles,
                                        int st, Frag<C> (&f)[2],
                                        floatx16 (&acc)[C::FM][C::FN], int lane) {
  using MC = MsCfg<C, S>;
  constexpr int R = C::BK / 8;
  cp.template issue<EDGE>(min(l + S - 1, k_tiles - 1), st == 0 ? S - 1 : st - 1);
  const float* cur = smem + st * MC::STAGE;
#pragma unroll
  for (int q = 0; q + 1 < R; ++q) {
    read_frag_ms(cur, lv, q + 1, f[(q + 1) & 1]);
    mfma_round<C, 0>(f[q & 1], acc);
  }
  if constexpr (Sched<C>::MQ == 4 && C::NT == 256) {
    __builtin_amdgcn_sched_barrier(0);
    ms_wait_tile_barrier<C, S>();
    __builtin_amdgcn_sched_barrier(0);
    ms_poison(smem, cp, lane, st);  // debug builds: tile l's stage is free from here on
    read_frag_ms(smem + (st + 1 == S ? 0 : st + 1) * MC::STAGE, lv, 0, f[0]);
    mfma_round<C, 0>(f[1], acc);
    return;
  }
  mfma_round<C, 1>(f[1], acc);
  Sched<C>::template rounds_with_reads<0>();
  sched_group<kSchedMfma, Sched<C>::MQ / 2>();
  // With few MFMAs per round (small wave tiles) the two sides of the barrier are kept
  // apart, as in the double-buffered step; with many, the compiler's own placement
  // measured faster.
  constexpr bool kFence = Sched<C>::MQ <= 8;
  if constexpr (kFence) __builtin_amdgcn_sched_barrier(0);
  ms_wait_tile_barrier<C, S>();
  if constexpr (kFence) __builtin_amdgcn_sched_barrier(0);
  ms_poison(smem, cp, lane, st);  // debug builds: tile l's stage is free from here on
  read_frag_ms(smem + (st + 1 == S ? 0 : st + 1) * MC::STAGE, lv, 0, f[0]);
  mfma_round<C, 2>(f[1], acc);
  Sched<C>::db_after_barrier();
}

// The MS K-loop: prologue (tiles 0 .. S-2 in flight, tile 0 landed), steps unrolled S at a
// time so that every stage address is fixed, the remaining steps one by one, and the
// last tile (nothing left to copy) peeled off.
template <class C, int S, bool EDGE>
__device__ inline void k_loop_ms(float* smem, const MsCopy<C, S>& cp,
                                 const LaneViewMs<C, S>& lv, int k_tiles,
                                 floatx16 (&acc)[C::FM][C::FN], int lane) {
  using MC = MsCfg<C, S>;
  constexpr int R = C::BK / 8;
#pragma unroll
  for (int t = 0; t < S; ++t) ms_poison(smem, cp, lane, t);  // debug builds: nothing valid yet
#pragma unroll
  for (int t = 0; t < S - 1; ++t) cp.template issue<EDGE>(min(t, k_tiles - 1), t);
  ms_wait_tile_barrier<C, S>();
  Frag<C> f[2];
  read_frag_ms(smem, lv, 0, f[0]);
  int l = 0;
  for (; l + S < k_tiles; l += S) {
#pragma unroll
    for (int u = 0; u < S; ++u)
      ms_step<C, S, EDGE>(smem, cp, lv, l + u, k_tiles, u, f, acc, lane);
  }
  for (; l + 1 < k_tiles; ++l)
    ms_step<C, S, EDGE>(smem, cp, lv, l, k_tiles, l % S, f, acc, lane);
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
                   int64_t ldc, int flags, SplitArgs sp) {
  using MC = MsCfg<C, S>;
  __shared__ __attribute__((aligned(1024))) float smem[MC::LDS_FLOATS];

  const SplitWork w = split_work(sp, K, A, B, ldb);
  TilePos<C> t;
  t.init(M, N, K, A, lda, B, ldb, flags, w.bid, sp.tiles);
  split_output(sp, w, N, t, Cmat, ldc);
  floatx16 acc[C::FM][C::FN];
  zero_acc<C>(acc);
  const int k_tiles = (K + C::BK - 1) / C::BK;
  if (k_tiles > 0) {
    if (t.unguarded() && K % C::BK == 0) {
      MsCopy<C, S> cp;
      cp.init(smem, t.wave, t.lane, A, lda, B, ldb, t.g.m0, t.g.n0, t.g.a_bytes, t.g.b_bytes);
      LaneViewMs<C, S> lv;
      lv.init(t.wm, t.wn, t.lane);
      if (t.m_full && t.n_full)
        k_loop_ms<C, S, false>(smem, cp, lv, k_tiles, acc, t.lane);
      else
        k_loop_ms<C, S, true>(smem, cp, lv, k_tiles, acc, t.lane);
    } else {
      // A K tail (its A columns past K must be zeroed, which a direct-to-LDS copy cannot
      // do) or offsets beyond the 32-bit range: the double-buffered loop, with 16-byte
      // copies and a masked last tile, or element-guarded copies.
      TileCopy<C> cp;
      cp.init(t.tid, lda, ldb);
      LaneView<C> lv;
      lv.init(t.wm, t.wn, t.lane);
      if (t.unguarded())
        k_loop_db<C, false, true>(smem, cp, lv, t.g, k_tiles, acc);
      else
        k_loop_db<C, true>(smem, cp, lv, t.g, k_tiles, acc);
    }
  }
  store_c<C>(acc, Cmat, ldc, t);
}

// Stage count per configuration: as many as fit (at most 4) in the 160 KiB of a CU.
template <class C>
constexpr int ms_stages() {
  constexpr int stage_bytes = 4 * (C::BM * C::BK + C::BK * C::BN);
  return (160 * 1024) / stage_bytes >= 4 ? 4 : (160 * 1024) / stage_bytes;
}

}  // namespace gemmf32
