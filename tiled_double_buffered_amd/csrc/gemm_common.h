// Shared device code of the gemmf32 kernels: tile configurations, the workgroup-to-tile
// order, the register-staged global -> LDS copy, the FP32 matrix-core micro-kernel, the
// instruction-interleaving hints, per-workgroup setup and the guarded epilogue.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

// Debug builds only (the library's lds-poison variant): every LDS slot or stage is filled
// with NaN right after the barrier that frees it (see TileCopy::poison).
#ifndef GEMMF32_LDS_POISON
#define GEMMF32_LDS_POISON 0
#endif

namespace gemmf32 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr bool kLdsPoison = GEMMF32_LDS_POISON != 0;

__device__ __forceinline__ floatx4 nan4() {
  const float q = __builtin_nanf("");
  return floatx4{q, q, q, q};
}

// ------------------------------------------------------------------------------------
// Tile configuration.
//   BM x BN : output tile of one workgroup        BK : K depth of one LDS tile
//   WAVES_M x WAVES_N waves per workgroup; each wave owns a TM x TN sub-tile made of
//   FM x FN blocks of 32 x 32, one 16-register accumulator per block.
// LDS layout of one slot (FP32):
//   As[BM][AS]  A tile with k contiguous.  K tiles of 16 (SWZ_A): unpadded rows (AS = BK)
//               whose 16-byte chunks are XOR-swizzled, chunk c of row r at chunk
//               c ^ swz_a<BK>(r) (below).  Deeper K tiles: rows padded to AS = BK + 4.
//   Bs[BK][BS]  B tile with n contiguous, row stride BS = BN + 8 (so the two half-waves,
//               which read rows 4 apart, land on opposite halves of the 64 banks)
//
// A fragment read has 16 lanes read one logical 16-byte chunk of 16 consecutive rows.
// With padded rows, row r starts on bank group (of 4 banks) r * (BK + 4) / 4 mod 16, an
// odd multiple of r for BK = 16, 32 and 64, so the 16 rows hit 16 different groups.  The
// copy's 16-byte stores of 16-row-deep tiles (four 16-float rows per 16 lanes) then wrap
// onto their own first banks, though: the counters measured 17% of LDS cycles lost to
// bank conflicts for the 256x256x16 tile, and none for the padded 32- and 64-deep tiles.
// The swizzle removes them for BK = 16: the 16 lanes of a store cover 64 consecutive
// words, only permuted inside each row, and each of the rows that start on the same bank
// group (unpadded, r * 4 mod 16) has its chunk moved by a different amount, so a read's
// 16 rows still land on 16 different bank groups.  (The swizzle is kept to BK = 16: on the
// deeper tiles it measured no faster, and the single-buffered 8-wave 128x256x32 tile ran
// 17% slower with it at 8192^3 though its counters showed no conflicts either way.)
// ------------------------------------------------------------------------------------
// Swizzle of A row r: constant over runs of 64/BK rows, stepping through 0 .. BK/4 - 1, so
// its period is 16 rows for every BK.
template <int BK>
__host__ __device__ constexpr int swz_a(int row) {
  return (row / (64 / BK)) % (BK / 4);
}

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr bool SWZ_A = BK == 16;
  static constexpr int AS = SWZ_A ? BK : BK + 4;
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
  static_assert(BK == 16 || BK == 32 || BK == 64, "A layouts");
  static_assert((BM * BK / 4) % NT == 0 && (BK * BN / 4) % NT == 0, "copy must divide");
  static_assert(NT % A_GROUPS_PER_ROW == 0, "copy rows of A");
  // NT a multiple of the B groups per row: every pass of the B copy starts at the same
  // column, one row stride further (otherwise, as for 192-wide tiles, per pass)
  static constexpr bool B_EVEN = NT % B_GROUPS_PER_ROW == 0;
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "copy work per thread");
};

// Flags passed to the kernel.
enum : int {
  kVecA = 1,  // every 16-byte copy offset inside a tile of A fits the 32-bit buffer range
  kVecB = 2,  // same for B
};

// ------------------------------------------------------------------------------------
// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin; renumber
// them so that consecutive ids run on one XCD (which has its own L2), then walk the
// tiles in column-major groups of `group_m` tile rows so that workgroups close in id
// share panels of A and B.  The renumbering holds for any number of workgroups: without
// it, neighbouring tiles of a decode product (16 rows, tiles side by side along N) sit on
// different XCDs, each fetching the 128-byte lines of B they share, and such products ran
// up to 2x slower whenever the tile count was not a multiple of 8.  Both choices can be changed per launch for measurement (flags
// bits 8..15: group_m, 0 = the default 4; bit 16: keep the hardware order of ids).
// Default 4: on the dispatched kernels at 8192^3, 4096^3, 1024 x 8192 x 8192 and
// 4096 x 11008 x 4096, group heights 4 and 8 run equally fast (within 0.1%), and 4 makes
// the L2s fetch fewer bytes (8% fewer at 8192^3, no more elsewhere) than 8 and every other
// height tried (1, 2, 3, 16, 32, with and without the renumbering).
// ------------------------------------------------------------------------------------
enum : int { kRasterGroupShift = 8, kRasterNoXcdRemap = 1 << 16 };

// `bid` is the tile's index in launch order and `nwg` the number of tiles of the product.
__device__ inline void tile_coords(int bid, int nwg, int tiles_m, int tiles_n, int flags,
                                   int& tm, int& tn) {
  constexpr int kXcds = 8;
  const int gm_flag = (flags >> kRasterGroupShift) & 0xff;
  const int group_m = gm_flag ? gm_flag : 4;
  if (!(flags & kRasterNoXcdRemap)) {
    // workgroup bid runs on XCD bid mod 8 as its (bid div 8)-th; XCD x runs q or q + 1 of
    // the nwg workgroups (q = nwg div 8, one more for x < nwg mod 8), so giving it the
    // consecutive ids from x q + min(x, nwg mod 8) on is a permutation of 0 .. nwg - 1
    const int q = nwg / kXcds, r = nwg % kXcds, x = bid % kXcds;
    bid = x * q + min(x, r) + bid / kXcds;
  }
  const int per_group = group_m * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * group_m;
  const int rows = min(tiles_m - first_m, group_m);
  const int in_group = bid - group * per_group;
  tm = first_m + in_group % rows;
  tn = in_group / rows;
}

// Buffer descriptor of the fast copies: a raw byte buffer (stride 0) whose range check
// admits every 32-bit offset below kBufferRange; word 3 selects 32-bit data, the
// untyped-load setting of this GPU family.
constexpr uint32_t kBufferRange = 0xFFFFFFF0u;
constexpr int kBufferFlags = 0x00020000;

// ------------------------------------------------------------------------------------
// The workgroup's copy of one K tile: global memory -> registers -> LDS.
// Thread t moves groups g = t + p * NT (p = 0 .. PER_T-1); group g of A is row
// g / (BK/4), columns 4 * (g % (BK/4)) .. +3 of the tile; likewise for B with BN/4.
// When NT is a multiple of the groups per row, pass p is pass 0 moved down by
// p * NT / (groups per row) rows; otherwise (B of a 192-wide tile) each pass has its own
// row and column.
// ------------------------------------------------------------------------------------
// Row and column of a thread's B group in each pass, kept only where passes differ in
// column (empty otherwise).
template <int N>
struct BPassCoords {
  int rows[N], cols[N];
};
template <>
struct BPassCoords<0> {};

template <class C>
struct TileCopy {
  floatx4 ra[C::A_PER_T];
  floatx4 rb[C::B_PER_T];

  // Per-thread coordinates inside the tile (B: of pass 0, or of every pass when the
  // passes do not share a column).
  int a_row, a_col, b_row, b_col;
  [[no_unique_address]] BPassCoords<C::B_EVEN ? 0 : C::B_PER_T> bp;

  __device__ inline int brow(int i) const {
    if constexpr (C::B_EVEN) return b_row + i * C::B_ROWS_PER_PASS;
    else return bp.rows[i];
  }
  __device__ inline int bcol(int i) const {
    if constexpr (C::B_EVEN) return b_col;
    else return bp.cols[i];
  }
  // Byte offsets of this thread's 16-byte groups from the tile's first element; they are
  // the same for every K tile (see the fast path below).
  uint32_t a_off[C::A_PER_T], b_off[C::B_PER_T];

  __device__ inline void init(int tid, int64_t lda, int64_t ldb) {
    a_row = tid / C::A_GROUPS_PER_ROW;
    a_col = 4 * (tid % C::A_GROUPS_PER_ROW);
    b_row = tid / C::B_GROUPS_PER_ROW;
    b_col = 4 * (tid % C::B_GROUPS_PER_ROW);
    if constexpr (!C::B_EVEN) {
#pragma unroll
      for (int i = 0; i < C::B_PER_T; ++i) {
        bp.rows[i] = (tid + i * C::NT) / C::B_GROUPS_PER_ROW;
        bp.cols[i] = 4 * ((tid + i * C::NT) % C::B_GROUPS_PER_ROW);
      }
    }
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      a_off[i] = (uint32_t)(((int64_t)(a_row + i * C::A_ROWS_PER_PASS) * lda + a_col) * 4);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      b_off[i] = (uint32_t)(((int64_t)brow(i) * ldb + bcol(i)) * 4);
  }

  // Fast path: 16-byte buffer loads.  The tile's first element is a workgroup-uniform
  // base (a buffer descriptor in scalar registers, rebuilt by scalar arithmetic per K
  // tile) and each thread adds its fixed 32-bit offset.  Plain global loads would need a
  // 64-bit vector address add per load and per tile, and that vector arithmetic measurably
  // slows the matrix instructions it is interleaved with.
  //
  // The descriptor's range ends where the operand ends (`bytes` = the byte extent of A or
  // B from its origin), and a buffer load returns 0 for every 4-byte word past the range.
  // That makes the same copy serve edge tiles and any leading dimension:
  //   * A rows at or past M and B rows at or past K lie past the range and read 0;
  //   * B columns at or past N read the start of the next row (or 0 past the range), and A
  //     rows inside the matrix read their padding or the next row past column K-1: such
  //     values reach only C rows >= M or columns >= N, which the epilogue never stores,
  //     except A's columns >= K, which would meet B's zero rows: a K-tail tile therefore
  //     zeroes them (load_a_fast_masked);
  //   * rows need only 4-byte alignment (16-byte loads from 4-byte-aligned addresses are
  //     served in the unaligned access mode of this GPU).
  // The host takes this path only when every offset inside a tile fits in 32 bits.
  static __device__ inline floatx4 buffer_load16(const float* base, uint32_t range,
                                                 uint32_t off) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(base), (short)0, (int)range, kBufferFlags);
    return __builtin_bit_cast(floatx4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  }
  // Bytes of the operand left from element offset `first` on, clamped to the range a
  // descriptor can hold.
  static __device__ inline uint32_t range_from(int64_t bytes, int64_t first) {
    const int64_t left = bytes - first * 4;
    return left <= 0 ? 0u : left >= (int64_t)kBufferRange ? kBufferRange : (uint32_t)left;
  }
  // EXACT: the range ends where A ends (edge tiles, the last tile); otherwise the tile
  // lies inside A and the widest range saves the scalar arithmetic.
  template <bool EXACT>
  __device__ inline void load_a_fast(const float* __restrict__ A, int64_t lda, int m0,
                                     int k0, int64_t a_bytes) {
    const int64_t first = (int64_t)m0 * lda + k0;
    const uint32_t range = EXACT ? range_from(a_bytes, first) : kBufferRange;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) ra[i] = buffer_load16(A + first, range, a_off[i]);
  }
  // The same for the tile that holds column K-1 when K is not a multiple of BK: columns
  // >= K are zeroed, so they add exact zeros against B's zero rows.
  __device__ inline void load_a_fast_masked(const float* __restrict__ A, int64_t lda, int m0,
                                            int k0, int64_t a_bytes, int K) {
    load_a_fast<true>(A, lda, m0, k0, a_bytes);
    const int c = k0 + a_col;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) ra[i][e] = c + e < K ? ra[i][e] : 0.0f;
  }
  template <bool EXACT>
  __device__ inline void load_b_fast(const float* __restrict__ B, int64_t ldb, int n0,
                                     int k0, int64_t b_bytes) {
    const int64_t first = (int64_t)k0 * ldb + n0;
    const uint32_t range = EXACT ? range_from(b_bytes, first) : kBufferRange;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) rb[i] = buffer_load16(B + first, range, b_off[i]);
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
      const int r = k0 + brow(i);
      const int c = n0 + bcol(i);
      const float* p = B + (int64_t)r * ldb + c;
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (r < K && c + e < N) ? p[e] : 0.0f;
      rb[i] = v;
    }
  }

  // Where pass i of this thread's A copy goes in a slot (floats); swizzled passes whose
  // rows differ by whole swizzle periods (16 rows) differ by a constant.
  __device__ inline int a_store_off(int i) const {
    const int row = a_row + i * C::A_ROWS_PER_PASS;
    if constexpr (!C::SWZ_A)
      return row * C::AS + a_col;
    else if constexpr (C::A_ROWS_PER_PASS % 16 == 0)
      return a_row * C::AS + 4 * ((a_col >> 2) ^ swz_a<C::BK>(a_row)) +
             i * C::A_ROWS_PER_PASS * C::AS;
    else
      return row * C::AS + 4 * ((a_col >> 2) ^ swz_a<C::BK>(row));
  }
  __device__ inline void store_a(float* slot) {
    float* As = slot;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      *reinterpret_cast<floatx4*>(As + a_store_off(i)) = ra[i];
  }
  __device__ inline void store_b(float* slot) {
    float* Bs = slot + C::A_SLOT;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      *reinterpret_cast<floatx4*>(Bs + brow(i) * C::BS + bcol(i)) = rb[i];
  }
  __device__ inline void store(float* slot) {
    store_a(slot);
    store_b(slot);
  }

  // LDS-poison debug mode: overwrite this thread's own part of a slot with NaN.  It is
  // called right after the barrier that certifies every wave has finished reading the
  // slot (the double-buffered hand-off, whose one barrier does that double duty: "Case
  // Study: The Double-Buffered GEMM", paragraph after the code figure), and at the start.
  // The slot's next tile is stored by the same thread at the same addresses, after this in
  // program order, so a correct loop never reads the NaN; a wave that read the slot in
  // between -- before the next tile's barrier -- would carry NaN into C.
  __device__ inline void poison(float* slot) {
    if constexpr (kLdsPoison) {
      float* Bs = slot + C::A_SLOT;
#pragma unroll
      for (int i = 0; i < C::A_PER_T; ++i)
        *reinterpret_cast<floatx4*>(slot + a_store_off(i)) = nan4();
#pragma unroll
      for (int i = 0; i < C::B_PER_T; ++i)
        *reinterpret_cast<floatx4*>(Bs + brow(i) * C::BS + bcol(i)) = nan4();
    }
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

// This lane's fragment offsets (in floats) inside an LDS slot.  Round q reads logical
// chunk 2q + h of its A rows: at float 8q + 4h of a padded row, or, swizzled, at chunk
// (2q + h) ^ swz = (2q) ^ a_x; the rows of the lane's blocks are 32 apart, whole swizzle
// periods, so one a_x serves all of them.
template <class C>
struct LaneView {
  int a_off, a_x, b_off;
  __device__ inline void init(int wm, int wn, int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    const int row = wm * C::TM + l32;
    a_off = row * C::AS + (C::SWZ_A ? 0 : 4 * h);
    a_x = C::SWZ_A ? h ^ swz_a<C::BK>(row) : 0;
    b_off = C::A_SLOT + (4 * h) * C::BS + wn * C::TN + l32;
  }
};

template <class C>
__device__ inline void read_frag(const float* slot, const LaneView<C>& lv, int q, Frag<C>& f) {
  const float* a_ptr =
      slot + lv.a_off + (C::SWZ_A ? 4 * ((2 * q) ^ lv.a_x) : 8 * q);
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
// alone, sinks the prefetch loads to just before their LDS stores, which exposes
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
  static constexpr int G = C::A_PER_T + C::B_PER_T;    // 16-byte buffer loads per tile
  static constexpr int W = C::A_PER_T + C::B_PER_T;    // 16-byte LDS stores per tile
  static constexpr int D = C::FM + 2 * C::FN;          // LDS read instructions per round

  // MFMAs kept between the last LDS store of a tile and the barrier that publishes it,
  // where a round has enough of them: the wait for the stores before the barrier then
  // finds them complete instead of stalling the matrix pipe for their latency.
  static constexpr int TAIL = MQ / 2 >= 16 ? 4 : 0;

  // Double-buffered, from the top of an iteration up to the barrier: round 0 carries the
  // global loads of tile l+1 and the LDS reads of round 1; middle rounds carry the reads
  // of the next round; the first half of the last round carries the LDS stores of tile
  // l+1 into the idle slot, then TAIL MFMAs.
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
      sched_interleave<kSchedDsWrite, W, MQ / 2 - TAIL>();
      sched_group<kSchedMfma, TAIL>();
    }
  }
  // After the barrier: the rest of tile l's last round with the first reads of tile l+1
  // spread over it, an MFMA first so that the matrix pipe restarts at once (its operands
  // are already in registers).
  static __device__ __forceinline__ void db_after_barrier() {
    sched_group<kSchedMfma, 1>();
    sched_interleave<kSchedDsRead, D, MQ - MQ / 2 - 1>();
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
  int64_t a_bytes, b_bytes;  // byte extents of A (M x K) and B (K x N) from A and B
  int M, N, K, m0, n0;
  bool vec_a, vec_b;
};

// MASKED: this tile may hold column K-1 of a K that is not a multiple of BK (the last
// tile of the loop); its A columns >= K are zeroed, and its copies use exact ranges.
// EDGE: the workgroup's tile sticks out of M or N (exact ranges for every K tile).  The
// guarded loop always uses exact ranges for the tiles it copies 16 bytes at a time.
template <class C, bool GUARD, bool MASKED = false, bool EDGE = true>
__device__ inline void load_tile_a(TileCopy<C>& cp, const LoopArgs<C>& g, int kt) {
  constexpr bool EXACT = GUARD || MASKED || EDGE;
  const int k0 = kt * C::BK;
  if (!GUARD || (g.vec_a && k0 + C::BK <= g.K)) {
    if constexpr (MASKED)
      cp.load_a_fast_masked(g.A, g.lda, g.m0, k0, g.a_bytes, g.K);
    else
      cp.template load_a_fast<EXACT>(g.A, g.lda, g.m0, k0, g.a_bytes);
  } else {
    cp.load_a_guarded(g.A, g.lda, g.M, g.K, g.m0, k0);
  }
}

template <class C, bool GUARD, bool MASKED = false, bool EDGE = true>
__device__ inline void load_tile_b(TileCopy<C>& cp, const LoopArgs<C>& g, int kt) {
  constexpr bool EXACT = GUARD || MASKED || EDGE;
  const int k0 = kt * C::BK;
  if (!GUARD || (g.vec_b && k0 + C::BK <= g.K))
    cp.template load_b_fast<EXACT>(g.B, g.ldb, g.n0, k0, g.b_bytes);
  else
    cp.load_b_guarded(g.B, g.ldb, g.N, g.K, g.n0, k0);
}

template <class C, bool GUARD, bool MASKED = false, bool EDGE = true>
__device__ inline void load_tile(TileCopy<C>& cp, const LoopArgs<C>& g, int kt) {
  load_tile_a<C, GUARD, MASKED, EDGE>(cp, g, kt);
  load_tile_b<C, GUARD, MASKED, EDGE>(cp, g, kt);
}

// ------------------------------------------------------------------------------------
// Per-workgroup setup shared by every kernel.
// ------------------------------------------------------------------------------------
// How a launch divides the product among workgroups.  Tiles 0 .. split_from-1 (in launch
// order) each run one workgroup over the whole K range into C.  Every later tile runs
// `chunks` workgroups; chunk y multiplies the K range [y*k_chunk, y*k_chunk + k_chunk)
// into a partial product that a reduction kernel then sums.  Workgroups: split_from +
// (tiles - split_from) * chunks, tile-major.
//   plain launch:  split_from = tiles;
//   full split-K:  split_from = 0, chunk y of every tile goes to its M x N plane at
//                  ws + y*plane (rows of N floats);
//   tail split:    split_from = the tiles of the full rounds of workgroups; only the tiles
//                  of the last, partly filled round are split, and chunk y of split tile u
//                  (u = tile - split_from) goes to a packed BM x BN block at
//                  ws + (y * (tiles - split_from) + u) * BM * BN.
struct SplitArgs {
  float* ws;
  int64_t plane;
  int k_chunk;
  int chunks;
  int split_from;
  int tiles;
};

struct SplitWork {
  int bid;    // the tile's index in launch order
  int chunk;  // its K chunk, or -1 for the whole K range
};

// This workgroup's tile and K chunk, with K, A and B moved to the chunk.
template <class PA, class PB>
__device__ __forceinline__ SplitWork split_work(const SplitArgs& sp, int& K, PA& A, PB& B,
                                                int64_t ldb) {
  const int id = blockIdx.x;
  if (id < sp.split_from) return SplitWork{id, -1};
  const int j = id - sp.split_from;
  const int y = j % sp.chunks;
  const int kb = y * sp.k_chunk;
  K = min(K - kb, sp.k_chunk);
  A += kb;
  B += (int64_t)kb * ldb;
  return SplitWork{sp.split_from + j / sp.chunks, y};
}

// Where this workgroup, wave and lane sit, and the copy arguments of the K-loop.
template <class C>
struct TilePos {
  int tid, lane, wave, wm, wn;
  bool m_full, n_full;  // the tile lies inside M (rows) / N (columns)
  LoopArgs<C> g;

  __device__ inline void init(int M, int N, int K, const float* A, int64_t lda,
                              const float* B, int64_t ldb, int flags, int bid, int nwg) {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wm = wave / C::WAVES_N;
    wn = wave % C::WAVES_N;
    int tm, tn;
    tile_coords(bid, nwg, (M + C::BM - 1) / C::BM, (N + C::BN - 1) / C::BN, flags, tm, tn);
    g.A = A;
    g.B = B;
    g.lda = lda;
    g.ldb = ldb;
    g.M = M;
    g.N = N;
    g.K = K;
    g.m0 = tm * C::BM;
    g.n0 = tn * C::BN;
    g.a_bytes = ((int64_t)(M - 1) * lda + K) * 4;
    g.b_bytes = ((int64_t)(K - 1) * ldb + N) * 4;
    m_full = g.m0 + C::BM <= M;
    n_full = g.n0 + C::BN <= N;
    g.vec_a = (flags & kVecA) != 0;
    g.vec_b = (flags & kVecB) != 0;
  }
  // Every K tile of this workgroup can be copied 16 bytes at a time (edge tiles and a K
  // tail included, see the fast path of TileCopy).
  __device__ inline bool unguarded() const { return g.vec_a && g.vec_b; }
};

// Where a K chunk's partial product goes (see SplitArgs): the output pointer is set so
// that the epilogue's usual (row * ldc + column) addressing of the tile lands in the
// chunk's plane or packed block.
template <class C, class PC>
__device__ __forceinline__ void split_output(const SplitArgs& sp, const SplitWork& w, int N,
                                             const TilePos<C>& t, PC& Cmat, int64_t& ldc) {
  if (w.chunk < 0) return;
  if (sp.split_from == 0) {
    Cmat = sp.ws + (int64_t)w.chunk * sp.plane;
    ldc = N;
    return;
  }
  const int64_t slot = (int64_t)w.chunk * (sp.tiles - sp.split_from) + (w.bid - sp.split_from);
  Cmat = sp.ws + slot * (C::BM * C::BN) - ((int64_t)t.g.m0 * C::BN + t.g.n0);
  ldc = C::BN;
}

template <class C>
__device__ inline void zero_acc(floatx16 (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
}

// Epilogue: C is written once, never read.  Lanes 0-31 of a store cover 32 consecutive
// columns of one row and lanes 32-63 the same columns four rows further down; tiles that
// stick out of M x N store only their inside part.
template <class C>
__device__ inline void store_c(const floatx16 (&acc)[C::FM][C::FN], float* Cmat, int64_t ldc,
                               const TilePos<C>& t) {
  const int row0 = t.g.m0 + t.wm * C::TM + 4 * (t.lane >> 5);
  const int col0 = t.g.n0 + t.wn * C::TN + (t.lane & 31);
  if (t.m_full && t.n_full) {
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
          if (row < t.g.M && col < t.g.N) Cmat[(int64_t)row * ldc + col] = acc[fm][fn][r];
        }
  }
}

}  // namespace gemmf32
