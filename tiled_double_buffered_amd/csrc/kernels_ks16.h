// The 16-row K-split kernel of gemmf32: few output rows against a wide B and a long K.
#pragma once

#include "gemm_common.h"

namespace gemmf32 {

// ------------------------------------------------------------------------------------
// Products with at most a few rows (the skinny regime the case study places LLM decode in:
// "Case Study: The Double-Buffered GEMM", paragraph on the three regimes) read B once and
// do little arithmetic per byte: at 16 x 4096 x 4096, B is 64 MiB and the product 0.5
// GFLOP, so reading B bounds the time.  The 32 x 32 blocks of the other kernels waste half
// their rows at M = 16, and a 32-column tile gives only 128 tiles at N = 4096.
//
// Here a workgroup owns a 16 x 16 CB tile of C (CB = 1: 256 tiles at N = 4096, one per
// compute unit) and its WAVES waves split the tile's K range: wave w multiplies its share
// of the K groups (KG k each) on v_mfma_f32_16x16x4_f32, one accumulator per 16-column
// block, then the waves' sums meet in LDS and are added in wave order.  Deterministic; no
// workspace.  Wider tiles (CB = 2, 4) read B in 128- and 256-byte row segments and load
// each A fragment once for CB blocks; they pay off where N leaves enough tiles.
//
// A K group's operands are used by one wave only, so nothing is shared through LDS: each
// wave loads them straight into the matrix instruction's operand registers, two register
// sets in turn -- group g + 1 is in flight while group g is multiplied (the prefetch of the
// next tile into the idle buffer, with registers as the buffers).  For the instruction,
// lane l supplies A[l mod 16][kk] and B[kk][l mod 16] with kk = l div 16, and register i of
// lane l receives D[4 (l div 16) + i][l mod 16].  Lane l (r = l mod 16, s = l div 16) reads
// A[r][k0 + 4s .. 4s + 3] with one 16-byte load per 16 k, and B[k0 + 4s + t][16c + r] for
// t = 0..3 and each block c with one 4-byte load each, so that step t of the 16 k consumes
// its k values k0 + 4s + t: the four steps cover the 16 k once each.
// ------------------------------------------------------------------------------------
template <int WAVES_, int BLOCKS_ = 4, bool STRIDED_ = false, int CB_ = 1>
struct Ks16Cfg {
  static constexpr int WAVES = WAVES_;
  static constexpr int NT = 64 * WAVES;
  static constexpr int CB = CB_;            // 16-column blocks of the tile
  static constexpr int BM = 16, BN = 16 * CB;
  static constexpr int BLOCKS = BLOCKS_;    // 16-k blocks per group
  static constexpr int KG = 16 * BLOCKS;    // k per group
  // STRIDED: wave w takes groups w, w + WAVES, w + 2 WAVES, ... (the workgroup walks K in
  // one front); otherwise a contiguous share of the groups
  static constexpr bool STRIDED = STRIDED_;
  static_assert(NT <= 1024, "threads of one workgroup");
  static_assert(NT >= 256, "the hand-off sums each 256-element column block with 256 threads");
};

// One group's operands in this lane's registers.
template <class D>
struct Ks16Set {
  floatx4 a[D::BLOCKS];            // A[r][k0 + 16j + 4s + t], t = 0..3
  float b[D::BLOCKS][D::CB][4];    // B[k0 + 16j + 4s + t][16c + r]
};

template <class D>
struct Ks16Loader {
  int M, N, K;
  const float* A;
  const float* B;
  int64_t lda, ldb;
  int64_t a_bytes, b_bytes;  // byte extents of A and B from A and B
  int m0, n0, r, s;
  uint32_t a_off;            // this lane's byte offset from a group's A origin
  uint32_t b_off[4];         // ... from the B origin of a 16-k block, for step t

  // 16-byte and 4-byte buffer loads from a workgroup-uniform base; past the range (rows of
  // A at or past M, rows of B at or past K) they read 0.  The host takes this path only when
  // every offset inside a 16-row block of A or B fits 32 bits.
  static __device__ inline __amdgpu_buffer_rsrc_t rsrc(const float* base, uint32_t range) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)range,
                                             kBufferFlags);
  }
  // Bytes of the operand left from element `first` on, clamped to a descriptor's range;
  // the clamp looks at the two 32-bit halves so that it stays in scalar instructions.
  static __device__ inline uint32_t range_from(int64_t bytes, int64_t first) {
    const int64_t left = bytes - first * 4;
    const int hi = (int)(left >> 32);
    const uint32_t lo = (uint32_t)left;
    return hi < 0 ? 0u : hi > 0 ? kBufferRange : lo < kBufferRange ? lo : kBufferRange;
  }

  __device__ inline void load_fast(int g, Ks16Set<D>& st) const {
    const int k0 = g * D::KG;
    const int64_t a_first = (int64_t)m0 * lda + k0;
    const auto ra = rsrc(A + a_first, range_from(a_bytes, a_first));
#pragma unroll
    for (int j = 0; j < D::BLOCKS; ++j)
      st.a[j] = __builtin_bit_cast(
          floatx4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(a_off + 64 * j), 0, 0));
#pragma unroll
    for (int j = 0; j < D::BLOCKS; ++j) {
      const int64_t b_first = (int64_t)(k0 + 16 * j) * ldb + n0;
      const auto rb = rsrc(B + b_first, range_from(b_bytes, b_first));
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int c = 0; c < D::CB; ++c)
          st.b[j][c][t] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rb, (int)(b_off[t] + 64 * c), 0, 0));
    }
  }

  // Element by element, anything outside M x K (A) or K x N (B) reads 0.
  __device__ inline void load_guarded(int g, Ks16Set<D>& st) const {
    const int k0 = g * D::KG;
    const int row = m0 + r;
#pragma unroll
    for (int j = 0; j < D::BLOCKS; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = k0 + 16 * j + 4 * s + t;
        st.a[j][t] = (row < M && k < K) ? A[(int64_t)row * lda + k] : 0.0f;
#pragma unroll
        for (int c = 0; c < D::CB; ++c) {
          const int col = n0 + 16 * c + r;
          st.b[j][c][t] = (k < K && col < N) ? B[(int64_t)k * ldb + col] : 0.0f;
        }
      }
  }

  // The group that holds k = K - 1 when K is not a multiple of KG: A's columns >= K
  // (padding or the next row) are zeroed so that they add exact zeros against B's zero rows.
  __device__ inline void mask_tail(int g, Ks16Set<D>& st) const {
    const int k0 = g * D::KG;
#pragma unroll
    for (int j = 0; j < D::BLOCKS; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        st.a[j][t] = k0 + 16 * j + 4 * s + t < K ? st.a[j][t] : 0.0f;
  }
};

template <class D>
__device__ __forceinline__ void ks16_mfma(const Ks16Set<D>& st, floatx4 (&acc)[D::CB]) {
#pragma unroll
  for (int j = 0; j < D::BLOCKS; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int c = 0; c < D::CB; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(st.a[j][t], st.b[j][c][t], acc[c], 0, 0,
                                                      0);
}

// Groups g0, g0 + gs, ... below g1 of one wave, two register sets in turn; FAST: buffer
// loads.
template <class D, bool FAST>
__device__ inline void ks16_loop(const Ks16Loader<D>& ld, int g0, int g1, int gs,
                                 floatx4 (&acc)[D::CB]) {
  const int tail = ld.K % D::KG ? (ld.K - 1) / D::KG : -1;  // the group to mask, if any
  Ks16Set<D> s0, s1;
  auto load = [&](int g, Ks16Set<D>& st) {
    if constexpr (FAST) ld.load_fast(g, st);
    else ld.load_guarded(g, st);
  };
  auto use = [&](int g, Ks16Set<D>& st) {
    if constexpr (FAST) {
      if (g == tail) ld.mask_tail(g, st);
    }
    ks16_mfma<D>(st, acc);
  };
  if (g0 >= g1) return;
  load(g0, s0);
  int g = g0;
  for (; g + 2 * gs < g1; g += 2 * gs) {
    load(g + gs, s1);
    use(g, s0);
    load(g + 2 * gs, s0);
    use(g + gs, s1);
  }
  if (g + gs < g1) {
    load(g + gs, s1);
    use(g, s0);
    use(g + gs, s1);
  } else {
    use(g, s0);
  }
}

template <class D>
__global__ void __launch_bounds__(D::NT)
gemm_f32_ks16_kernel(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                     const float* __restrict__ B, int64_t ldb, float* __restrict__ Cmat,
                     int64_t ldc, int flags, SplitArgs sp) {
  __shared__ __attribute__((aligned(16))) float red[D::WAVES * 256 * D::CB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_coords(blockIdx.x, sp.tiles, (M + D::BM - 1) / D::BM, (N + D::BN - 1) / D::BN, flags,
              tm, tn);
  Ks16Loader<D> ld;
  ld.M = M;
  ld.N = N;
  ld.K = K;
  ld.A = A;
  ld.B = B;
  ld.lda = lda;
  ld.ldb = ldb;
  ld.a_bytes = ((int64_t)(M - 1) * lda + K) * 4;
  ld.b_bytes = ((int64_t)(K - 1) * ldb + N) * 4;
  ld.m0 = tm * D::BM;
  ld.n0 = tn * D::BN;
  ld.r = lane & 15;
  ld.s = lane >> 4;
  ld.a_off = (uint32_t)(((int64_t)ld.r * lda + 4 * ld.s) * 4);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    ld.b_off[t] = (uint32_t)(((int64_t)(4 * ld.s + t) * ldb + ld.r) * 4);

  // This wave's share of the K groups: every WAVES-th group from its own (STRIDED), or a
  // contiguous run as even as integer division makes it.
  const int groups = (K + D::KG - 1) / D::KG;
  int g0, g1, gs;
  if constexpr (D::STRIDED) {
    g0 = wave;
    g1 = groups;
    gs = D::WAVES;
  } else {
    g0 = (int)((int64_t)groups * wave / D::WAVES);
    g1 = (int)((int64_t)groups * (wave + 1) / D::WAVES);
    gs = 1;
  }
  floatx4 acc[D::CB];
#pragma unroll
  for (int c = 0; c < D::CB; ++c) acc[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  if ((flags & kVecA) && (flags & kVecB))
    ks16_loop<D, true>(ld, g0, g1, gs, acc);
  else
    ks16_loop<D, false>(ld, g0, g1, gs, acc);

  // Hand-off: register i of lane l of wave w, column block c, goes to red[w][c][i][l];
  // then element e (e = tid, tid + NT, ... below 256 CB) is added over the WAVES sums in
  // wave order and stored: column block c = e div 256, row 4 (l div 16) + i, column
  // 16 c + l mod 16 of the tile, with i = (e div 64) mod 4 and l = e mod 64.
#pragma unroll
  for (int c = 0; c < D::CB; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * D::CB + c) * 256 + i * 64 + lane] = acc[c][i];
  __syncthreads();
#pragma unroll
  for (int e0 = 0; e0 < 256 * D::CB; e0 += D::NT) {
    const int e = e0 + tid;
    if (e < 256 * D::CB) {
      float sum = red[e];
#pragma unroll
      for (int w = 1; w < D::WAVES; ++w) sum += red[w * 256 * D::CB + e];
      const int c = e >> 8, l = e & 63, i = (e >> 6) & 3;
      const int row = ld.m0 + 4 * (l >> 4) + i, col = ld.n0 + 16 * c + (l & 15);
      if (row < M && col < N) Cmat[(int64_t)row * ldc + col] = sum;
    }
  }
}

}  // namespace gemmf32
