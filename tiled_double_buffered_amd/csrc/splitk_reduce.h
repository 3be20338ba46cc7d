// The split-K reduction kernel of gemmf32.
#pragma once

#include "gemm_common.h"

namespace gemmf32 {

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

// Tail split: only the tiles split_from .. tiles-1 (in launch order) were split; chunk y
// of split tile u is a packed bm x bn block at P + (y * U + u) * bm * bn (U split tiles),
// and the sum P[0] + P[1] + ... + P[S-1] is taken in that order as above.  Workgroup
// (u, b) sums elements b*256 .. b*256+255 of split tile u, one per thread, its S loads
// issued ahead of the additions; the tile's place in C comes from the same launch-order
// -> tile mapping as in the GEMM launch (tile configuration bm x bn, the same flags).
__global__ void __launch_bounds__(256)
gemm_f32_splitk_reduce_tiles(int M, int N, int S, const float* __restrict__ P,
                             float* __restrict__ C, int64_t ldc, int bm, int bn,
                             int split_from, int tiles, int flags) {
  const int u = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int r = e / bn, c = e % bn;
  int tm, tn;
  tile_coords(split_from + u, tiles, (M + bm - 1) / bm, (N + bn - 1) / bn, flags, tm, tn);
  const int i = tm * bm + r, j = tn * bn + c;
  if (r >= bm || i >= M || j >= N) return;
  const int64_t block = (int64_t)bm * bn;
  const int64_t chunk = (int64_t)(tiles - split_from) * block;
  const float* p = P + (int64_t)u * block + e;
  float acc = p[0];
  int sp = 1;
  for (; sp + 4 <= S; sp += 4) {
    const float v0 = p[sp * chunk], v1 = p[(sp + 1) * chunk], v2 = p[(sp + 2) * chunk],
                v3 = p[(sp + 3) * chunk];
    acc += v0;
    acc += v1;
    acc += v2;
    acc += v3;
  }
  for (; sp < S; ++sp) acc += p[sp * chunk];
  C[(int64_t)i * ldc + j] = acc;
}

}  // namespace gemmf32
