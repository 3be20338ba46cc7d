// Per-shape dispatch table: (M, N, K) -> variant and tile configuration.
//
// The pages' central measured lesson is that double buffering wins at some sizes and
// loses or ties at others, so a library has to pick a variant per shape ("Double
// Buffering", last two paragraphs; "Case Study: The Double-Buffered GEMM", paragraph on
// the three regimes).  The rows below were measured on AMD Radeon Graphics (gfx950:sramecc+:xnack-) by
// tiled_double_buffered_amd/tune.py (2 rotated rounds x 5 batches of >= 20 ms
// per pair), which rewrites this file; a shape that is not in the table takes the row
// nearest to it in (log2 M, log2 N, log2 K).
//
// Columns: M, N, K, best variant (1 = single-buffered, 2 = double-buffered, 3 = multi-stage
// direct-to-LDS), its tile configuration, and the best configuration of each variant.
// Trailing comments: measured microseconds of the best run of each variant.
#pragma once

#include <cmath>
#include <cstdint>

namespace gemmf32 {

struct DispatchRow {
  int64_t m, n, k;
  int variant, cfg, sb_cfg, db_cfg, ms_cfg;
};

static const DispatchRow kDispatch[] = {
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.45 us, db 4.42 us, ms 4.51 us
    {127, 193, 61, 2, 6, 6, 6, 6},  // sb 5.23 us, db 5.03 us, ms 5.10 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 8.86 us, db 7.93 us, ms 8.04 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.76 us, db 19.71 us, ms 18.91 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 4.72 us, db 4.68 us, ms 4.76 us
    {1024, 128, 256, 3, 6, 7, 6, 6},  // sb 7.10 us, db 6.65 us, ms 6.60 us
    {4096, 4096, 4096, 2, 1, 9, 1, 8},  // sb 991.23 us, db 916.88 us, ms 934.18 us
    {8192, 8192, 8192, 2, 1, 9, 1, 8},  // sb 8092.22 us, db 7260.77 us, ms 7386.64 us
    {256, 256, 256, 3, 6, 7, 6, 6},  // sb 7.07 us, db 6.61 us, ms 6.57 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.22 us, db 10.83 us, ms 10.50 us
    {2048, 2048, 2048, 2, 4, 7, 4, 3},  // sb 139.70 us, db 121.76 us, ms 125.62 us
    {6144, 6144, 6144, 2, 4, 4, 4, 3},  // sb 3456.96 us, db 3189.65 us, ms 3238.56 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 96.27 us, db 69.05 us, ms 64.65 us
    {4096, 4096, 512, 2, 0, 9, 0, 9},  // sb 133.19 us, db 125.99 us, ms 128.76 us
    {2048, 8192, 2048, 2, 0, 9, 0, 8},  // sb 502.22 us, db 466.38 us, ms 474.34 us
    {16, 4096, 4096, 2, 7, 7, 7, 7},  // sb 120.90 us, db 101.65 us, ms 102.15 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 123.10 us, db 73.21 us, ms 65.14 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 96.44 us, db 69.26 us, ms 64.88 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 247.14 us, db 150.22 us, ms 127.74 us
};

static inline double dispatch_log2(int64_t x) { return x > 0 ? std::log2((double)x) : -1.0; }

static inline const DispatchRow& dispatch_nearest(int64_t M, int64_t N, int64_t K) {
  const double lm = dispatch_log2(M), ln = dispatch_log2(N), lk = dispatch_log2(K);
  int best = 0;
  double best_d = 1e300;
  for (int i = 0; i < (int)(sizeof(kDispatch) / sizeof(kDispatch[0])); ++i) {
    const DispatchRow& r = kDispatch[i];
    const double dm = lm - dispatch_log2(r.m), dn = ln - dispatch_log2(r.n),
                 dk = lk - dispatch_log2(r.k);
    const double d = dm * dm + dn * dn + dk * dk;
    if (d < best_d) {
      best_d = d;
      best = i;
    }
  }
  return kDispatch[best];
}

static inline void select_shape(int64_t M, int64_t N, int64_t K, int* variant, int* cfg) {
  const DispatchRow& r = dispatch_nearest(M, N, K);
  *variant = r.variant;
  *cfg = r.cfg;
}

static inline int select_for_variant(int64_t M, int64_t N, int64_t K, int variant) {
  const DispatchRow& r = dispatch_nearest(M, N, K);
  return variant == 1 ? r.sb_cfg : variant == 3 ? r.ms_cfg : r.db_cfg;
}

// Split-K: measured best number of K chunks per shape (1 = do not split), nearest row in
// (log2 M, log2 N, log2 K).  Trailing comments: microseconds of each measured choice.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 8},  // 1: 101.4, 2: 54.6, 4: 31.4, 8: 28.9, 16: 33.7
    {32, 4096, 4096, 8},  // 1: 65.3, 2: 36.7, 4: 23.0, 8: 19.8, 16: 32.8
    {64, 4096, 4096, 4},  // 1: 64.8, 2: 37.0, 4: 23.5, 8: 26.7, 16: 31.3
    {128, 4096, 4096, 2},  // 1: 64.9, 2: 38.4, 4: 40.6, 8: 43.7, 16: 47.7
    {32, 8192, 8192, 4},  // 1: 127.7, 2: 68.4, 4: 46.2, 8: 50.3, 16: 56.3
    {64, 8192, 8192, 2},  // 1: 128.2, 2: 72.7, 4: 76.5, 8: 81.7, 16: 88.5
    {256, 256, 8192, 16},  // 1: 126.2, 2: 66.9, 4: 36.6, 8: 22.7, 16: 17.6
    {512, 512, 8192, 4},  // 1: 127.0, 2: 67.6, 4: 39.1, 8: 40.9, 16: 45.6
    {1024, 1024, 1024, 1},  // 1: 18.9, 2: 25.7, 4: 26.9, 8: 31.3, 16: 38.7
    {2048, 2048, 2048, 1},  // 1: 122.1, 2: 134.1, 4: 140.7, 8: 157.1, 16: 190.4
    {4096, 4096, 4096, 1},  // 1: 924.3, 2: 966.0, 4: 1018.1, 8: 1104.9, 16: 1292.7
};

static inline int select_splits(int64_t M, int64_t N, int64_t K) {
  const double lm = dispatch_log2(M), ln = dispatch_log2(N), lk = dispatch_log2(K);
  int best = 0;
  double best_d = 1e300;
  for (int i = 0; i < (int)(sizeof(kSplitK) / sizeof(kSplitK[0])); ++i) {
    const SplitRow& r = kSplitK[i];
    const double dm = lm - dispatch_log2(r.m), dn = ln - dispatch_log2(r.n),
                 dk = lk - dispatch_log2(r.k);
    const double d = dm * dm + dn * dn + dk * dk;
    if (d < best_d) {
      best_d = d;
      best = i;
    }
  }
  return kSplitK[best].splits;
}

}  // namespace gemmf32
