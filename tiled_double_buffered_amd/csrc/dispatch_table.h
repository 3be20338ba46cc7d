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
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.65 us, db 4.28 us, ms 4.48 us
    {127, 193, 61, 2, 6, 6, 6, 6},  // sb 5.24 us, db 5.04 us, ms 5.05 us
    {513, 257, 129, 3, 6, 6, 6, 6},  // sb 8.96 us, db 7.80 us, ms 7.79 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.49 us, db 18.24 us, ms 17.93 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 4.85 us, db 4.47 us, ms 4.70 us
    {1024, 128, 256, 2, 6, 7, 6, 6},  // sb 7.16 us, db 6.27 us, ms 6.45 us
    {4096, 4096, 4096, 2, 1, 7, 1, 3},  // sb 953.50 us, db 903.45 us, ms 914.58 us
    {8192, 8192, 8192, 2, 2, 3, 2, 3},  // sb 7407.52 us, db 7166.92 us, ms 7202.52 us
    {256, 256, 256, 2, 6, 7, 6, 6},  // sb 7.13 us, db 6.25 us, ms 6.41 us
    {512, 512, 512, 2, 6, 7, 6, 6},  // sb 12.23 us, db 10.03 us, ms 10.05 us
    {2048, 2048, 2048, 2, 3, 6, 3, 6},  // sb 124.48 us, db 117.82 us, ms 120.52 us
    {6144, 6144, 6144, 2, 4, 4, 4, 3},  // sb 3171.01 us, db 3051.21 us, ms 3057.85 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.21 us, db 64.88 us, ms 61.00 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 128.32 us, db 122.37 us, ms 124.91 us
    {2048, 8192, 2048, 2, 2, 7, 2, 3},  // sb 484.53 us, db 457.29 us, ms 462.59 us
    {16, 4096, 4096, 2, 10, 7, 10, 10},  // sb 115.59 us, db 98.35 us, ms 99.30 us
    {32, 4096, 4096, 3, 10, 10, 10, 10},  // sb 120.45 us, db 69.07 us, ms 63.05 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.45 us, db 64.80 us, ms 61.20 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 242.10 us, db 143.74 us, ms 123.84 us
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
    {16, 4096, 4096, 8},  // 1: 99.6, 2: 53.7, 4: 30.6, 8: 27.5, 16: 30.9
    {32, 4096, 4096, 8},  // 1: 62.9, 2: 35.4, 4: 22.1, 8: 19.3, 16: 29.8
    {64, 4096, 4096, 4},  // 1: 60.7, 2: 34.7, 4: 21.7, 8: 24.4, 16: 26.9
    {128, 4096, 4096, 2},  // 1: 60.9, 2: 35.5, 4: 36.6, 8: 38.4, 16: 46.5
    {32, 8192, 8192, 4},  // 1: 123.8, 2: 66.5, 4: 46.3, 8: 48.2, 16: 54.8
    {64, 8192, 8192, 2},  // 1: 124.0, 2: 66.0, 4: 68.8, 8: 74.7, 16: 82.5
    {256, 256, 8192, 16},  // 1: 118.2, 2: 62.7, 4: 34.6, 8: 21.7, 16: 16.9
    {512, 512, 8192, 4},  // 1: 118.8, 2: 63.6, 4: 35.9, 8: 37.8, 16: 43.1
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.7, 4: 26.1, 8: 31.1, 16: 38.5
    {2048, 2048, 2048, 1},  // 1: 117.9, 2: 128.6, 4: 138.1, 8: 157.5, 16: 199.8
    {4096, 4096, 4096, 1},  // 1: 903.9, 2: 946.6, 4: 988.7, 8: 1096.1, 16: 1284.7
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
