// Per-shape dispatch table: (M, N, K) -> variant and tile configuration.
//
// The pages' central measured lesson is that double buffering wins at some sizes and
// loses or ties at others, so a library has to pick a variant per shape ("Double
// Buffering", last two paragraphs; "Case Study: The Double-Buffered GEMM", paragraph on
// the three regimes).  The rows below were measured on MI355X (gfx950) by
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
    {128, 128, 128, 2, 7, 7, 7, 10},  // sb 4.36 us, db 4.35 us, ms 4.58 us
    {127, 193, 61, 2, 6, 6, 6, 6},  // sb 5.15 us, db 5.07 us, ms 5.14 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 8.86 us, db 8.20 us, ms 8.31 us
    {1024, 1024, 1024, 3, 7, 7, 6, 7},  // sb 23.80 us, db 22.27 us, ms 21.49 us
    {256, 1024, 128, 2, 7, 7, 7, 10},  // sb 4.65 us, db 4.65 us, ms 4.83 us
    {1024, 128, 256, 2, 6, 7, 6, 10},  // sb 7.11 us, db 6.99 us, ms 7.09 us
    {4096, 4096, 4096, 2, 1, 9, 1, 8},  // sb 994.83 us, db 937.29 us, ms 952.47 us
    {8192, 8192, 8192, 2, 1, 9, 1, 8},  // sb 8095.20 us, db 7433.89 us, ms 7586.61 us
    {256, 256, 256, 2, 6, 7, 6, 10},  // sb 7.06 us, db 6.94 us, ms 7.03 us
    {512, 512, 512, 3, 10, 7, 6, 10},  // sb 12.21 us, db 11.90 us, ms 11.73 us
    {2048, 2048, 2048, 2, 4, 7, 4, 3},  // sb 139.42 us, db 129.64 us, ms 135.79 us
    {6144, 6144, 6144, 2, 4, 4, 4, 3},  // sb 3459.10 us, db 3308.22 us, ms 3352.21 us
    {64, 4096, 4096, 3, 7, 7, 6, 7},  // sb 96.51 us, db 80.12 us, ms 76.17 us
    {4096, 4096, 512, 2, 2, 9, 2, 8},  // sb 133.53 us, db 128.64 us, ms 131.04 us
    {2048, 8192, 2048, 2, 1, 9, 1, 8},  // sb 501.87 us, db 476.36 us, ms 482.86 us
    {16, 4096, 4096, 2, 7, 7, 7, 7},  // sb 120.42 us, db 106.55 us, ms 106.64 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 123.20 us, db 80.86 us, ms 76.44 us
    {128, 4096, 4096, 3, 7, 7, 6, 7},  // sb 96.70 us, db 80.27 us, ms 76.33 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 248.04 us, db 165.12 us, ms 151.43 us
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
    {16, 4096, 4096, 8},  // 1: 119.6, 2: 63.5, 4: 35.2, 8: 30.2, 16: 33.6
    {32, 4096, 4096, 8},  // 1: 119.6, 2: 63.8, 4: 35.7, 8: 30.5, 16: 33.1
    {64, 4096, 4096, 4},  // 1: 77.3, 2: 43.0, 4: 26.2, 8: 27.3, 16: 31.3
    {128, 4096, 4096, 4},  // 1: 77.3, 2: 43.9, 4: 42.0, 8: 43.7, 16: 47.8
    {32, 8192, 8192, 4},  // 1: 237.3, 2: 124.7, 4: 96.6, 8: 99.3, 16: 105.4
    {64, 8192, 8192, 4},  // 1: 152.2, 2: 82.1, 4: 79.2, 8: 84.3, 16: 92.3
    {256, 256, 8192, 16},  // 1: 151.0, 2: 79.0, 4: 42.5, 8: 25.5, 16: 18.6
    {512, 512, 8192, 8},  // 1: 151.6, 2: 79.9, 4: 43.9, 8: 42.4, 16: 46.1
    {1024, 1024, 1024, 1},  // 1: 21.7, 2: 26.3, 4: 27.4, 8: 31.3, 16: 39.1
    {2048, 2048, 2048, 1},  // 1: 129.3, 2: 137.9, 4: 143.3, 8: 157.9, 16: 194.1
    {4096, 4096, 4096, 1},  // 1: 938.9, 2: 981.0, 4: 1033.1, 8: 1121.1, 16: 1308.6
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
