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
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.43 us, db 4.43 us, ms 4.50 us
    {127, 193, 61, 2, 6, 6, 6, 6},  // sb 5.13 us, db 5.01 us, ms 5.07 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 8.86 us, db 7.92 us, ms 8.02 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.75 us, db 20.48 us, ms 19.31 us
    {256, 1024, 128, 1, 7, 7, 6, 6},  // sb 4.68 us, db 4.70 us, ms 4.73 us
    {1024, 128, 256, 3, 6, 7, 6, 6},  // sb 7.08 us, db 6.75 us, ms 6.61 us
    {4096, 4096, 4096, 2, 1, 9, 1, 9},  // sb 989.81 us, db 924.86 us, ms 934.96 us
    {8192, 8192, 8192, 2, 1, 9, 1, 9},  // sb 8065.19 us, db 7316.10 us, ms 7395.04 us
    {256, 256, 256, 3, 6, 7, 6, 6},  // sb 7.07 us, db 6.73 us, ms 6.60 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.20 us, db 11.16 us, ms 10.60 us
    {2048, 2048, 2048, 2, 4, 7, 4, 3},  // sb 139.36 us, db 123.99 us, ms 125.80 us
    {6144, 6144, 6144, 2, 4, 4, 4, 4},  // sb 3452.80 us, db 3192.19 us, ms 3260.80 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.78 us, db 72.37 us, ms 66.00 us
    {4096, 4096, 512, 2, 2, 9, 2, 9},  // sb 133.30 us, db 126.83 us, ms 127.96 us
    {2048, 8192, 2048, 2, 1, 9, 1, 9},  // sb 501.66 us, db 469.61 us, ms 474.87 us
    {16, 4096, 4096, 2, 7, 7, 7, 10},  // sb 120.72 us, db 101.40 us, ms 101.75 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 123.07 us, db 76.51 us, ms 67.45 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.83 us, db 72.66 us, ms 66.34 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 246.72 us, db 157.68 us, ms 132.25 us
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
    {16, 4096, 4096, 8},  // 1: 101.3, 2: 54.1, 4: 30.6, 8: 27.5, 16: 30.9
    {32, 4096, 4096, 8},  // 1: 67.6, 2: 37.4, 4: 22.4, 8: 19.4, 16: 32.9
    {64, 4096, 4096, 4},  // 1: 67.6, 2: 38.3, 4: 24.4, 8: 29.7, 16: 29.9
    {128, 4096, 4096, 2},  // 1: 68.0, 2: 39.6, 4: 42.8, 8: 43.2, 16: 48.9
    {32, 8192, 8192, 4},  // 1: 132.9, 2: 71.0, 4: 46.2, 8: 50.6, 16: 56.7
    {64, 8192, 8192, 2},  // 1: 133.6, 2: 74.9, 4: 78.6, 8: 89.5, 16: 104.5
    {256, 256, 8192, 16},  // 1: 130.9, 2: 69.9, 4: 38.1, 8: 23.3, 16: 18.2
    {512, 512, 8192, 4},  // 1: 132.2, 2: 70.6, 4: 40.6, 8: 41.2, 16: 45.1
    {1024, 1024, 1024, 1},  // 1: 20.1, 2: 26.8, 4: 27.5, 8: 34.0, 16: 44.8
    {2048, 2048, 2048, 1},  // 1: 123.9, 2: 134.6, 4: 141.4, 8: 156.5, 16: 193.1
    {4096, 4096, 4096, 1},  // 1: 931.4, 2: 973.2, 4: 1022.9, 8: 1112.9, 16: 1296.4
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
