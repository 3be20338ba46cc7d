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
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.79 us, db 4.47 us, ms 4.52 us
    {127, 193, 61, 2, 7, 7, 7, 6},  // sb 4.31 us, db 4.28 us, ms 4.32 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 6.46 us, db 5.90 us, ms 5.97 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.74 us, db 18.52 us, ms 17.96 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 5.02 us, db 4.71 us, ms 4.74 us
    {1024, 128, 256, 3, 6, 7, 6, 6},  // sb 7.44 us, db 6.49 us, ms 6.47 us
    {4096, 4096, 4096, 2, 0, 5, 0, 3},  // sb 960.21 us, db 902.68 us, ms 911.33 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7443.01 us, db 7150.15 us, ms 7197.94 us
    {256, 256, 256, 3, 6, 7, 6, 6},  // sb 7.40 us, db 6.47 us, ms 6.45 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.55 us, db 10.29 us, ms 10.10 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.03 us, db 14.48 us, ms 14.04 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 77.24 us, db 68.51 us, ms 68.80 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 127.19 us, db 117.92 us, ms 121.26 us
    {3072, 3072, 3072, 3, 6, 7, 6, 6},  // sb 421.76 us, db 417.91 us, ms 403.43 us
    {6144, 6144, 6144, 3, 3, 4, 4, 3},  // sb 3176.84 us, db 3052.01 us, ms 3051.46 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.86 us, db 65.11 us, ms 60.84 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 127.30 us, db 122.49 us, ms 124.06 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 486.63 us, db 457.56 us, ms 462.29 us
    {4096, 1024, 1024, 2, 3, 7, 3, 6},  // sb 66.35 us, db 61.92 us, ms 63.67 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.93 us, db 127.86 us, ms 121.35 us
    {1023, 1023, 1023, 2, 6, 7, 6, 6},  // sb 25.26 us, db 20.74 us, ms 20.74 us
    {4095, 4095, 4095, 2, 9, 9, 9, 0},  // sb 1003.51 us, db 913.94 us, ms 917.32 us
    {16, 4096, 4096, 3, 6, 7, 6, 6},  // sb 97.49 us, db 70.28 us, ms 69.57 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 98.10 us, db 69.43 us, ms 63.57 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.96 us, db 65.33 us, ms 61.26 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 197.49 us, db 143.35 us, ms 124.26 us
};
constexpr int kDispatchRows = (int)(sizeof(kDispatch) / sizeof(kDispatch[0]));

static inline double dispatch_log2(int64_t x) { return x > 0 ? std::log2((double)x) : -1.0; }

// (log2 M, log2 N, log2 K) of every row, computed once (thread-safe static initialization),
// so that a lookup costs three logarithms instead of three per row.
struct DispatchLogs {
  double v[kDispatchRows][3];
  DispatchLogs() {
    for (int i = 0; i < kDispatchRows; ++i) {
      v[i][0] = dispatch_log2(kDispatch[i].m);
      v[i][1] = dispatch_log2(kDispatch[i].n);
      v[i][2] = dispatch_log2(kDispatch[i].k);
    }
  }
};

static inline const DispatchRow& dispatch_nearest(int64_t M, int64_t N, int64_t K) {
  static const DispatchLogs logs;
  const double lm = dispatch_log2(M), ln = dispatch_log2(N), lk = dispatch_log2(K);
  int best = 0;
  double best_d = 1e300;
  for (int i = 0; i < kDispatchRows; ++i) {
    const double dm = lm - logs.v[i][0], dn = ln - logs.v[i][1], dk = lk - logs.v[i][2];
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
    {16, 4096, 4096, 8},  // 1: 75.6, 2: 42.2, 4: 26.2, 8: 21.4, 16: 22.6
    {32, 4096, 4096, 8},  // 1: 63.5, 2: 35.9, 4: 22.8, 8: 19.6, 16: 28.8
    {64, 4096, 4096, 4},  // 1: 60.9, 2: 35.2, 4: 22.5, 8: 25.8, 16: 29.8
    {128, 4096, 4096, 2},  // 1: 61.2, 2: 36.1, 4: 38.2, 8: 39.8, 16: 45.8
    {32, 8192, 8192, 4},  // 1: 124.3, 2: 67.0, 4: 46.1, 8: 48.7, 16: 55.1
    {64, 8192, 8192, 2},  // 1: 125.1, 2: 73.1, 4: 74.9, 8: 78.5, 16: 86.5
    {256, 256, 8192, 16},  // 1: 117.9, 2: 62.8, 4: 37.3, 8: 23.4, 16: 17.7
    {512, 512, 8192, 4},  // 1: 118.7, 2: 63.8, 4: 36.3, 8: 38.9, 16: 41.0
    {1024, 1024, 1024, 1},  // 1: 17.9, 2: 24.6, 4: 26.2, 8: 30.8, 16: 39.8
    {2048, 2048, 2048, 1},  // 1: 117.9, 2: 145.7, 4: 136.7, 8: 151.4, 16: 191.9
    {4096, 4096, 4096, 1},  // 1: 902.9, 2: 1003.1, 4: 981.3, 8: 1076.1, 16: 1262.5
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
