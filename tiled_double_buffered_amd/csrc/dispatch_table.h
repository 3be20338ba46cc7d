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
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.58 us, db 4.39 us, ms 4.46 us
    {127, 193, 61, 3, 6, 6, 6, 6},  // sb 5.23 us, db 5.11 us, ms 5.11 us
    {513, 257, 129, 3, 6, 6, 6, 6},  // sb 8.95 us, db 7.78 us, ms 7.77 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.52 us, db 18.27 us, ms 17.91 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 4.74 us, db 4.46 us, ms 4.66 us
    {1024, 128, 256, 2, 6, 7, 6, 6},  // sb 7.14 us, db 6.25 us, ms 6.39 us
    {4096, 4096, 4096, 2, 1, 9, 1, 3},  // sb 960.86 us, db 901.85 us, ms 914.64 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7434.30 us, db 7155.08 us, ms 7238.40 us
    {256, 256, 256, 2, 6, 7, 6, 6},  // sb 7.12 us, db 6.27 us, ms 6.38 us
    {512, 512, 512, 2, 6, 7, 6, 6},  // sb 12.28 us, db 10.04 us, ms 10.05 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 17.74 us, db 14.21 us, ms 13.91 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 77.41 us, db 68.47 us, ms 68.93 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 127.27 us, db 117.95 us, ms 121.40 us
    {3072, 3072, 3072, 3, 6, 7, 6, 6},  // sb 422.96 us, db 417.88 us, ms 406.66 us
    {6144, 6144, 6144, 2, 4, 4, 4, 3},  // sb 3189.78 us, db 3060.80 us, ms 3063.22 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.11 us, db 64.82 us, ms 60.75 us
    {4096, 4096, 512, 2, 2, 4, 2, 3},  // sb 128.00 us, db 122.20 us, ms 124.03 us
    {2048, 8192, 2048, 2, 2, 4, 2, 3},  // sb 486.43 us, db 457.18 us, ms 463.14 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 67.09 us, db 61.64 us, ms 63.67 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.59 us, db 127.87 us, ms 122.01 us
    {16, 4096, 4096, 2, 10, 7, 10, 10},  // sb 116.15 us, db 98.37 us, ms 99.12 us
    {32, 4096, 4096, 3, 10, 10, 10, 10},  // sb 120.25 us, db 69.00 us, ms 63.14 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.11 us, db 64.81 us, ms 60.82 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 241.83 us, db 143.57 us, ms 124.43 us
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
    {16, 4096, 4096, 8},  // 1: 98.2, 2: 53.2, 4: 30.8, 8: 22.5, 16: 22.7
    {32, 4096, 4096, 8},  // 1: 63.4, 2: 35.6, 4: 22.0, 8: 19.0, 16: 29.8
    {64, 4096, 4096, 4},  // 1: 60.8, 2: 34.7, 4: 21.7, 8: 24.4, 16: 27.0
    {128, 4096, 4096, 2},  // 1: 61.0, 2: 35.7, 4: 37.2, 8: 39.6, 16: 46.8
    {32, 8192, 8192, 4},  // 1: 124.0, 2: 67.0, 4: 46.3, 8: 48.4, 16: 55.1
    {64, 8192, 8192, 2},  // 1: 125.2, 2: 68.7, 4: 71.8, 8: 77.6, 16: 85.4
    {256, 256, 8192, 16},  // 1: 117.6, 2: 67.2, 4: 37.1, 8: 23.2, 16: 17.4
    {512, 512, 8192, 4},  // 1: 118.9, 2: 63.7, 4: 37.0, 8: 39.1, 16: 41.1
    {1024, 1024, 1024, 1},  // 1: 17.9, 2: 24.6, 4: 25.3, 8: 31.2, 16: 39.5
    {2048, 2048, 2048, 1},  // 1: 118.4, 2: 128.5, 4: 137.0, 8: 151.7, 16: 191.3
    {4096, 4096, 4096, 1},  // 1: 910.2, 2: 951.8, 4: 983.6, 8: 1085.1, 16: 1260.3
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
