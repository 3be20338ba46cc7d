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
    {128, 128, 128, 1, 7, 7, 7, 6},  // sb 4.63 us, db 4.63 us, ms 4.79 us
    {127, 193, 61, 2, 6, 6, 6, 6},  // sb 5.31 us, db 5.22 us, ms 5.25 us
    {513, 257, 129, 3, 6, 6, 6, 6},  // sb 9.09 us, db 8.49 us, ms 8.46 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.96 us, db 22.42 us, ms 21.54 us
    {256, 1024, 128, 1, 7, 7, 7, 6},  // sb 4.87 us, db 4.87 us, ms 5.02 us
    {1024, 128, 256, 2, 6, 7, 6, 6},  // sb 7.29 us, db 7.21 us, ms 7.22 us
    {4096, 4096, 4096, 2, 1, 3, 1, 0},  // sb 1011.75 us, db 940.94 us, ms 978.54 us
    {8192, 8192, 8192, 2, 1, 3, 1, 0},  // sb 8142.95 us, db 7414.98 us, ms 7736.04 us
    {256, 256, 256, 2, 6, 7, 6, 6},  // sb 7.26 us, db 7.18 us, ms 7.20 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.36 us, db 12.08 us, ms 11.80 us
    {2048, 2048, 2048, 2, 4, 7, 4, 3},  // sb 140.55 us, db 129.64 us, ms 135.12 us
    {6144, 6144, 6144, 2, 4, 4, 4, 3},  // sb 3471.42 us, db 3318.59 us, ms 3340.08 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 96.02 us, db 80.36 us, ms 75.74 us
    {4096, 4096, 512, 2, 2, 3, 2, 0},  // sb 134.82 us, db 129.02 us, ms 134.30 us
    {2048, 8192, 2048, 2, 1, 3, 1, 0},  // sb 511.14 us, db 477.13 us, ms 497.06 us
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

}  // namespace gemmf32
