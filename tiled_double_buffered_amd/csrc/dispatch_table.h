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
// Columns: M, N, K, best variant (1 = single-buffered, 2 = double-buffered), its tile
// configuration, best single-buffered configuration, best double-buffered configuration.
// Trailing comments: measured microseconds of the best single- and double-buffered runs.
#pragma once

#include <cmath>
#include <cstdint>

namespace gemmf32 {

struct DispatchRow {
  int64_t m, n, k;
  int variant, cfg, sb_cfg, db_cfg;
};

static const DispatchRow kDispatch[] = {
    {128, 128, 128, 1, 7, 7, 7},  // sb 4.57 us, db 4.58 us
    {127, 193, 61, 2, 6, 6, 6},  // sb 5.35 us, db 5.25 us
    {513, 257, 129, 2, 6, 6, 6},  // sb 9.09 us, db 8.57 us
    {1024, 1024, 1024, 2, 6, 7, 6},  // sb 24.15 us, db 22.56 us
    {256, 1024, 128, 1, 7, 7, 7},  // sb 4.91 us, db 4.93 us
    {1024, 128, 256, 2, 6, 7, 6},  // sb 7.30 us, db 7.24 us
    {4096, 4096, 4096, 2, 1, 3, 1},  // sb 1022.90 us, db 948.27 us
    {8192, 8192, 8192, 2, 1, 3, 1},  // sb 8203.52 us, db 7496.10 us
    {256, 256, 256, 2, 6, 7, 6},  // sb 7.28 us, db 7.21 us
    {512, 512, 512, 2, 6, 7, 6},  // sb 12.38 us, db 12.12 us
    {2048, 2048, 2048, 2, 4, 7, 4},  // sb 140.76 us, db 130.70 us
    {6144, 6144, 6144, 2, 4, 4, 4},  // sb 3483.24 us, db 3319.05 us
    {64, 4096, 4096, 2, 6, 7, 6},  // sb 96.10 us, db 80.34 us
    {4096, 4096, 512, 2, 2, 3, 2},  // sb 135.36 us, db 129.20 us
    {2048, 8192, 2048, 2, 1, 3, 1},  // sb 514.65 us, db 479.69 us
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
  return variant == 1 ? r.sb_cfg : r.db_cfg;
}

}  // namespace gemmf32
