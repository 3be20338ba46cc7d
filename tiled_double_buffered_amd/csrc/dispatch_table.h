// Per-shape dispatch table: (M, N, K) -> variant and tile configuration.
//
// The pages' central measured lesson is that double buffering wins at some sizes and
// loses or ties at others, so a library has to pick a variant per shape ("Double
// Buffering", last two paragraphs; "Case Study: The Double-Buffered GEMM", paragraph on
// the three regimes).  The rows below are measured on MI355X by the tuning sweep in
// tiled_double_buffered_amd/tune.py, which rewrites this file; a shape that is not in the
// table takes the row nearest to it in (log2 M, log2 N, log2 K).
//
// Columns: M, N, K, best variant (1 = single-buffered, 2 = double-buffered), its tile
// configuration, best single-buffered configuration, best double-buffered configuration.
#pragma once

#include <cmath>
#include <cstdint>

namespace gemmf32 {

struct DispatchRow {
  int64_t m, n, k;
  int variant, cfg, sb_cfg, db_cfg;
};

// Interim rows from a first sweep (one run per configuration, not yet counterbalanced).
static const DispatchRow kDispatch[] = {
    {128, 128, 128, 2, 7, 7, 7},
    {127, 193, 61, 2, 7, 7, 7},
    {513, 257, 129, 2, 7, 7, 7},
    {1024, 1024, 1024, 2, 7, 7, 7},
    {256, 1024, 128, 2, 7, 7, 7},
    {1024, 128, 256, 2, 7, 7, 7},
    {4096, 4096, 4096, 1, 3, 3, 1},
    {8192, 8192, 8192, 2, 2, 3, 2},
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
