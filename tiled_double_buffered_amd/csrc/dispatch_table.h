// Per-shape dispatch table: (M, N, K) -> variant and tile configuration.
//
// The pages' central measured lesson is that double buffering wins at some sizes and
// loses or ties at others, so a library has to pick a variant per shape ("Double
// Buffering", last two paragraphs; "Case Study: The Double-Buffered GEMM", paragraph on
// the three regimes).  The rows below were measured on AMD Radeon Graphics (gfx950:sramecc+:xnack-) by
// tiled_double_buffered_amd/tune.py (2 rotated rounds x 5 batches of >= 20 ms
// per pair), which rewrites this file.  A shape in the table takes its measured pick; any
// other shape takes the pick of the cost model further down, fitted to the same runs.
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
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.81 us, db 4.69 us, ms 4.76 us
    {127, 193, 61, 1, 7, 7, 6, 7},  // sb 4.55 us, db 4.58 us, ms 4.60 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 6.49 us, db 5.93 us, ms 6.03 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.76 us, db 18.54 us, ms 17.98 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 5.02 us, db 4.72 us, ms 4.76 us
    {1024, 128, 256, 3, 6, 7, 6, 6},  // sb 7.44 us, db 6.52 us, ms 6.49 us
    {4096, 4096, 4096, 2, 0, 9, 0, 8},  // sb 962.85 us, db 909.98 us, ms 919.79 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7459.57 us, db 7198.21 us, ms 7239.15 us
    {256, 256, 256, 3, 6, 7, 6, 6},  // sb 7.43 us, db 6.45 us, ms 6.42 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.58 us, db 10.31 us, ms 10.12 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.06 us, db 14.49 us, ms 14.05 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 77.21 us, db 68.59 us, ms 68.78 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 127.85 us, db 118.23 us, ms 121.70 us
    {3072, 3072, 3072, 3, 6, 7, 6, 6},  // sb 426.68 us, db 422.58 us, ms 407.06 us
    {6144, 6144, 6144, 3, 3, 4, 4, 3},  // sb 3188.94 us, db 3061.77 us, ms 3060.85 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.64 us, db 65.18 us, ms 61.10 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 128.09 us, db 123.19 us, ms 124.79 us
    {2048, 8192, 2048, 2, 2, 9, 2, 8},  // sb 487.98 us, db 458.02 us, ms 466.23 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 66.70 us, db 61.99 us, ms 63.79 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.92 us, db 128.79 us, ms 122.49 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.30 us, db 21.03 us, ms 20.79 us
    {4095, 4095, 4095, 2, 9, 9, 9, 0},  // sb 999.12 us, db 916.25 us, ms 924.16 us
    {16, 4096, 4096, 3, 6, 7, 6, 6},  // sb 97.43 us, db 70.26 us, ms 69.49 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 97.83 us, db 69.37 us, ms 63.40 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.72 us, db 65.15 us, ms 61.12 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 198.26 us, db 144.27 us, ms 124.57 us
};
constexpr int kDispatchRows = (int)(sizeof(kDispatch) / sizeof(kDispatch[0]));

static inline double dispatch_log2(int64_t x) { return x > 0 ? std::log2((double)x) : -1.0; }

static inline const DispatchRow* dispatch_exact(int64_t M, int64_t N, int64_t K) {
  for (int i = 0; i < kDispatchRows; ++i)
    if (kDispatch[i].m == M && kDispatch[i].n == N && kDispatch[i].k == K) return &kDispatch[i];
  return nullptr;
}

// Cost model of every (variant, configuration) for shapes outside the table.  The features
// are the two the regimes turn on: how many tiles the busiest compute unit multiplies,
// rounds = ceil(workgroups / 256), and the K tiles per tile, k_tiles = ceil(K / BK).  A
// launch is modelled as
//     a + g * rounds * k_tiles   microseconds,
// a being the fixed cost (launch, first copy, epilogue) and g the time of one K tile of one
// round.  a and g were fitted per pair by least squares on relative error, both kept
// >= 0, to the 74 shapes measured for this file (the table's 26 and 48 seeded
// shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, g_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.5674, 4.10572},  // median |error| 3.4%
    {1, 1, 9.4552, 7.82883},  // median |error| 2.2%
    {1, 2, 6.0537, 2.21105},  // median |error| 4.4%
    {1, 3, 3.8813, 1.20448},  // median |error| 7.6%
    {1, 4, 4.1597, 2.21729},  // median |error| 5.0%
    {1, 5, 3.4672, 1.19244},  // median |error| 7.1%
    {1, 6, 3.3127, 0.63058},  // median |error| 10.0%
    {1, 7, 3.2708, 1.17486},  // median |error| 7.6%
    {1, 8, 6.2370, 7.69616},  // median |error| 2.0%
    {1, 9, 4.4140, 4.04300},  // median |error| 2.1%
    {1, 10, 3.3128, 0.65921},  // median |error| 10.2%
    {2, 0, 10.2762, 3.47966},  // median |error| 1.3%
    {2, 1, 10.6630, 6.96635},  // median |error| 1.3%
    {2, 2, 6.5401, 1.76496},  // median |error| 1.3%
    {2, 3, 4.3756, 0.91607},  // median |error| 1.7%
    {2, 4, 4.5750, 1.78336},  // median |error| 1.2%
    {2, 5, 4.0593, 0.93737},  // median |error| 1.8%
    {2, 6, 3.3433, 0.50129},  // median |error| 4.1%
    {2, 7, 3.4119, 1.04691},  // median |error| 3.6%
    {2, 8, 7.0341, 7.09064},  // median |error| 1.0%
    {2, 9, 5.1901, 3.51445},  // median |error| 1.1%
    {2, 10, 3.3231, 0.53594},  // median |error| 4.5%
    {3, 0, 10.4842, 3.55750},  // median |error| 2.2%
    {3, 1, 10.3217, 7.13801},  // median |error| 2.3%
    {3, 2, 6.7027, 1.80775},  // median |error| 2.1%
    {3, 3, 4.6181, 0.91260},  // median |error| 1.8%
    {3, 4, 4.5367, 1.84703},  // median |error| 2.0%
    {3, 5, 4.1379, 0.96627},  // median |error| 1.8%
    {3, 6, 3.4314, 0.49893},  // median |error| 4.6%
    {3, 7, 3.3658, 1.09070},  // median |error| 4.2%
    {3, 8, 7.6671, 7.08704},  // median |error| 1.1%
    {3, 9, 5.0893, 3.55513},  // median |error| 1.3%
    {3, 10, 3.3973, 0.52273},  // median |error| 5.3%
};
constexpr int kModelRows = (int)(sizeof(kModel) / sizeof(kModel[0]));
constexpr int64_t kModelCUs = 256;

// Modelled microseconds of one launch; wg_factor multiplies the workgroup count (the K
// chunks of a split-K launch run side by side in one grid).
static inline double model_us(const ModelRow& r, int64_t M, int64_t N, int64_t K,
                              int64_t wg_factor) {
  const CfgEntry& e = kConfigs[r.cfg];
  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn) * wg_factor;
  const int64_t rounds = (tiles + kModelCUs - 1) / kModelCUs;
  const int64_t k_tiles = (K + e.bk - 1) / e.bk;
  return r.a_us + r.g_us * (double)rounds * (double)k_tiles;
}

// The row with the least modelled time (variant 0: any variant), first row on ties.
static inline const ModelRow& model_pick(int64_t M, int64_t N, int64_t K, int variant,
                                         int64_t wg_factor) {
  int best = 0;
  double best_t = 0.0;
  bool found = false;
  for (int i = 0; i < kModelRows; ++i) {
    if (variant != 0 && kModel[i].variant != variant) continue;
    const double t = model_us(kModel[i], M, N, K, wg_factor);
    if (!found || t < best_t) {
      best = i;
      best_t = t;
      found = true;
    }
  }
  return kModel[best];
}

static inline void select_shape(int64_t M, int64_t N, int64_t K, int* variant, int* cfg) {
  if (const DispatchRow* r = dispatch_exact(M, N, K)) {
    *variant = r->variant;
    *cfg = r->cfg;
    return;
  }
  const ModelRow& m = model_pick(M, N, K, 0, 1);
  *variant = m.variant;
  *cfg = m.cfg;
}

static inline int select_for_variant(int64_t M, int64_t N, int64_t K, int variant) {
  if (const DispatchRow* r = dispatch_exact(M, N, K))
    return variant == 1 ? r->sb_cfg : variant == 3 ? r->ms_cfg : r->db_cfg;
  return model_pick(M, N, K, variant, 1).cfg;
}

// Split-K: measured best number of K chunks per shape (1 = do not split), nearest row in
// (log2 M, log2 N, log2 K).  Trailing comments: microseconds of each measured choice.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 8},  // 1: 69.5, 2: 38.6, 4: 22.8, 8: 19.9, 16: 21.9
    {32, 4096, 4096, 8},  // 1: 63.4, 2: 39.0, 4: 23.4, 8: 19.1, 16: 22.1
    {64, 4096, 4096, 4},  // 1: 60.8, 2: 34.8, 4: 21.8, 8: 24.3, 16: 29.6
    {128, 4096, 4096, 2},  // 1: 61.0, 2: 35.8, 4: 37.8, 8: 39.6, 16: 43.7
    {32, 8192, 8192, 4},  // 1: 124.2, 2: 73.0, 4: 46.5, 8: 48.6, 16: 55.2
    {64, 8192, 8192, 2},  // 1: 119.4, 2: 72.3, 4: 74.6, 8: 78.4, 16: 86.8
    {256, 256, 8192, 16},  // 1: 118.1, 2: 62.9, 4: 34.8, 8: 21.8, 16: 17.1
    {512, 512, 8192, 4},  // 1: 119.1, 2: 63.5, 4: 36.9, 8: 39.0, 16: 40.7
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.6, 4: 25.4, 8: 30.2, 16: 39.6
    {2048, 2048, 2048, 1},  // 1: 118.2, 2: 130.6, 4: 140.1, 8: 158.4, 16: 206.3
    {4096, 4096, 4096, 1},  // 1: 907.6, 2: 949.6, 4: 992.8, 8: 1101.4, 16: 1295.1
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
