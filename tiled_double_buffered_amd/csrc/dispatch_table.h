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
    {128, 128, 128, 2, 6, 7, 6, 6},  // sb 4.79 us, db 4.48 us, ms 4.51 us
    {127, 193, 61, 2, 7, 7, 7, 7},  // sb 4.19 us, db 4.15 us, ms 4.18 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 6.45 us, db 5.92 us, ms 5.98 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.72 us, db 18.55 us, ms 17.97 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 4.98 us, db 4.69 us, ms 4.72 us
    {1024, 128, 256, 3, 6, 7, 6, 6},  // sb 7.41 us, db 6.46 us, ms 6.44 us
    {4096, 4096, 4096, 2, 0, 9, 0, 3},  // sb 967.15 us, db 907.21 us, ms 918.32 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7435.37 us, db 7169.95 us, ms 7243.42 us
    {256, 256, 256, 3, 6, 7, 6, 6},  // sb 7.38 us, db 6.46 us, ms 6.44 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.55 us, db 10.29 us, ms 10.09 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.10 us, db 14.51 us, ms 14.07 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 77.22 us, db 69.00 us, ms 69.01 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 127.95 us, db 118.15 us, ms 121.56 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 426.36 us, db 386.39 us, ms 401.51 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3195.06 us, db 3050.72 us, ms 3066.50 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.32 us, db 65.15 us, ms 60.91 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 127.49 us, db 123.14 us, ms 124.68 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 487.67 us, db 459.34 us, ms 463.65 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 66.75 us, db 61.97 us, ms 63.78 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 191.05 us, db 128.71 us, ms 122.64 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.16 us, db 21.10 us, ms 20.74 us
    {4095, 4095, 4095, 2, 0, 9, 0, 0},  // sb 1005.94 us, db 919.57 us, ms 920.66 us
    {16, 4096, 4096, 3, 6, 7, 6, 6},  // sb 97.70 us, db 70.21 us, ms 69.54 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 98.09 us, db 69.60 us, ms 63.57 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.54 us, db 65.13 us, ms 61.14 us
    {32, 8192, 8192, 3, 10, 7, 7, 10},  // sb 196.96 us, db 143.04 us, ms 124.04 us
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
    {1, 0, 9.5762, 4.10180},  // median |error| 3.3%
    {1, 1, 9.4564, 7.82131},  // median |error| 2.3%
    {1, 2, 6.0338, 2.20983},  // median |error| 4.3%
    {1, 3, 3.8545, 1.20407},  // median |error| 7.5%
    {1, 4, 4.1413, 2.21554},  // median |error| 5.1%
    {1, 5, 3.4404, 1.19323},  // median |error| 7.2%
    {1, 6, 3.0823, 0.63464},  // median |error| 10.3%
    {1, 7, 3.0535, 1.18353},  // median |error| 7.6%
    {1, 8, 6.2496, 7.68663},  // median |error| 2.0%
    {1, 9, 4.4084, 4.04096},  // median |error| 2.2%
    {1, 10, 3.1288, 0.66092},  // median |error| 10.6%
    {1, 11, 6.0678, 2.52124},  // median |error| 4.2%
    {1, 12, 6.5667, 4.68467},  // median |error| 2.9%
    {2, 0, 10.2937, 3.47376},  // median |error| 1.1%
    {2, 1, 10.6765, 6.95484},  // median |error| 1.2%
    {2, 2, 6.5270, 1.76279},  // median |error| 1.2%
    {2, 3, 4.3504, 0.91518},  // median |error| 1.9%
    {2, 4, 4.5535, 1.78263},  // median |error| 1.0%
    {2, 5, 4.0253, 0.93750},  // median |error| 1.8%
    {2, 6, 3.1323, 0.50612},  // median |error| 3.2%
    {2, 7, 3.1419, 1.05879},  // median |error| 2.7%
    {2, 8, 7.0478, 7.08027},  // median |error| 0.9%
    {2, 9, 5.1862, 3.51099},  // median |error| 1.1%
    {2, 10, 3.1392, 0.54142},  // median |error| 4.1%
    {2, 11, 6.8706, 1.99730},  // median |error| 0.9%
    {2, 12, 7.4940, 3.95635},  // median |error| 0.9%
    {3, 0, 10.4925, 3.55269},  // median |error| 2.3%
    {3, 1, 10.3382, 7.12597},  // median |error| 2.3%
    {3, 2, 6.6884, 1.80543},  // median |error| 2.0%
    {3, 3, 4.5946, 0.91211},  // median |error| 1.7%
    {3, 4, 4.5204, 1.84514},  // median |error| 2.0%
    {3, 5, 4.1040, 0.96609},  // median |error| 1.8%
    {3, 6, 3.2114, 0.50393},  // median |error| 3.2%
    {3, 7, 3.1263, 1.10119},  // median |error| 2.8%
    {3, 8, 7.6829, 7.07705},  // median |error| 1.0%
    {3, 9, 5.0848, 3.55197},  // median |error| 1.3%
    {3, 10, 3.1867, 0.52778},  // median |error| 5.3%
    {3, 11, 7.2231, 2.04638},  // median |error| 2.4%
    {3, 12, 7.5777, 4.07320},  // median |error| 2.8%
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

// Split-K: the number of K chunks (1 = do not split) with the least modelled time among
// the counts the split study measured.  A split launch costs the GEMM of its chunks, all in
// one grid (the model above, with the workgroups multiplied by the chunks), plus
//     0.0000 us (the reduction's launch)
//   + 0.20133 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.2828 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 0.0000;
constexpr double kSplitUsPerMB = 0.20133;
constexpr double kSplitUsPerRound = 0.2828;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 8},  // 1: 69.2, 2: 38.7, 4: 23.3, 8: 17.5, 16: 21.5
    {32, 4096, 4096, 8},  // 1: 63.1, 2: 39.2, 4: 23.6, 8: 17.3, 16: 21.7
    {64, 4096, 4096, 8},  // 1: 60.5, 2: 34.8, 4: 23.0, 8: 23.0, 16: 26.1
    {128, 4096, 4096, 2},  // 1: 61.2, 2: 35.7, 4: 37.1, 8: 39.2, 16: 43.3
    {32, 8192, 8192, 4},  // 1: 124.1, 2: 73.5, 4: 45.7, 8: 46.6, 16: 52.0
    {64, 8192, 8192, 2},  // 1: 119.3, 2: 68.2, 4: 70.9, 8: 75.4, 16: 87.1
    {256, 256, 8192, 16},  // 1: 117.9, 2: 62.7, 4: 34.7, 8: 22.5, 16: 17.2
    {512, 512, 8192, 4},  // 1: 118.9, 2: 63.8, 4: 35.5, 8: 37.4, 16: 40.2
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.9, 4: 29.2, 8: 35.0, 16: 38.7
    {2048, 2048, 2048, 1},  // 1: 117.9, 2: 130.0, 4: 139.3, 8: 157.8, 16: 203.2
    {4096, 4096, 4096, 1},  // 1: 903.4, 2: 945.2, 4: 996.1, 8: 1113.6, 16: 1278.0, -2: 1068.4, -4: 1079.3, -8: 1122.3, -16: 1166.7
    {1536, 1536, 1536, -4},  // 1: 68.2, 2: 66.5, 4: 64.8, 8: 76.6, 16: 88.2, -2: 61.4, -4: 57.1, -8: 57.9, -16: 63.8
    {1536, 1536, 4096, -8},  // 1: 174.1, 2: 154.5, 4: 143.5, 8: 154.9, 16: 176.1, -2: 149.2, -4: 138.5, -8: 136.8, -16: 139.3
    {2560, 2560, 2560, -8},  // 1: 255.7, 2: 263.2, 4: 272.2, 8: 292.0, 16: 366.3, -2: 244.1, -4: 240.5, -8: 234.3, -16: 240.4
    {1280, 1280, 2048, -4},  // 1: 62.0, 2: 66.0, 4: 66.0, 8: 71.4, 16: 82.1, -2: 66.6, -4: 61.1, -8: 62.0, -16: 66.2
    {5000, 5000, 1000, -8},  // 1: 393.7, 2: 442.1, 4: 532.5, 8: 742.7, 16: 1145.0, -2: 402.9, -4: 403.2, -8: 382.7, -16: 386.2
    {1536, 3072, 4096, -8},  // 1: 289.7, 2: 270.2, 4: 280.8, 8: 302.0, 16: 369.9, -2: 272.5, -4: 266.6, -8: 266.3, -16: 270.2
    {39, 432, 6224, 16},  // 1: 104.9, 2: 56.0, 4: 31.8, 8: 20.5, 16: 16.1
    {11, 1640, 2822, 16},  // 1: 49.5, 2: 29.2, 4: 18.4, 8: 13.1, 16: 12.3
    {11, 1486, 1136, 16},  // 1: 21.7, 2: 14.5, 4: 10.9, 8: 9.7, 16: 9.5
    {66, 326, 1317, 8},  // 1: 24.8, 2: 17.1, 4: 12.0, 8: 9.7, 16: 9.7
    {63, 4495, 1443, 8},  // 1: 29.0, 2: 20.0, 4: 19.0, 8: 18.9, 16: 19.7
    {24, 2252, 14173, 8},  // 1: 235.2, 2: 121.7, 4: 64.5, 8: 38.1, 16: 40.1
    {132, 1012, 15340, 16},  // 1: 254.9, 2: 131.3, 4: 69.3, 8: 65.6, 16: 55.4
    {10, 5016, 2286, 4},  // 1: 41.1, 2: 24.9, 4: 16.7, 8: 19.6, 16: 16.9
    {16, 385, 2409, 16},  // 1: 42.5, 2: 24.9, 4: 15.9, 8: 11.8, 16: 11.0
    {420, 479, 5136, 4},  // 1: 88.2, 2: 48.1, 4: 28.6, 8: 31.3, 16: 34.0
    {178, 931, 4676, 4},  // 1: 86.7, 2: 44.9, 4: 26.3, 8: 28.9, 16: 27.3
    {11, 315, 1813, 16},  // 1: 32.7, 2: 20.6, 4: 13.8, 8: 10.6, 16: 10.3
    {217, 1127, 2447, 4},  // 1: 43.5, 2: 26.6, 4: 18.3, 8: 21.4, 16: 23.9
    {137, 1231, 2351, 4},  // 1: 46.8, 2: 25.4, 4: 17.6, 8: 19.7, 16: 24.6
    {378, 2886, 2015, -8},  // 1: 64.7, 2: 55.9, 4: 52.2, 8: 52.2, 16: 68.1, -2: 55.5, -4: 48.0, -8: 45.7, -16: 47.4
    {130, 1580, 11590, 8},  // 1: 204.2, 2: 102.7, 4: 94.2, 8: 73.9, 16: 75.6
    {276, 694, 15508, 8},  // 1: 275.3, 2: 134.7, 4: 69.9, 8: 67.9, 16: 73.0
    {14, 1090, 8356, 16},  // 1: 139.7, 2: 73.4, 4: 39.8, 8: 24.7, 16: 18.6
    {17, 1394, 1142, 16},  // 1: 21.7, 2: 14.5, 4: 10.9, 8: 9.6, 16: 9.4
    {205, 3623, 5015, 4},  // 1: 99.4, 2: 83.7, 4: 83.1, 8: 85.3, 16: 89.7
    {560, 759, 7039, 8},  // 1: 120.6, 2: 64.6, 4: 61.6, 8: 61.4, 16: 62.1
    {143, 1910, 3628, 2},  // 1: 67.0, 2: 36.3, 4: 36.5, 8: 40.4, 16: 44.1
    {471, 6763, 3812, -2},  // 1: 219.9, 2: 215.2, 4: 214.9, 8: 237.4, 16: 280.2, -2: 206.8, -4: 253.6, -8: 253.8, -16: 257.8
    {201, 316, 7161, 8},  // 1: 128.1, 2: 65.5, 4: 35.5, 8: 22.4, 16: 25.0
};

static inline double model_best_us(int64_t M, int64_t N, int64_t K, int64_t wg_factor) {
  return model_us(model_pick(M, N, K, 0, wg_factor), M, N, K, wg_factor);
}

static inline double split_model_us(int64_t M, int64_t N, int64_t K, int splits) {
  int64_t kc = K;
  int used = 1;
  if (K > 0) splitk_plan(K, splits, &kc, &used);
  if (used <= 1) return model_best_us(M, N, K, 1);
  const ModelRow& r = model_pick(M, N, kc, 0, used);
  const CfgEntry& e = kConfigs[r.cfg];
  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn) * used;
  const double rounds = (double)((tiles + kModelCUs - 1) / kModelCUs);
  const double mb = (double)(2 * used + 1) * (double)M * (double)N * 4.0 / 1e6;
  return model_us(r, M, N, kc, used) + kSplitFixedUs + kSplitUsPerMB * mb +
         kSplitUsPerRound * rounds;
}

// Tail split: only the tiles of the last, partly filled round of workgroups are split (the
// full rounds run whole), priced like a split launch whose overhead covers just those
// tiles.  The pick with the least modelled time among the configurations whose tiles make
// at least one full round and a partly filled one; found = false when there is none.
struct TailPick {
  bool found;
  int variant, cfg;
  int64_t split_from;
  double us;
};

static inline TailPick tail_pick(int64_t M, int64_t N, int64_t K, int used, int64_t kc) {
  TailPick best{false, 0, 0, 0, 0.0};
  for (int i = 0; i < kModelRows; ++i) {
    const ModelRow& r = kModel[i];
    const CfgEntry& e = kConfigs[r.cfg];
    const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
    const int64_t full = tiles / kModelCUs * kModelCUs, tail = tiles - full;
    if (full == 0 || tail == 0) continue;
    const double tail_rounds = (double)((tail * used + kModelCUs - 1) / kModelCUs);
    const double mb = (double)(2 * used + 1) * (double)tail * e.bm * e.bn * 4.0 / 1e6;
    const double t = r.a_us +
                     r.g_us * ((double)(full / kModelCUs) * (double)((K + e.bk - 1) / e.bk) +
                               tail_rounds * (double)((kc + e.bk - 1) / e.bk)) +
                     kSplitFixedUs + kSplitUsPerMB * mb + kSplitUsPerRound * tail_rounds;
    if (!best.found || t < best.us) best = TailPick{true, r.variant, r.cfg, full, t};
  }
  return best;
}

// The split count: > 1 splits every tile, 1 does not split, -s splits only the tail tiles
// into s chunks.
static inline int select_splits(int64_t M, int64_t N, int64_t K) {
  int best = 1;
  double best_t = 0.0;
  for (int i = 0; i < (int)(sizeof(kSplitChoices) / sizeof(kSplitChoices[0])); ++i) {
    const double t = split_model_us(M, N, K, kSplitChoices[i]);
    if (i == 0 || t < best_t) {
      best = kSplitChoices[i];
      best_t = t;
    }
  }
  for (int i = 0; i < (int)(sizeof(kSplitChoices) / sizeof(kSplitChoices[0])); ++i) {
    const int s = kSplitChoices[i];
    if (s < 2 || K <= 0) continue;
    int64_t kc = 0;
    int used = 1;
    splitk_plan(K, s, &kc, &used);
    if (used <= 1) continue;
    const TailPick tp = tail_pick(M, N, K, used, kc);
    if (tp.found && tp.us < best_t) {
      best = -s;
      best_t = tp.us;
    }
  }
  return best;
}

}  // namespace gemmf32
