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
    {128, 128, 128, 3, 6, 7, 6, 6},  // sb 4.77 us, db 4.55 us, ms 4.52 us
    {127, 193, 61, 3, 10, 10, 10, 10},  // sb 4.23 us, db 4.21 us, ms 4.16 us
    {513, 257, 129, 2, 6, 6, 6, 6},  // sb 6.44 us, db 5.87 us, ms 5.94 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.73 us, db 18.53 us, ms 17.97 us
    {256, 1024, 128, 2, 6, 7, 6, 6},  // sb 4.98 us, db 4.67 us, ms 4.70 us
    {1024, 128, 256, 3, 6, 7, 6, 6},  // sb 7.42 us, db 6.49 us, ms 6.48 us
    {4096, 4096, 4096, 2, 0, 9, 0, 8},  // sb 963.16 us, db 907.44 us, ms 920.75 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7443.92 us, db 7172.62 us, ms 7219.22 us
    {256, 256, 256, 3, 6, 7, 6, 6},  // sb 7.41 us, db 6.47 us, ms 6.45 us
    {512, 512, 512, 3, 6, 7, 6, 6},  // sb 12.51 us, db 10.28 us, ms 10.09 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.06 us, db 14.49 us, ms 14.07 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 77.09 us, db 68.68 us, ms 68.99 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 128.24 us, db 118.28 us, ms 121.97 us
    {3072, 3072, 3072, 3, 6, 7, 6, 6},  // sb 424.33 us, db 422.11 us, ms 406.21 us
    {6144, 6144, 6144, 3, 3, 4, 4, 3},  // sb 3190.50 us, db 3049.85 us, ms 3050.87 us
    {64, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.86 us, db 64.97 us, ms 60.78 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 127.95 us, db 122.90 us, ms 124.53 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 488.20 us, db 461.13 us, ms 464.31 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 66.77 us, db 61.88 us, ms 63.77 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.63 us, db 128.54 us, ms 121.95 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.19 us, db 20.94 us, ms 20.70 us
    {4095, 4095, 4095, 2, 0, 9, 0, 0},  // sb 1003.19 us, db 919.44 us, ms 921.98 us
    {16, 4096, 4096, 3, 6, 7, 6, 6},  // sb 97.52 us, db 70.24 us, ms 69.55 us
    {32, 4096, 4096, 3, 10, 7, 10, 10},  // sb 97.74 us, db 69.27 us, ms 63.33 us
    {128, 4096, 4096, 3, 6, 7, 6, 6},  // sb 95.93 us, db 65.19 us, ms 61.15 us
    {32, 8192, 8192, 3, 10, 7, 10, 10},  // sb 197.78 us, db 143.76 us, ms 124.18 us
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
    {1, 0, 9.6025, 4.10568},  // median |error| 3.3%
    {1, 1, 9.4886, 7.82862},  // median |error| 2.0%
    {1, 2, 6.0496, 2.21215},  // median |error| 4.3%
    {1, 3, 3.8712, 1.20347},  // median |error| 7.6%
    {1, 4, 4.1555, 2.21474},  // median |error| 5.0%
    {1, 5, 3.4583, 1.19254},  // median |error| 7.2%
    {1, 6, 3.1208, 0.63470},  // median |error| 10.0%
    {1, 7, 3.0794, 1.18107},  // median |error| 7.4%
    {1, 8, 6.2696, 7.69579},  // median |error| 2.1%
    {1, 9, 4.4221, 4.04198},  // median |error| 2.1%
    {1, 10, 3.1323, 0.66385},  // median |error| 10.2%
    {2, 0, 10.3141, 3.47871},  // median |error| 1.3%
    {2, 1, 10.7009, 6.96492},  // median |error| 1.4%
    {2, 2, 6.5465, 1.76328},  // median |error| 1.1%
    {2, 3, 4.3633, 0.91470},  // median |error| 2.0%
    {2, 4, 4.5710, 1.78125},  // median |error| 1.1%
    {2, 5, 4.0455, 0.93638},  // median |error| 1.6%
    {2, 6, 3.1691, 0.50436},  // median |error| 3.5%
    {2, 7, 3.2308, 1.05355},  // median |error| 2.9%
    {2, 8, 7.0628, 7.08961},  // median |error| 0.8%
    {2, 9, 5.1976, 3.51237},  // median |error| 0.9%
    {2, 10, 3.1690, 0.53871},  // median |error| 3.9%
    {3, 0, 10.5231, 3.55626},  // median |error| 2.3%
    {3, 1, 10.3626, 7.13541},  // median |error| 2.3%
    {3, 2, 6.7082, 1.80632},  // median |error| 2.0%
    {3, 3, 4.6086, 0.91163},  // median |error| 1.8%
    {3, 4, 4.5355, 1.84429},  // median |error| 1.9%
    {3, 5, 4.1289, 0.96506},  // median |error| 1.8%
    {3, 6, 3.2594, 0.50167},  // median |error| 3.3%
    {3, 7, 3.1774, 1.09819},  // median |error| 2.8%
    {3, 8, 7.6960, 7.08562},  // median |error| 1.1%
    {3, 9, 5.0972, 3.55414},  // median |error| 1.2%
    {3, 10, 3.2235, 0.52565},  // median |error| 5.4%
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
//     2.5816 us (the reduction's launch)
//   + 0.16456 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.9034 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 35 shapes of the split study below.
constexpr double kSplitFixedUs = 2.5816;
constexpr double kSplitUsPerMB = 0.16456;
constexpr double kSplitUsPerRound = 0.9034;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 8},  // 1: 69.4, 2: 38.7, 4: 24.1, 8: 20.4, 16: 23.5
    {32, 4096, 4096, 8},  // 1: 63.4, 2: 39.2, 4: 24.5, 8: 19.6, 16: 23.8
    {64, 4096, 4096, 4},  // 1: 60.9, 2: 35.0, 4: 23.8, 8: 24.6, 16: 29.8
    {128, 4096, 4096, 2},  // 1: 61.3, 2: 36.2, 4: 38.3, 8: 40.0, 16: 44.9
    {32, 8192, 8192, 4},  // 1: 124.4, 2: 73.2, 4: 46.5, 8: 48.7, 16: 55.2
    {64, 8192, 8192, 2},  // 1: 119.3, 2: 71.4, 4: 74.8, 8: 78.9, 16: 86.8
    {256, 256, 8192, 16},  // 1: 117.8, 2: 62.9, 4: 34.8, 8: 23.4, 16: 17.7
    {512, 512, 8192, 4},  // 1: 119.1, 2: 64.0, 4: 38.1, 8: 38.9, 16: 40.7
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 22.9, 4: 25.4, 8: 30.1, 16: 39.6
    {2048, 2048, 2048, 1},  // 1: 118.2, 2: 130.6, 4: 140.2, 8: 158.9, 16: 206.0
    {4096, 4096, 4096, 1},  // 1: 908.4, 2: 949.6, 4: 992.6, 8: 1100.8, 16: 1292.0
    {39, 432, 6224, 16},  // 1: 105.2, 2: 56.3, 4: 31.9, 8: 20.8, 16: 16.3
    {11, 1640, 2822, 16},  // 1: 49.8, 2: 29.2, 4: 18.5, 8: 13.4, 16: 12.3
    {11, 1486, 1136, 16},  // 1: 21.7, 2: 14.4, 4: 10.9, 8: 9.6, 16: 9.5
    {66, 326, 1317, 8},  // 1: 25.0, 2: 17.2, 4: 12.1, 8: 9.8, 16: 9.8
    {63, 4495, 1443, 8},  // 1: 29.1, 2: 19.8, 4: 18.0, 8: 17.5, 16: 20.2
    {24, 2252, 14173, 8},  // 1: 236.2, 2: 122.4, 4: 64.7, 8: 38.7, 16: 45.3
    {132, 1012, 15340, 8},  // 1: 256.0, 2: 132.2, 4: 70.0, 8: 65.9, 16: 67.2
    {10, 5016, 2286, 4},  // 1: 41.2, 2: 24.8, 4: 16.8, 8: 19.7, 16: 17.2
    {16, 385, 2409, 16},  // 1: 42.6, 2: 25.0, 4: 15.9, 8: 11.7, 16: 11.0
    {420, 479, 5136, 4},  // 1: 88.5, 2: 48.3, 4: 28.7, 8: 30.3, 16: 33.8
    {178, 931, 4676, 4},  // 1: 86.9, 2: 47.9, 4: 26.8, 8: 28.1, 16: 27.0
    {11, 315, 1813, 16},  // 1: 32.8, 2: 20.6, 4: 13.8, 8: 10.5, 16: 10.2
    {217, 1127, 2447, 4},  // 1: 43.9, 2: 26.8, 4: 21.6, 8: 23.5, 16: 23.8
    {137, 1231, 2351, 4},  // 1: 47.0, 2: 27.2, 4: 18.7, 8: 19.2, 16: 23.6
    {378, 2886, 2015, 4},  // 1: 64.6, 2: 54.2, 4: 53.0, 8: 61.0, 16: 71.8
    {130, 1580, 11590, 16},  // 1: 205.2, 2: 109.3, 4: 94.1, 8: 76.0, 16: 73.9
    {276, 694, 15508, 8},  // 1: 276.3, 2: 145.3, 4: 81.9, 8: 76.8, 16: 81.8
    {14, 1090, 8356, 16},  // 1: 140.4, 2: 73.7, 4: 39.8, 8: 25.1, 16: 18.4
    {17, 1394, 1142, 16},  // 1: 21.7, 2: 14.5, 4: 10.9, 8: 9.5, 16: 9.4
    {205, 3623, 5015, 4},  // 1: 100.3, 2: 84.0, 4: 83.0, 8: 86.2, 16: 106.2
    {560, 759, 7039, 4},  // 1: 121.3, 2: 66.5, 4: 62.2, 8: 63.4, 16: 65.2
    {143, 1910, 3628, 8},  // 1: 67.3, 2: 38.7, 4: 36.4, 8: 35.5, 16: 40.6
    {471, 6763, 3812, 2},  // 1: 221.7, 2: 219.3, 4: 240.3, 8: 228.2, 16: 282.2
    {201, 316, 7161, 8},  // 1: 128.5, 2: 68.3, 4: 37.9, 8: 23.4, 16: 24.6
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
  return best;
}

}  // namespace gemmf32
