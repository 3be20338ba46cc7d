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
// direct-to-LDS, 5 = K split inside the workgroup), its tile configuration, and the best
// configuration of the single-buffered, double-buffered and multi-stage variants.
// Trailing comments: measured microseconds of the best configuration of each variant.
#pragma once

#include <cmath>
#include <cstdint>

namespace gemmf32 {

struct DispatchRow {
  int64_t m, n, k;
  int variant, cfg, sb_cfg, db_cfg, ms_cfg;
};

static const DispatchRow kDispatch[] = {
    {128, 128, 128, 5, 13, 7, 6, 6},  // sb 4.73 us, db 4.43 us, ms 4.50 us, ks 4.21 us
    {127, 193, 61, 1, 7, 7, 10, 6},  // sb 4.16 us, db 4.23 us, ms 4.24 us, ks 4.25 us
    {513, 257, 129, 5, 13, 13, 13, 6},  // sb 6.23 us, db 5.85 us, ms 5.97 us, ks 4.91 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.69 us, db 18.50 us, ms 17.92 us, ks 23.47 us
    {256, 1024, 128, 5, 13, 7, 13, 6},  // sb 5.00 us, db 4.59 us, ms 4.78 us, ks 4.14 us
    {1024, 128, 256, 5, 13, 7, 13, 6},  // sb 7.44 us, db 6.43 us, ms 6.50 us, ks 4.64 us
    {4096, 4096, 4096, 2, 0, 9, 0, 3},  // sb 957.80 us, db 901.83 us, ms 910.75 us, ks 1199.23 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7411.74 us, db 7148.75 us, ms 7182.64 us, ks 9570.10 us
    {256, 256, 256, 5, 13, 7, 13, 6},  // sb 7.40 us, db 6.40 us, ms 6.47 us, ks 4.61 us
    {512, 512, 512, 5, 13, 7, 13, 6},  // sb 12.51 us, db 10.19 us, ms 10.10 us, ks 6.14 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 17.98 us, db 14.44 us, ms 14.02 us, ks 15.80 us
    {1536, 1536, 1536, 3, 6, 7, 6, 6},  // sb 76.90 us, db 68.57 us, ms 68.51 us, ks 71.07 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 127.57 us, db 118.04 us, ms 121.20 us, ks 156.85 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 422.83 us, db 383.35 us, ms 398.32 us, ks 520.17 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3172.35 us, db 3030.98 us, ms 3048.23 us, ks 4001.96 us
    {64, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.33 us, db 63.67 us, ms 60.63 us, ks 24.75 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 127.21 us, db 123.48 us, ms 124.02 us, ks 213.64 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 484.60 us, db 457.84 us, ms 460.76 us, ks 621.85 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 66.20 us, db 61.74 us, ms 63.50 us, ks 87.71 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.55 us, db 128.44 us, ms 121.62 us, ks 152.31 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.21 us, db 20.88 us, ms 20.60 us, ks 27.43 us
    {4095, 4095, 4095, 2, 0, 9, 0, 0},  // sb 996.07 us, db 911.86 us, ms 915.77 us, ks 1334.17 us
    {16, 4096, 4096, 5, 13, 7, 6, 6},  // sb 97.50 us, db 70.04 us, ms 69.31 us, ks 25.29 us
    {32, 4096, 4096, 5, 13, 7, 13, 10},  // sb 98.07 us, db 63.75 us, ms 63.28 us, ks 24.56 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.39 us, db 64.05 us, ms 60.78 us, ks 40.37 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 196.22 us, db 128.89 us, ms 123.66 us, ks 48.45 us
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
//     a + b * rounds + g * rounds * k_tiles   microseconds,
// a being the fixed cost (launch, first copy, epilogue), g the time of one K tile of one
// round, and b a cost per round that only the K-split kernel has (each of its rounds ends
// in a hand-off through LDS; b = 0 elsewhere).  They were fitted per pair by least squares
// on relative error, all kept >= 0, to the 74 shapes measured for this file (the
// table's 26 and 48 seeded shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, b_us, g_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.0792, 0.0000, 4.10873},  // median |error| 3.2%
    {1, 1, 9.7787, 0.0000, 7.83957},  // median |error| 1.7%
    {1, 2, 6.0249, 0.0000, 2.21005},  // median |error| 4.3%
    {1, 3, 4.0767, 0.0000, 1.20157},  // median |error| 7.8%
    {1, 4, 4.1564, 0.0000, 2.21339},  // median |error| 5.2%
    {1, 5, 3.3637, 0.0000, 1.19056},  // median |error| 6.8%
    {1, 6, 3.0767, 0.0000, 0.63507},  // median |error| 10.4%
    {1, 7, 3.0846, 0.0000, 1.17834},  // median |error| 7.9%
    {1, 8, 6.4504, 0.0000, 7.69130},  // median |error| 2.1%
    {1, 9, 4.4464, 0.0000, 4.04007},  // median |error| 2.1%
    {1, 10, 3.1429, 0.0000, 0.66035},  // median |error| 10.2%
    {1, 11, 6.0420, 0.0000, 2.52160},  // median |error| 4.1%
    {1, 12, 6.4635, 0.0000, 4.68883},  // median |error| 2.7%
    {1, 13, 4.5155, 0.0000, 0.18013},  // median |error| 20.7%
    {2, 0, 10.0121, 0.0000, 3.47979},  // median |error| 1.1%
    {2, 1, 10.3348, 0.0000, 6.96116},  // median |error| 0.9%
    {2, 2, 6.6774, 0.0000, 1.76002},  // median |error| 1.3%
    {2, 3, 4.2903, 0.0000, 0.91310},  // median |error| 1.7%
    {2, 4, 4.5954, 0.0000, 1.77679},  // median |error| 1.2%
    {2, 5, 4.0255, 0.0000, 0.93558},  // median |error| 1.8%
    {2, 6, 3.1580, 0.0000, 0.50346},  // median |error| 3.6%
    {2, 7, 3.1683, 0.0000, 1.05166},  // median |error| 3.0%
    {2, 8, 7.2518, 0.0000, 7.08358},  // median |error| 0.9%
    {2, 9, 5.1378, 0.0000, 3.50939},  // median |error| 0.8%
    {2, 10, 3.1639, 0.0000, 0.53814},  // median |error| 3.9%
    {2, 11, 7.0809, 0.0000, 1.99546},  // median |error| 0.8%
    {2, 12, 7.4522, 0.0000, 3.95336},  // median |error| 0.9%
    {2, 13, 4.4271, 0.0000, 0.16656},  // median |error| 15.7%
    {3, 0, 10.5551, 0.0000, 3.55819},  // median |error| 2.1%
    {3, 1, 10.4079, 0.0000, 7.12838},  // median |error| 2.3%
    {3, 2, 6.7312, 0.0000, 1.80362},  // median |error| 1.9%
    {3, 3, 4.5485, 0.0000, 0.91036},  // median |error| 1.8%
    {3, 4, 4.6895, 0.0000, 1.83901},  // median |error| 2.0%
    {3, 5, 4.1234, 0.0000, 0.96177},  // median |error| 1.9%
    {3, 6, 3.2249, 0.0000, 0.50069},  // median |error| 3.3%
    {3, 7, 3.1828, 0.0000, 1.09597},  // median |error| 2.7%
    {3, 8, 7.7100, 0.0000, 7.08211},  // median |error| 0.9%
    {3, 9, 5.3586, 0.0000, 3.54632},  // median |error| 1.1%
    {3, 10, 3.2036, 0.0000, 0.52522},  // median |error| 5.5%
    {3, 11, 7.2084, 0.0000, 2.04488},  // median |error| 2.4%
    {3, 12, 7.5921, 0.0000, 4.06798},  // median |error| 2.9%
    {5, 13, 2.7552, 0.9877, 0.15787},  // median |error| 7.7%
};
constexpr int kModelRows = (int)(sizeof(kModel) / sizeof(kModel[0]));
constexpr int kVariantKS = 5;
constexpr int64_t kModelCUs = 256;

// Modelled microseconds of one launch; wg_factor multiplies the workgroup count (the K
// chunks of a split-K launch run side by side in one grid).
static inline double model_us(const ModelRow& r, int64_t M, int64_t N, int64_t K,
                              int64_t wg_factor) {
  const CfgEntry& e = kConfigs[r.cfg];
  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn) * wg_factor;
  const int64_t rounds = (tiles + kModelCUs - 1) / kModelCUs;
  const int64_t k_tiles = (K + e.bk - 1) / e.bk;
  return r.a_us + r.b_us * (double)rounds + r.g_us * (double)rounds * (double)k_tiles;
}

// The row with the least modelled time (variant 0: any variant), first row on ties.
static inline const ModelRow& model_pick(int64_t M, int64_t N, int64_t K, int variant,
                                         int64_t wg_factor) {
  int best = 0;
  double best_t = 0.0;
  bool found = false;
  for (int i = 0; i < kModelRows; ++i) {
    if (variant != 0 && kModel[i].variant != variant) continue;
    // a split-K launch takes neither the K-split kernel (it divides K itself) nor a
    // one-wave configuration (its plain kernels keep one SIMD of a CU busy)
    if (wg_factor != 1 &&
        (kModel[i].variant == kVariantKS || kConfigs[kModel[i].cfg].nt == 64))
      continue;
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
  const DispatchRow* r = variant != kVariantKS ? dispatch_exact(M, N, K) : nullptr;
  if (r) return variant == 1 ? r->sb_cfg : variant == 3 ? r->ms_cfg : r->db_cfg;
  return model_pick(M, N, K, variant, 1).cfg;
}

// Split-K: the number of K chunks (1 = do not split) with the least modelled time among
// the counts the split study measured.  A split launch costs the GEMM of its chunks, all in
// one grid (the model above, with the workgroups multiplied by the chunks), plus
//     0.0000 us (the reduction's launch)
//   + 0.20000 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.4335 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 0.0000;
constexpr double kSplitUsPerMB = 0.20000;
constexpr double kSplitUsPerRound = 0.4335;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 8},  // 1: 25.8, 2: 38.9, 4: 23.1, 8: 17.5, 16: 21.3
    {32, 4096, 4096, 8},  // 1: 24.9, 2: 39.3, 4: 23.4, 8: 17.3, 16: 21.7
    {64, 4096, 4096, 4},  // 1: 25.1, 2: 35.0, 4: 21.6, 8: 24.4, 16: 29.2
    {128, 4096, 4096, 2},  // 1: 41.2, 2: 36.0, 4: 38.0, 8: 39.5, 16: 43.5
    {32, 8192, 8192, 4},  // 1: 48.6, 2: 73.4, 4: 44.7, 8: 46.8, 16: 52.9
    {64, 8192, 8192, 2},  // 1: 82.6, 2: 69.3, 4: 73.9, 8: 77.3, 16: 88.3
    {256, 256, 8192, 16},  // 1: 45.9, 2: 62.8, 4: 34.7, 8: 21.8, 16: 17.3
    {512, 512, 8192, 4},  // 1: 46.1, 2: 63.8, 4: 35.9, 8: 38.3, 16: 40.4
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.9, 4: 29.2, 8: 34.9, 16: 38.8
    {2048, 2048, 2048, 1},  // 1: 118.5, 2: 130.4, 4: 139.8, 8: 158.5, 16: 204.0
    {4096, 4096, 4096, 1},  // 1: 905.1, 2: 946.0, 4: 996.8, 8: 1114.9, 16: 1278.5, -2: 1067.7, -4: 1080.0, -8: 1123.3, -16: 1168.1
    {1536, 1536, 1536, -4},  // 1: 68.8, 2: 67.0, 4: 65.2, 8: 77.0, 16: 88.6, -2: 61.8, -4: 57.9, -8: 58.3, -16: 63.9
    {1536, 1536, 4096, -8},  // 1: 175.1, 2: 156.5, 4: 143.2, 8: 154.5, 16: 177.4, -2: 150.9, -4: 142.6, -8: 137.8, -16: 141.7
    {2560, 2560, 2560, -8},  // 1: 258.3, 2: 265.8, 4: 274.4, 8: 292.8, 16: 366.7, -2: 248.0, -4: 242.2, -8: 237.2, -16: 242.5
    {1280, 1280, 2048, 1},  // 1: 61.7, 2: 65.9, 4: 66.2, 8: 71.9, 16: 82.9, -2: 67.0, -4: 62.0, -8: 63.2, -16: 66.6
    {5000, 5000, 1000, -8},  // 1: 392.5, 2: 442.8, 4: 535.1, 8: 745.4, 16: 1145.4, -2: 403.5, -4: 406.2, -8: 381.9, -16: 386.7
    {1536, 3072, 4096, -8},  // 1: 291.5, 2: 269.5, 4: 280.2, 8: 304.5, 16: 369.8, -2: 275.5, -4: 269.9, -8: 265.9, -16: 269.5
    {39, 432, 6224, 16},  // 1: 36.8, 2: 56.1, 4: 31.9, 8: 20.5, 16: 16.3
    {11, 1640, 2822, 16},  // 1: 19.8, 2: 29.1, 4: 18.4, 8: 13.1, 16: 12.4
    {11, 1486, 1136, 16},  // 1: 9.9, 2: 14.5, 4: 10.9, 8: 9.6, 16: 9.4
    {66, 326, 1317, 8},  // 1: 11.4, 2: 17.4, 4: 12.1, 8: 9.8, 16: 10.0
    {63, 4495, 1443, 8},  // 1: 25.8, 2: 19.9, 4: 19.0, 8: 19.0, 16: 19.8
    {24, 2252, 14173, 8},  // 1: 78.4, 2: 121.4, 4: 64.3, 8: 38.0, 16: 40.1
    {132, 1012, 15340, 16},  // 1: 84.8, 2: 131.4, 4: 69.2, 8: 65.4, 16: 55.9
    {10, 5016, 2286, 1},  // 1: 16.7, 2: 24.5, 4: 16.8, 8: 19.7, 16: 16.9
    {16, 385, 2409, 16},  // 1: 16.7, 2: 24.9, 4: 16.0, 8: 11.8, 16: 11.0
    {420, 479, 5136, 4},  // 1: 32.0, 2: 48.2, 4: 28.6, 8: 31.2, 16: 34.1
    {178, 931, 4676, 4},  // 1: 30.7, 2: 44.9, 4: 26.3, 8: 28.7, 16: 33.3
    {11, 315, 1813, 16},  // 1: 14.1, 2: 20.6, 4: 13.9, 8: 10.5, 16: 10.3
    {217, 1127, 2447, 4},  // 1: 21.1, 2: 26.7, 4: 18.3, 8: 21.6, 16: 22.9
    {137, 1231, 2351, 4},  // 1: 21.2, 2: 25.4, 4: 17.6, 8: 19.9, 16: 24.7
    {378, 2886, 2015, -8},  // 1: 65.9, 2: 55.8, 4: 52.3, 8: 52.5, 16: 68.3, -2: 55.5, -4: 48.4, -8: 46.0, -16: 47.6
    {130, 1580, 11590, 8},  // 1: 94.9, 2: 103.0, 4: 94.6, 8: 74.4, 16: 75.8
    {276, 694, 15508, 8},  // 1: 86.9, 2: 135.2, 4: 70.3, 8: 68.2, 16: 73.8
    {14, 1090, 8356, 16},  // 1: 48.3, 2: 73.6, 4: 39.9, 8: 24.4, 16: 18.6
    {17, 1394, 1142, 16},  // 1: 10.0, 2: 14.5, 4: 10.9, 8: 9.6, 16: 9.3
    {205, 3623, 5015, 4},  // 1: 99.5, 2: 83.9, 4: 83.3, 8: 85.7, 16: 90.2
    {560, 759, 7039, 8},  // 1: 72.8, 2: 64.9, 4: 61.9, 8: 61.8, 16: 62.5
    {143, 1910, 3628, 2},  // 1: 53.9, 2: 36.4, 4: 36.5, 8: 40.4, 16: 44.1
    {471, 6763, 3812, -2},  // 1: 221.0, 2: 217.9, 4: 216.9, 8: 238.2, 16: 281.2, -2: 209.4, -4: 252.4, -8: 252.4, -16: 256.0
    {201, 316, 7161, 8},  // 1: 42.0, 2: 65.5, 4: 35.6, 8: 22.6, 16: 25.0
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
    if (r.variant == kVariantKS || e.nt == 64) continue;  // as in a full split
    const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
    const int64_t full = tiles / kModelCUs * kModelCUs, tail = tiles - full;
    if (full == 0 || tail == 0) continue;
    const double tail_rounds = (double)((tail * used + kModelCUs - 1) / kModelCUs);
    const double mb = (double)(2 * used + 1) * (double)tail * e.bm * e.bn * 4.0 / 1e6;
    const double t = r.a_us + r.b_us * ((double)(full / kModelCUs) + tail_rounds) +
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
