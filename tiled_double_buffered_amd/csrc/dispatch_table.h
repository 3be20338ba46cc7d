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
    {128, 128, 128, 5, 17, 7, 6, 6},  // sb 4.76 us, db 4.52 us, ms 4.55 us, ks 4.06 us
    {127, 193, 61, 5, 17, 7, 6, 7},  // sb 4.12 us, db 4.14 us, ms 4.16 us, ks 4.06 us
    {513, 257, 129, 5, 16, 13, 13, 6},  // sb 6.16 us, db 5.81 us, ms 5.97 us, ks 4.14 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.79 us, db 18.60 us, ms 18.05 us, ks 24.08 us
    {256, 1024, 128, 5, 17, 13, 13, 6},  // sb 4.97 us, db 4.63 us, ms 4.77 us, ks 4.03 us
    {1024, 128, 256, 5, 15, 7, 13, 6},  // sb 7.42 us, db 6.42 us, ms 6.47 us, ks 4.01 us
    {4096, 4096, 4096, 2, 0, 9, 0, 3},  // sb 965.74 us, db 907.13 us, ms 915.79 us, ks 1184.60 us
    {8192, 8192, 8192, 2, 0, 9, 0, 3},  // sb 7394.38 us, db 7173.85 us, ms 7200.74 us, ks 9478.37 us
    {256, 256, 256, 5, 17, 7, 13, 6},  // sb 7.40 us, db 6.40 us, ms 6.48 us, ks 4.05 us
    {512, 512, 512, 5, 16, 7, 13, 6},  // sb 12.52 us, db 10.20 us, ms 10.11 us, ks 5.68 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.04 us, db 14.51 us, ms 14.14 us, ks 14.67 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 76.62 us, db 68.66 us, ms 68.90 us, ks 72.32 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 127.98 us, db 117.42 us, ms 121.10 us, ks 158.88 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 419.44 us, db 385.81 us, ms 401.05 us, ks 509.22 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3174.61 us, db 3041.77 us, ms 3057.62 us, ks 3962.03 us
    {64, 4096, 4096, 5, 16, 7, 13, 6},  // sb 95.13 us, db 63.56 us, ms 60.90 us, ks 24.85 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 128.08 us, db 123.02 us, ms 124.54 us, ks 202.22 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 488.57 us, db 460.36 us, ms 464.46 us, ks 620.96 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 66.93 us, db 61.82 us, ms 63.79 us, ks 88.99 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.78 us, db 128.55 us, ms 121.40 us, ks 149.63 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.14 us, db 21.02 us, ms 20.81 us, ks 27.59 us
    {4095, 4095, 4095, 3, 0, 9, 9, 0},  // sb 1003.93 us, db 916.98 us, ms 921.21 us, ks 1307.13 us
    {16, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.38 us, db 70.31 us, ms 69.46 us, ks 15.50 us
    {32, 4096, 4096, 5, 15, 7, 13, 10},  // sb 97.70 us, db 63.49 us, ms 63.46 us, ks 17.13 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.66 us, db 64.22 us, ms 61.30 us, ks 40.28 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 197.15 us, db 128.76 us, ms 124.63 us, ks 48.28 us
    {1, 4096, 4096, 5, 14, 7, 6, 6},  // sb 96.46 us, db 70.08 us, ms 69.26 us, ks 14.20 us
    {8, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.29 us, db 70.31 us, ms 69.44 us, ks 14.57 us
    {16, 11008, 4096, 5, 16, 7, 13, 6},  // sb 100.25 us, db 70.81 us, ms 70.05 us, ks 30.70 us
    {16, 4096, 11008, 5, 14, 7, 6, 7},  // sb 262.15 us, db 183.89 us, ms 180.76 us, ks 37.63 us
    {16, 8192, 8192, 5, 17, 7, 13, 6},  // sb 195.12 us, db 140.28 us, ms 136.04 us, ks 39.60 us
    {4, 1024, 1024, 5, 14, 7, 6, 6},  // sb 23.37 us, db 19.68 us, ms 19.69 us, ks 4.54 us
    {16, 32000, 4096, 3, 10, 13, 13, 10},  // sb 154.87 us, db 108.87 us, ms 85.32 us, ks 96.40 us
    {1024, 8192, 8192, 2, 2, 7, 2, 9},  // sb 1006.13 us, db 901.61 us, ms 919.58 us, ks 1178.68 us
};
constexpr int kDispatchRows = (int)(sizeof(kDispatch) / sizeof(kDispatch[0]));

static inline double dispatch_log2(int64_t x) { return x > 0 ? std::log2((double)x) : -1.0; }

static inline const DispatchRow* dispatch_exact(int64_t M, int64_t N, int64_t K) {
  for (int i = 0; i < kDispatchRows; ++i)
    if (kDispatch[i].m == M && kDispatch[i].n == N && kDispatch[i].k == K) return &kDispatch[i];
  return nullptr;
}

// Cost model of every (variant, configuration) for shapes outside the table.  Its features
// are what the regimes turn on: how many tiles the busiest compute unit multiplies,
// rounds = ceil(workgroups / 256), the K tiles per tile, k_tiles = ceil(K / BK), and the
// whole launch's tile work spread over the 256 compute units, work = workgroups * k_tiles
// / 256.  A launch is modelled as
//     a + b * rounds + g * rounds * k_tiles + h * work   microseconds,
// a being the fixed cost (launch, first copy, epilogue), g the time of one K tile of one
// round when the compute units run side by side (the matrix cores bound it), h the time of
// one K tile of work when the memory system that all compute units share bounds it (a
// product that streams B, where a partly filled round of workgroups is not cheaper per
// byte), and b a cost per round that only the K-split kernels have (each of their rounds
// ends in a hand-off through LDS; b = 0 elsewhere).  They were fitted per pair by least
// squares on relative error, all kept >= 0, to the 82 shapes measured for this file
// (the table's 34 and 48 seeded shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, b_us, g_us, h_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.3915, 0.0000, 4.01728, 0.38009},  // median |error| 2.0%
    {1, 1, 10.1300, 0.0000, 7.71576, 0.50833},  // median |error| 1.3%
    {1, 2, 5.7403, 0.0000, 2.21796, 0.00000},  // median |error| 4.3%
    {1, 3, 3.9902, 0.0000, 1.20930, 0.00000},  // median |error| 8.8%
    {1, 4, 4.0128, 0.0000, 2.22143, 0.00000},  // median |error| 4.9%
    {1, 5, 3.4668, 0.0000, 1.19290, 0.00000},  // median |error| 7.2%
    {1, 6, 3.0817, 0.0000, 0.64546, 0.00000},  // median |error| 11.4%
    {1, 7, 3.0154, 0.0000, 1.18495, 0.00000},  // median |error| 7.9%
    {1, 8, 6.7400, 0.0000, 7.60066, 0.37294},  // median |error| 1.5%
    {1, 9, 4.4994, 0.0000, 4.05955, 0.00000},  // median |error| 2.4%
    {1, 10, 3.1592, 0.0000, 0.67001, 0.00000},  // median |error| 14.0%
    {1, 11, 6.4923, 0.0000, 2.43613, 0.28970},  // median |error| 2.9%
    {1, 12, 6.8563, 0.0000, 4.54440, 0.41346},  // median |error| 1.7%
    {1, 13, 4.5029, 0.0000, 0.18287, 0.00000},  // median |error| 22.8%
    {2, 0, 10.3735, 0.0000, 3.45257, 0.10785},  // median |error| 1.2%
    {2, 1, 10.6782, 0.0000, 6.91691, 0.20482},  // median |error| 1.2%
    {2, 2, 6.4788, 0.0000, 1.74697, 0.05170},  // median |error| 1.4%
    {2, 3, 4.4297, 0.0000, 0.88305, 0.07185},  // median |error| 2.4%
    {2, 4, 4.6388, 0.0000, 1.75081, 0.06255},  // median |error| 1.5%
    {2, 5, 4.0136, 0.0000, 0.92361, 0.00873},  // median |error| 1.9%
    {2, 6, 3.1363, 0.0000, 0.50117, 0.00000},  // median |error| 4.0%
    {2, 7, 3.1396, 0.0000, 1.04871, 0.00000},  // median |error| 3.4%
    {2, 8, 7.2826, 0.0000, 7.03134, 0.24844},  // median |error| 0.8%
    {2, 9, 5.2442, 0.0000, 3.46853, 0.13170},  // median |error| 0.8%
    {2, 10, 3.1852, 0.0000, 0.53280, 0.00000},  // median |error| 4.5%
    {2, 11, 7.2126, 0.0000, 1.97914, 0.05161},  // median |error| 0.8%
    {2, 12, 7.7431, 0.0000, 3.90943, 0.12893},  // median |error| 0.7%
    {2, 13, 4.4277, 0.0000, 0.16737, 0.00000},  // median |error| 18.3%
    {3, 0, 10.3464, 0.0000, 3.53425, 0.15316},  // median |error| 1.8%
    {3, 1, 10.8598, 0.0000, 7.07143, 0.39410},  // median |error| 1.8%
    {3, 2, 6.8939, 0.0000, 1.78449, 0.07958},  // median |error| 1.8%
    {3, 3, 4.5750, 0.0000, 0.90808, 0.01300},  // median |error| 2.0%
    {3, 4, 4.6242, 0.0000, 1.80046, 0.11449},  // median |error| 1.6%
    {3, 5, 4.2278, 0.0000, 0.92066, 0.07597},  // median |error| 1.6%
    {3, 6, 3.2809, 0.0000, 0.49687, 0.00000},  // median |error| 4.0%
    {3, 7, 3.2538, 0.0000, 1.04240, 0.07365},  // median |error| 3.3%
    {3, 8, 7.7592, 0.0000, 7.05088, 0.23420},  // median |error| 1.0%
    {3, 9, 5.2837, 0.0000, 3.51167, 0.15012},  // median |error| 1.1%
    {3, 10, 3.2366, 0.0000, 0.52150, 0.00000},  // median |error| 4.6%
    {3, 11, 7.2551, 0.0000, 2.03094, 0.07740},  // median |error| 2.4%
    {3, 12, 7.7815, 0.0000, 4.01947, 0.22703},  // median |error| 2.5%
    {5, 13, 2.7918, 0.9769, 0.15470, 0.00000},  // median |error| 6.6%
    {5, 14, 2.9068, 0.5996, 0.04711, 0.02438},  // median |error| 8.8%
    {5, 15, 2.7497, 0.5848, 0.09412, 0.00000},  // median |error| 9.4%
    {5, 16, 1.4950, 1.9692, 0.15712, 0.01368},  // median |error| 4.8%
    {5, 17, 3.2329, 0.1463, 0.09917, 0.00000},  // median |error| 9.0%
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
  return r.a_us + r.b_us * (double)rounds + r.g_us * (double)rounds * (double)k_tiles +
         r.h_us * (double)tiles * (double)k_tiles / (double)kModelCUs;
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
//     3.4019 us (the reduction's launch)
//   + 0.13900 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.3463 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 3.4019;
constexpr double kSplitUsPerMB = 0.13900;
constexpr double kSplitUsPerRound = 0.3463;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 1},  // 1: 15.4, 2: 38.9, 4: 23.4, 8: 17.6, 16: 21.5
    {32, 4096, 4096, 1},  // 1: 17.1, 2: 39.3, 4: 23.7, 8: 17.3, 16: 21.7
    {64, 4096, 4096, 4},  // 1: 24.8, 2: 35.0, 4: 23.0, 8: 23.6, 16: 26.9
    {128, 4096, 4096, 2},  // 1: 40.9, 2: 36.2, 4: 38.1, 8: 39.6, 16: 43.5
    {32, 8192, 8192, 4},  // 1: 48.5, 2: 72.9, 4: 45.1, 8: 46.8, 16: 52.6
    {64, 8192, 8192, 2},  // 1: 83.4, 2: 69.5, 4: 73.9, 8: 77.6, 16: 89.2
    {256, 256, 8192, 16},  // 1: 24.1, 2: 62.9, 4: 34.8, 8: 22.6, 16: 17.3
    {512, 512, 8192, 4},  // 1: 46.1, 2: 63.9, 4: 35.9, 8: 38.2, 16: 40.3
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.8, 4: 29.3, 8: 32.9, 16: 40.2
    {2048, 2048, 2048, 1},  // 1: 117.7, 2: 129.8, 4: 140.4, 8: 158.6, 16: 207.4
    {4096, 4096, 4096, 1},  // 1: 905.8, 2: 946.6, 4: 997.8, 8: 1126.6, 16: 1294.8, -2: 1078.3, -4: 1089.6, -8: 1124.2, -16: 1175.2
    {1536, 1536, 1536, -4},  // 1: 69.1, 2: 66.9, 4: 64.8, 8: 77.4, 16: 89.5, -2: 62.2, -4: 58.2, -8: 58.3, -16: 63.9
    {1536, 1536, 4096, -8},  // 1: 174.4, 2: 155.7, 4: 143.5, 8: 154.8, 16: 184.7, -2: 151.0, -4: 143.7, -8: 138.4, -16: 142.1
    {2560, 2560, 2560, -8},  // 1: 258.6, 2: 262.7, 4: 273.9, 8: 308.7, 16: 365.2, -2: 249.5, -4: 243.0, -8: 237.9, -16: 244.3
    {1280, 1280, 2048, 1},  // 1: 62.1, 2: 66.2, 4: 68.0, 8: 72.2, 16: 82.9, -2: 67.3, -4: 62.4, -8: 64.9, -16: 67.1
    {5000, 5000, 1000, -8},  // 1: 393.5, 2: 450.3, 4: 528.5, 8: 761.6, 16: 1150.3, -2: 391.2, -4: 391.0, -8: 380.2, -16: 385.4
    {1536, 3072, 4096, -8},  // 1: 291.8, 2: 270.4, 4: 280.6, 8: 320.8, 16: 372.5, -2: 276.5, -4: 270.2, -8: 266.3, -16: 270.1
    {39, 432, 6224, 1},  // 1: 13.8, 2: 56.1, 4: 32.0, 8: 20.7, 16: 16.4
    {11, 1640, 2822, 1},  // 1: 7.5, 2: 29.1, 4: 18.5, 8: 13.1, 16: 12.3
    {11, 1486, 1136, 1},  // 1: 5.4, 2: 14.5, 4: 10.9, 8: 9.5, 16: 9.6
    {66, 326, 1317, 1},  // 1: 5.4, 2: 16.8, 4: 12.2, 8: 9.7, 16: 9.9
    {63, 4495, 1443, 1},  // 1: 17.7, 2: 19.2, 4: 19.1, 8: 19.0, 16: 19.6
    {24, 2252, 14173, 8},  // 1: 55.4, 2: 121.5, 4: 64.5, 8: 38.1, 16: 40.6
    {132, 1012, 15340, 16},  // 1: 85.1, 2: 132.1, 4: 69.6, 8: 65.6, 16: 56.0
    {10, 5016, 2286, 1},  // 1: 10.7, 2: 24.6, 4: 16.9, 8: 19.8, 16: 17.1
    {16, 385, 2409, 1},  // 1: 7.0, 2: 25.0, 4: 16.0, 8: 12.0, 16: 11.0
    {420, 479, 5136, 4},  // 1: 32.1, 2: 48.3, 4: 28.6, 8: 31.1, 16: 34.2
    {178, 931, 4676, 16},  // 1: 29.9, 2: 44.4, 4: 26.4, 8: 28.8, 16: 25.9
    {11, 315, 1813, 1},  // 1: 6.0, 2: 20.7, 4: 13.9, 8: 10.6, 16: 10.2
    {217, 1127, 2447, 1},  // 1: 18.4, 2: 26.7, 4: 18.5, 8: 21.4, 16: 23.2
    {137, 1231, 2351, 1},  // 1: 17.6, 2: 25.4, 4: 17.6, 8: 19.8, 16: 22.4
    {378, 2886, 2015, -8},  // 1: 56.3, 2: 57.4, 4: 52.7, 8: 56.9, 16: 67.7, -2: 52.3, -4: 47.0, -8: 44.7, -16: 45.7
    {130, 1580, 11590, 1},  // 1: 65.8, 2: 101.1, 4: 94.1, 8: 74.3, 16: 71.5
    {276, 694, 15508, 8},  // 1: 88.1, 2: 133.0, 4: 70.0, 8: 68.4, 16: 73.7
    {14, 1090, 8356, 16},  // 1: 25.0, 2: 73.6, 4: 39.8, 8: 24.4, 16: 18.7
    {17, 1394, 1142, 1},  // 1: 5.4, 2: 14.5, 4: 11.0, 8: 9.4, 16: 9.3
    {205, 3623, 5015, 4},  // 1: 87.0, 2: 83.4, 4: 83.2, 8: 84.7, 16: 93.3
    {560, 759, 7039, 4},  // 1: 73.1, 2: 64.8, 4: 61.4, 8: 61.6, 16: 68.4
    {143, 1910, 3628, 2},  // 1: 41.6, 2: 35.8, 4: 36.1, 8: 40.2, 16: 38.5
    {471, 6763, 3812, -8},  // 1: 221.8, 2: 218.7, 4: 217.0, 8: 243.0, 16: 303.0, -2: 210.7, -4: 211.9, -8: 207.0, -16: 208.5
    {201, 316, 7161, 8},  // 1: 29.7, 2: 64.6, 4: 35.7, 8: 22.5, 16: 24.9
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
    const double kt = (double)((K + e.bk - 1) / e.bk), kct = (double)((kc + e.bk - 1) / e.bk);
    const double t = r.a_us + r.b_us * ((double)(full / kModelCUs) + tail_rounds) +
                     r.g_us * ((double)(full / kModelCUs) * kt + tail_rounds * kct) +
                     r.h_us * ((double)full * kt + (double)(tail * used) * kct) /
                         (double)kModelCUs +
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
