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
    {128, 128, 128, 5, 13, 7, 6, 6},  // sb 4.79 us, db 4.53 us, ms 4.55 us, ks 4.10 us
    {127, 193, 61, 5, 14, 13, 13, 6},  // sb 4.19 us, db 4.25 us, ms 4.29 us, ks 4.11 us
    {513, 257, 129, 5, 16, 13, 13, 6},  // sb 6.17 us, db 5.82 us, ms 5.97 us, ks 4.18 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.72 us, db 18.53 us, ms 17.98 us, ks 24.02 us
    {256, 1024, 128, 5, 17, 7, 13, 6},  // sb 5.06 us, db 4.56 us, ms 4.75 us, ks 4.07 us
    {1024, 128, 256, 5, 17, 7, 13, 6},  // sb 7.44 us, db 6.42 us, ms 6.51 us, ks 4.03 us
    {4096, 4096, 4096, 2, 0, 18, 0, 3},  // sb 947.74 us, db 900.41 us, ms 908.38 us, ks 1183.99 us
    {8192, 8192, 8192, 2, 0, 4, 0, 3},  // sb 7315.52 us, db 7138.96 us, ms 7152.85 us, ks 9456.04 us
    {256, 256, 256, 5, 17, 7, 13, 6},  // sb 7.41 us, db 6.38 us, ms 6.48 us, ks 3.71 us
    {512, 512, 512, 5, 16, 7, 13, 6},  // sb 12.52 us, db 10.19 us, ms 10.10 us, ks 5.64 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 17.99 us, db 14.46 us, ms 14.09 us, ks 14.64 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 76.45 us, db 68.69 us, ms 68.75 us, ks 70.71 us
    {2048, 2048, 2048, 2, 3, 6, 3, 18},  // sb 127.55 us, db 117.14 us, ms 119.54 us, ks 158.06 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 419.15 us, db 383.39 us, ms 399.19 us, ks 510.89 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3160.44 us, db 3021.55 us, ms 3039.85 us, ks 3934.46 us
    {64, 4096, 4096, 5, 16, 7, 13, 6},  // sb 95.68 us, db 63.53 us, ms 61.06 us, ks 24.87 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 127.11 us, db 122.36 us, ms 123.86 us, ks 201.26 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 485.42 us, db 457.45 us, ms 460.96 us, ks 620.24 us
    {4096, 1024, 1024, 2, 3, 7, 3, 18},  // sb 66.84 us, db 61.80 us, ms 63.15 us, ks 88.67 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.71 us, db 128.90 us, ms 121.78 us, ks 150.66 us
    {512, 4096, 4096, 3, 18, 6, 18, 18},  // sb 135.10 us, db 118.95 us, ms 116.43 us, ks 152.02 us
    {512, 4096, 11008, 3, 18, 6, 18, 18},  // sb 345.00 us, db 314.00 us, ms 307.22 us, ks 391.58 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.15 us, db 20.94 us, ms 20.76 us, ks 27.87 us
    {4095, 4095, 4095, 3, 0, 9, 0, 0},  // sb 999.86 us, db 913.77 us, ms 913.29 us, ks 1308.75 us
    {16, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.71 us, db 70.49 us, ms 69.65 us, ks 15.55 us
    {32, 4096, 4096, 5, 15, 7, 13, 10},  // sb 98.34 us, db 63.75 us, ms 63.71 us, ks 17.19 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.46 us, db 63.82 us, ms 61.04 us, ks 40.15 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 196.58 us, db 128.41 us, ms 124.35 us, ks 48.26 us
    {1, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.17 us, db 70.41 us, ms 69.49 us, ks 14.29 us
    {8, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.62 us, db 70.55 us, ms 69.63 us, ks 14.65 us
    {16, 11008, 4096, 5, 16, 7, 13, 6},  // sb 100.02 us, db 70.60 us, ms 69.73 us, ks 30.89 us
    {16, 4096, 11008, 5, 14, 7, 6, 6},  // sb 262.42 us, db 184.35 us, ms 182.06 us, ks 37.64 us
    {16, 8192, 8192, 5, 17, 7, 13, 6},  // sb 195.68 us, db 140.39 us, ms 136.27 us, ks 39.77 us
    {4, 1024, 1024, 5, 14, 7, 6, 6},  // sb 23.37 us, db 19.67 us, ms 19.67 us, ks 4.55 us
    {16, 32000, 4096, 3, 10, 13, 13, 10},  // sb 154.37 us, db 108.74 us, ms 85.64 us, ks 96.38 us
    {1024, 8192, 8192, 2, 2, 7, 2, 3},  // sb 1002.50 us, db 899.50 us, ms 912.77 us, ks 1181.05 us
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
// squares on relative error, all kept >= 0, to the 84 shapes measured for this file
// (the table's 36 and 48 seeded shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, b_us, g_us, h_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.3728, 0.0000, 4.02716, 0.35254},  // median |error| 2.0%
    {1, 1, 10.1124, 0.0000, 7.73141, 0.46750},  // median |error| 1.4%
    {1, 2, 5.7328, 0.0000, 2.22072, 0.00000},  // median |error| 4.2%
    {1, 3, 3.9777, 0.0000, 1.21180, 0.00000},  // median |error| 9.0%
    {1, 4, 4.0103, 0.0000, 2.22303, 0.00000},  // median |error| 5.0%
    {1, 5, 3.4672, 0.0000, 1.19755, 0.00000},  // median |error| 7.6%
    {1, 6, 3.1125, 0.0000, 0.63582, 0.00000},  // median |error| 12.6%
    {1, 7, 3.0355, 0.0000, 1.18089, 0.00000},  // median |error| 7.6%
    {1, 8, 6.7480, 0.0000, 7.60802, 0.31901},  // median |error| 1.4%
    {1, 9, 4.5195, 0.0000, 4.05620, 0.00000},  // median |error| 2.3%
    {1, 10, 3.1991, 0.0000, 0.65901, 0.00000},  // median |error| 13.5%
    {1, 11, 6.4931, 0.0000, 2.43914, 0.27751},  // median |error| 3.0%
    {1, 12, 6.8586, 0.0000, 4.55077, 0.38531},  // median |error| 1.7%
    {1, 13, 4.5417, 0.0000, 0.17999, 0.00000},  // median |error| 20.7%
    {1, 18, 3.0616, 0.0000, 1.17536, 0.00000},  // median |error| 7.4%
    {2, 0, 10.3909, 0.0000, 3.45493, 0.08922},  // median |error| 1.1%
    {2, 1, 10.6935, 0.0000, 6.92182, 0.16154},  // median |error| 1.1%
    {2, 2, 6.4851, 0.0000, 1.74713, 0.04255},  // median |error| 1.4%
    {2, 3, 4.4366, 0.0000, 0.88252, 0.06461},  // median |error| 2.5%
    {2, 4, 4.6436, 0.0000, 1.75111, 0.05179},  // median |error| 1.6%
    {2, 5, 4.0199, 0.0000, 0.92530, 0.00147},  // median |error| 1.9%
    {2, 6, 3.1559, 0.0000, 0.49918, 0.00000},  // median |error| 4.3%
    {2, 7, 3.1606, 0.0000, 1.04411, 0.00000},  // median |error| 3.7%
    {2, 8, 7.2927, 0.0000, 7.03681, 0.18584},  // median |error| 0.6%
    {2, 9, 5.2522, 0.0000, 3.46922, 0.11304},  // median |error| 0.8%
    {2, 10, 3.2135, 0.0000, 0.53034, 0.00000},  // median |error| 5.2%
    {2, 11, 7.2219, 0.0000, 1.97990, 0.04487},  // median |error| 0.8%
    {2, 12, 7.7526, 0.0000, 3.91210, 0.10987},  // median |error| 0.7%
    {2, 13, 4.4355, 0.0000, 0.16450, 0.00000},  // median |error| 18.6%
    {2, 18, 3.3699, 0.0000, 0.93567, 0.00542},  // median |error| 2.6%
    {3, 0, 10.3392, 0.0000, 3.54088, 0.12892},  // median |error| 1.8%
    {3, 1, 10.8395, 0.0000, 7.08836, 0.33020},  // median |error| 2.0%
    {3, 2, 6.8914, 0.0000, 1.78580, 0.07044},  // median |error| 1.8%
    {3, 3, 4.5746, 0.0000, 0.90866, 0.00732},  // median |error| 1.9%
    {3, 4, 4.6235, 0.0000, 1.80187, 0.10390},  // median |error| 1.6%
    {3, 5, 4.2282, 0.0000, 0.92429, 0.06108},  // median |error| 1.7%
    {3, 6, 3.2620, 0.0000, 0.49482, 0.00000},  // median |error| 4.5%
    {3, 7, 3.2399, 0.0000, 1.04965, 0.05124},  // median |error| 3.6%
    {3, 8, 7.7692, 0.0000, 7.05560, 0.18000},  // median |error| 0.9%
    {3, 9, 5.2880, 0.0000, 3.51405, 0.12731},  // median |error| 1.0%
    {3, 10, 3.2503, 0.0000, 0.51917, 0.00000},  // median |error| 4.9%
    {3, 11, 7.2534, 0.0000, 2.03371, 0.06878},  // median |error| 2.4%
    {3, 12, 7.7739, 0.0000, 4.02706, 0.19922},  // median |error| 2.7%
    {3, 18, 3.5252, 0.0000, 0.93274, 0.02597},  // median |error| 2.5%
    {5, 13, 2.7933, 0.9870, 0.15334, 0.00000},  // median |error| 7.2%
    {5, 14, 2.8822, 0.6060, 0.04779, 0.02341},  // median |error| 8.8%
    {5, 15, 2.7821, 0.5928, 0.09326, 0.00000},  // median |error| 8.6%
    {5, 16, 1.5213, 1.9727, 0.15725, 0.01218},  // median |error| 4.9%
    {5, 17, 3.2518, 0.1547, 0.09870, 0.00000},  // median |error| 8.8%
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
//     3.4594 us (the reduction's launch)
//   + 0.14133 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.3726 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 3.4594;
constexpr double kSplitUsPerMB = 0.14133;
constexpr double kSplitUsPerRound = 0.3726;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 1},  // 1: 15.4, 2: 39.0, 4: 23.1, 8: 17.6, 16: 21.5
    {32, 4096, 4096, 1},  // 1: 17.0, 2: 39.4, 4: 23.5, 8: 17.3, 16: 21.6
    {64, 4096, 4096, 4},  // 1: 24.8, 2: 35.1, 4: 21.6, 8: 23.3, 16: 26.9
    {128, 4096, 4096, 2},  // 1: 41.2, 2: 36.1, 4: 37.2, 8: 39.7, 16: 43.7
    {32, 8192, 8192, 4},  // 1: 48.8, 2: 73.2, 4: 45.1, 8: 46.9, 16: 52.7
    {64, 8192, 8192, 2},  // 1: 83.9, 2: 70.9, 4: 74.7, 8: 76.7, 16: 83.8
    {256, 256, 8192, 16},  // 1: 24.1, 2: 63.2, 4: 34.9, 8: 22.0, 16: 17.3
    {512, 512, 8192, 4},  // 1: 46.2, 2: 64.3, 4: 36.0, 8: 37.2, 16: 40.9
    {1024, 1024, 1024, 1},  // 1: 18.1, 2: 24.4, 4: 28.0, 8: 32.8, 16: 39.9
    {2048, 2048, 2048, 1},  // 1: 118.2, 2: 130.2, 4: 141.0, 8: 159.2, 16: 207.5
    {4096, 4096, 4096, 1},  // 1: 909.2, 2: 950.8, 4: 1001.5, 8: 1128.0, 16: 1304.3, -2: 1076.7, -4: 1089.7, -8: 1122.8, -16: 1176.0
    {1536, 1536, 1536, -4},  // 1: 68.9, 2: 67.0, 4: 64.9, 8: 77.6, 16: 89.4, -2: 62.1, -4: 58.3, -8: 58.4, -16: 64.0
    {1536, 1536, 4096, -8},  // 1: 178.3, 2: 156.0, 4: 143.6, 8: 155.2, 16: 184.5, -2: 151.0, -4: 145.0, -8: 138.3, -16: 143.4
    {2560, 2560, 2560, -8},  // 1: 258.7, 2: 262.6, 4: 273.9, 8: 307.0, 16: 365.3, -2: 249.2, -4: 243.0, -8: 238.6, -16: 244.2
    {1280, 1280, 2048, 1},  // 1: 61.9, 2: 66.0, 4: 66.8, 8: 71.9, 16: 82.9, -2: 67.4, -4: 62.2, -8: 64.8, -16: 67.2
    {5000, 5000, 1000, -8},  // 1: 392.3, 2: 451.2, 4: 527.7, 8: 761.9, 16: 1148.8, -2: 393.5, -4: 390.4, -8: 380.5, -16: 385.9
    {1536, 3072, 4096, -8},  // 1: 292.8, 2: 269.8, 4: 280.4, 8: 320.8, 16: 372.6, -2: 277.8, -4: 271.6, -8: 266.4, -16: 270.2
    {39, 432, 6224, 1},  // 1: 13.9, 2: 56.2, 4: 31.9, 8: 20.6, 16: 16.4
    {11, 1640, 2822, 1},  // 1: 7.5, 2: 29.0, 4: 18.5, 8: 13.2, 16: 12.4
    {11, 1486, 1136, 1},  // 1: 5.5, 2: 14.6, 4: 11.2, 8: 9.6, 16: 9.7
    {66, 326, 1317, 1},  // 1: 5.4, 2: 16.9, 4: 12.1, 8: 9.7, 16: 9.7
    {63, 4495, 1443, 1},  // 1: 17.7, 2: 19.2, 4: 19.4, 8: 19.1, 16: 19.7
    {24, 2252, 14173, 8},  // 1: 55.1, 2: 121.5, 4: 64.5, 8: 38.2, 16: 40.6
    {132, 1012, 15340, 16},  // 1: 85.0, 2: 131.8, 4: 69.4, 8: 65.4, 16: 56.3
    {10, 5016, 2286, 1},  // 1: 10.7, 2: 24.5, 4: 17.0, 8: 19.8, 16: 17.1
    {16, 385, 2409, 1},  // 1: 7.1, 2: 25.1, 4: 16.1, 8: 11.8, 16: 11.2
    {420, 479, 5136, 4},  // 1: 32.1, 2: 48.2, 4: 28.6, 8: 30.9, 16: 33.3
    {178, 931, 4676, 4},  // 1: 30.0, 2: 44.4, 4: 26.3, 8: 28.5, 16: 30.3
    {11, 315, 1813, 1},  // 1: 6.0, 2: 20.7, 4: 13.9, 8: 10.6, 16: 10.3
    {217, 1127, 2447, 1},  // 1: 18.5, 2: 26.8, 4: 18.5, 8: 21.4, 16: 22.9
    {137, 1231, 2351, 1},  // 1: 17.6, 2: 25.4, 4: 17.7, 8: 19.8, 16: 22.4
    {378, 2886, 2015, -8},  // 1: 56.5, 2: 57.3, 4: 52.5, 8: 56.9, 16: 65.1, -2: 52.3, -4: 46.9, -8: 44.7, -16: 45.6
    {130, 1580, 11590, 1},  // 1: 65.9, 2: 101.4, 4: 94.4, 8: 74.4, 16: 71.7
    {276, 694, 15508, 8},  // 1: 88.1, 2: 133.3, 4: 70.4, 8: 68.0, 16: 71.0
    {14, 1090, 8356, 16},  // 1: 24.9, 2: 73.9, 4: 40.0, 8: 24.5, 16: 18.7
    {17, 1394, 1142, 1},  // 1: 5.4, 2: 14.6, 4: 11.0, 8: 9.5, 16: 9.3
    {205, 3623, 5015, 4},  // 1: 87.5, 2: 83.7, 4: 83.3, 8: 84.7, 16: 93.1
    {560, 759, 7039, 4},  // 1: 73.4, 2: 65.0, 4: 61.6, 8: 61.8, 16: 67.9
    {143, 1910, 3628, 2},  // 1: 41.7, 2: 36.0, 4: 36.1, 8: 40.3, 16: 38.4
    {471, 6763, 3812, -2},  // 1: 222.3, 2: 219.0, 4: 217.5, 8: 243.8, 16: 303.1, -2: 210.3, -4: 212.5, -8: 210.8, -16: 212.1
    {201, 316, 7161, 8},  // 1: 29.7, 2: 64.8, 4: 35.7, 8: 22.6, 16: 24.6
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
