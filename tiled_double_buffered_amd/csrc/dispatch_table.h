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
    {128, 128, 128, 5, 17, 7, 6, 6},  // sb 4.84 us, db 4.48 us, ms 4.53 us, ks 4.12 us
    {127, 193, 61, 1, 7, 7, 6, 6},  // sb 4.24 us, db 4.25 us, ms 4.28 us, ks 4.23 us
    {513, 257, 129, 5, 16, 13, 6, 6},  // sb 6.29 us, db 5.90 us, ms 5.94 us, ks 4.30 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.71 us, db 18.55 us, ms 17.95 us, ks 23.99 us
    {256, 1024, 128, 5, 13, 7, 13, 6},  // sb 4.99 us, db 4.60 us, ms 4.79 us, ks 4.20 us
    {1024, 128, 256, 5, 17, 7, 13, 6},  // sb 7.44 us, db 6.44 us, ms 6.49 us, ks 4.25 us
    {4096, 4096, 4096, 2, 0, 9, 0, 3},  // sb 965.98 us, db 908.88 us, ms 915.24 us, ks 1196.04 us
    {8192, 8192, 8192, 2, 0, 4, 0, 3},  // sb 7363.37 us, db 7191.36 us, ms 7188.20 us, ks 9542.48 us
    {256, 256, 256, 5, 17, 7, 13, 6},  // sb 7.39 us, db 6.41 us, ms 6.44 us, ks 4.27 us
    {512, 512, 512, 5, 16, 7, 13, 6},  // sb 12.55 us, db 10.23 us, ms 10.11 us, ks 5.73 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.05 us, db 14.50 us, ms 14.08 us, ks 14.43 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 76.44 us, db 68.60 us, ms 68.71 us, ks 72.13 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 128.36 us, db 118.02 us, ms 121.21 us, ks 159.02 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 422.78 us, db 387.03 us, ms 402.36 us, ks 515.01 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3175.97 us, db 3050.02 us, ms 3050.39 us, ks 3979.43 us
    {64, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.73 us, db 63.76 us, ms 60.80 us, ks 24.96 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 128.32 us, db 122.78 us, ms 124.60 us, ks 201.56 us
    {2048, 8192, 2048, 2, 0, 9, 0, 8},  // sb 488.51 us, db 459.73 us, ms 466.93 us, ks 623.76 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 66.89 us, db 61.92 us, ms 63.66 us, ks 88.52 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.96 us, db 129.19 us, ms 121.45 us, ks 151.08 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.24 us, db 21.05 us, ms 20.67 us, ks 27.55 us
    {4095, 4095, 4095, 2, 0, 9, 0, 0},  // sb 998.93 us, db 918.50 us, ms 921.34 us, ks 1324.24 us
    {16, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.40 us, db 70.18 us, ms 69.52 us, ks 16.30 us
    {32, 4096, 4096, 5, 15, 7, 13, 10},  // sb 98.03 us, db 63.76 us, ms 63.39 us, ks 18.29 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 96.09 us, db 64.61 us, ms 61.33 us, ks 40.60 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 196.30 us, db 129.22 us, ms 124.08 us, ks 48.23 us
    {1, 4096, 4096, 5, 14, 7, 6, 6},  // sb 96.71 us, db 69.85 us, ms 69.28 us, ks 14.79 us
    {8, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.57 us, db 70.13 us, ms 69.43 us, ks 15.27 us
    {16, 11008, 4096, 5, 16, 7, 13, 6},  // sb 100.36 us, db 70.96 us, ms 69.97 us, ks 31.02 us
    {16, 4096, 11008, 5, 14, 7, 6, 6},  // sb 261.49 us, db 183.44 us, ms 181.77 us, ks 37.43 us
    {16, 8192, 8192, 5, 17, 7, 6, 6},  // sb 195.26 us, db 140.69 us, ms 135.87 us, ks 39.91 us
    {4, 1024, 1024, 5, 14, 7, 6, 6},  // sb 23.33 us, db 19.57 us, ms 19.62 us, ks 4.54 us
    {16, 32000, 4096, 3, 10, 13, 13, 10},  // sb 154.80 us, db 109.30 us, ms 86.97 us, ks 96.00 us
    {1024, 8192, 8192, 2, 2, 7, 2, 9},  // sb 1008.51 us, db 905.22 us, ms 922.78 us, ks 1192.77 us
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
    {1, 0, 9.9281, 0.0000, 4.01675, 0.39740},  // median |error| 2.6%
    {1, 1, 10.1421, 0.0000, 7.71133, 0.54964},  // median |error| 1.5%
    {1, 2, 6.0464, 0.0000, 2.22482, 0.00000},  // median |error| 4.5%
    {1, 3, 3.9765, 0.0000, 1.21346, 0.00000},  // median |error| 8.7%
    {1, 4, 4.0922, 0.0000, 2.22598, 0.00000},  // median |error| 4.9%
    {1, 5, 3.3456, 0.0000, 1.19737, 0.00000},  // median |error| 7.4%
    {1, 6, 3.0330, 0.0000, 0.65224, 0.00000},  // median |error| 11.0%
    {1, 7, 3.0580, 0.0000, 1.19515, 0.00000},  // median |error| 8.6%
    {1, 8, 6.5966, 0.0000, 7.60006, 0.40400},  // median |error| 1.7%
    {1, 9, 4.3247, 0.0000, 4.06315, 0.00000},  // median |error| 2.5%
    {1, 10, 3.0957, 0.0000, 0.68083, 0.00000},  // median |error| 13.1%
    {1, 11, 6.1924, 0.0000, 2.44348, 0.28951},  // median |error| 3.0%
    {1, 12, 6.7232, 0.0000, 4.56872, 0.40817},  // median |error| 2.0%
    {1, 13, 4.5780, 0.0000, 0.18851, 0.00000},  // median |error| 22.3%
    {2, 0, 10.0852, 0.0000, 3.45023, 0.12353},  // median |error| 0.9%
    {2, 1, 10.3766, 0.0000, 6.90613, 0.24533},  // median |error| 1.0%
    {2, 2, 6.7344, 0.0000, 1.74021, 0.06564},  // median |error| 1.5%
    {2, 3, 4.4884, 0.0000, 0.88123, 0.08257},  // median |error| 2.4%
    {2, 4, 4.6158, 0.0000, 1.74775, 0.07432},  // median |error| 1.5%
    {2, 5, 4.1019, 0.0000, 0.92273, 0.01650},  // median |error| 2.1%
    {2, 6, 3.1616, 0.0000, 0.50655, 0.00000},  // median |error| 3.3%
    {2, 7, 3.1937, 0.0000, 1.05516, 0.00000},  // median |error| 2.9%
    {2, 8, 7.1824, 0.0000, 7.05075, 0.26023},  // median |error| 0.9%
    {2, 9, 5.2791, 0.0000, 3.45981, 0.15439},  // median |error| 0.8%
    {2, 10, 3.1464, 0.0000, 0.54148, 0.00000},  // median |error| 3.9%
    {2, 11, 7.0375, 0.0000, 1.97715, 0.06783},  // median |error| 0.5%
    {2, 12, 7.6551, 0.0000, 3.89994, 0.16284},  // median |error| 0.6%
    {2, 13, 4.4517, 0.0000, 0.17340, 0.00000},  // median |error| 20.1%
    {3, 0, 10.5682, 0.0000, 3.52960, 0.17267},  // median |error| 1.9%
    {3, 1, 10.4518, 0.0000, 7.06253, 0.42085},  // median |error| 2.0%
    {3, 2, 6.7157, 0.0000, 1.78372, 0.08819},  // median |error| 1.7%
    {3, 3, 4.6112, 0.0000, 0.90753, 0.01718},  // median |error| 2.3%
    {3, 4, 4.8341, 0.0000, 1.79443, 0.12482},  // median |error| 1.8%
    {3, 5, 4.1385, 0.0000, 0.92014, 0.08154},  // median |error| 1.7%
    {3, 6, 3.2057, 0.0000, 0.50231, 0.00000},  // median |error| 3.2%
    {3, 7, 3.2716, 0.0000, 1.03723, 0.08240},  // median |error| 3.2%
    {3, 8, 7.6083, 0.0000, 7.02449, 0.27064},  // median |error| 0.8%
    {3, 9, 5.3482, 0.0000, 3.50292, 0.16839},  // median |error| 1.2%
    {3, 10, 3.2019, 0.0000, 0.52832, 0.00000},  // median |error| 4.4%
    {3, 11, 7.2619, 0.0000, 2.02824, 0.08562},  // median |error| 2.5%
    {3, 12, 7.7497, 0.0000, 4.01336, 0.24822},  // median |error| 2.6%
    {5, 13, 2.7636, 1.0023, 0.16111, 0.00000},  // median |error| 6.5%
    {5, 14, 2.9479, 0.5975, 0.04658, 0.02869},  // median |error| 10.7%
    {5, 15, 2.8145, 0.6020, 0.09744, 0.00000},  // median |error| 11.2%
    {5, 16, 1.6035, 1.9345, 0.15741, 0.02239},  // median |error| 7.8%
    {5, 17, 3.2906, 0.1720, 0.10182, 0.00000},  // median |error| 11.8%
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

// Above 16 rows every 16-row tile streams its strip of B again, ceil(M / 16) times in all.
// How fast that goes depends on how much of it the caches catch, which the model above does
// not see; measured, the 16-row kernels win above 16 rows while those re-reads stay small
// and lose by up to 2x beyond (a 208 x 5875 x 8154 product streams 2.5 GB).  So the model
// offers them above 16 rows only up to this many bytes of B streamed.
constexpr double kRowTileStreamLimitBytes = 100e6;

static inline bool model_allows(const CfgEntry& e, int64_t M, int64_t N, int64_t K) {
  if (e.bm != 16 || M <= 16) return true;
  return (double)((M + 15) / 16) * 4.0 * (double)N * (double)K <= kRowTileStreamLimitBytes;
}

// The row with the least modelled time (variant 0: any variant), first row on ties.
static inline const ModelRow& model_pick(int64_t M, int64_t N, int64_t K, int variant,
                                         int64_t wg_factor) {
  int best = 0;
  double best_t = 0.0;
  bool found = false;
  for (int i = 0; i < kModelRows; ++i) {
    if (variant != 0 && kModel[i].variant != variant) continue;
    if (!model_allows(kConfigs[kModel[i].cfg], M, N, K)) continue;
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
//     3.1327 us (the reduction's launch)
//   + 0.12757 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.5608 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 3.1327;
constexpr double kSplitUsPerMB = 0.12757;
constexpr double kSplitUsPerRound = 0.5608;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 1},  // 1: 16.4, 2: 38.9, 4: 23.0, 8: 17.5, 16: 21.3
    {32, 4096, 4096, 8},  // 1: 18.5, 2: 39.2, 4: 23.4, 8: 17.2, 16: 21.7
    {64, 4096, 4096, 4},  // 1: 25.1, 2: 34.9, 4: 21.1, 8: 24.1, 16: 28.9
    {128, 4096, 4096, 2},  // 1: 39.7, 2: 35.7, 4: 37.3, 8: 39.3, 16: 43.4
    {32, 8192, 8192, 4},  // 1: 48.1, 2: 73.3, 4: 45.2, 8: 46.4, 16: 52.2
    {64, 8192, 8192, 2},  // 1: 79.2, 2: 66.6, 4: 70.6, 8: 74.5, 16: 85.3
    {256, 256, 8192, 16},  // 1: 45.7, 2: 62.8, 4: 34.7, 8: 21.8, 16: 17.1
    {512, 512, 8192, 4},  // 1: 46.0, 2: 63.4, 4: 35.6, 8: 37.6, 16: 40.3
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.8, 4: 29.3, 8: 32.9, 16: 40.4
    {2048, 2048, 2048, 1},  // 1: 117.4, 2: 129.2, 4: 140.0, 8: 157.8, 16: 206.2
    {4096, 4096, 4096, 1},  // 1: 903.5, 2: 943.8, 4: 996.2, 8: 1124.1, 16: 1291.0, -2: 1064.5, -4: 1076.5, -8: 1119.3, -16: 1170.7
    {1536, 1536, 1536, -4},  // 1: 68.1, 2: 66.3, 4: 64.7, 8: 77.8, 16: 88.7, -2: 61.4, -4: 57.0, -8: 57.9, -16: 64.1
    {1536, 1536, 4096, -4},  // 1: 174.0, 2: 153.8, 4: 142.9, 8: 154.5, 16: 174.7, -2: 149.3, -4: 136.5, -8: 136.9, -16: 139.5
    {2560, 2560, 2560, -8},  // 1: 255.7, 2: 258.3, 4: 267.9, 8: 302.6, 16: 363.5, -2: 242.3, -4: 240.3, -8: 233.3, -16: 241.5
    {1280, 1280, 2048, -4},  // 1: 61.9, 2: 66.0, 4: 66.0, 8: 71.4, 16: 82.8, -2: 66.6, -4: 61.1, -8: 62.3, -16: 66.5
    {5000, 5000, 1000, -4},  // 1: 392.8, 2: 442.8, 4: 522.5, 8: 758.3, 16: 1153.5, -2: 381.5, -4: 376.4, -8: 379.9, -16: 385.7
    {1536, 3072, 4096, -4},  // 1: 289.4, 2: 269.6, 4: 280.2, 8: 310.0, 16: 370.0, -2: 266.9, -4: 265.8, -8: 265.9, -16: 269.6
    {39, 432, 6224, 16},  // 1: 17.5, 2: 56.1, 4: 31.8, 8: 20.5, 16: 16.2
    {11, 1640, 2822, 1},  // 1: 9.8, 2: 29.1, 4: 18.4, 8: 13.1, 16: 12.2
    {11, 1486, 1136, 1},  // 1: 5.3, 2: 14.6, 4: 11.0, 8: 9.6, 16: 9.6
    {66, 326, 1317, 1},  // 1: 5.3, 2: 17.6, 4: 12.1, 8: 9.9, 16: 9.9
    {63, 4495, 1443, 2},  // 1: 25.8, 2: 18.8, 4: 20.2, 8: 21.0, 16: 22.3
    {24, 2252, 14173, 8},  // 1: 78.6, 2: 121.3, 4: 64.2, 8: 38.0, 16: 40.2
    {132, 1012, 15340, 16},  // 1: 85.0, 2: 131.5, 4: 69.2, 8: 65.3, 16: 55.0
    {10, 5016, 2286, 1},  // 1: 13.9, 2: 24.6, 4: 16.8, 8: 19.8, 16: 17.0
    {16, 385, 2409, 1},  // 1: 7.0, 2: 24.9, 4: 16.0, 8: 11.8, 16: 11.1
    {420, 479, 5136, 4},  // 1: 32.0, 2: 48.1, 4: 28.5, 8: 31.3, 16: 34.0
    {178, 931, 4676, 4},  // 1: 30.6, 2: 44.8, 4: 26.3, 8: 28.9, 16: 33.3
    {11, 315, 1813, 1},  // 1: 5.9, 2: 20.5, 4: 13.9, 8: 10.6, 16: 10.3
    {217, 1127, 2447, 4},  // 1: 20.7, 2: 26.6, 4: 18.3, 8: 21.2, 16: 25.5
    {137, 1231, 2351, 4},  // 1: 20.0, 2: 25.4, 4: 17.6, 8: 19.9, 16: 23.8
    {378, 2886, 2015, -8},  // 1: 82.3, 2: 55.3, 4: 51.1, 8: 56.6, 16: 69.1, -2: 53.9, -4: 48.0, -8: 45.8, -16: 47.5
    {130, 1580, 11590, 8},  // 1: 94.2, 2: 103.1, 4: 94.4, 8: 74.3, 16: 76.7
    {276, 694, 15508, 8},  // 1: 86.6, 2: 132.4, 4: 69.8, 8: 67.5, 16: 72.2
    {14, 1090, 8356, 16},  // 1: 27.3, 2: 73.4, 4: 39.7, 8: 24.4, 16: 18.6
    {17, 1394, 1142, 1},  // 1: 5.3, 2: 14.6, 4: 10.9, 8: 9.6, 16: 9.4
    {205, 3623, 5015, 4},  // 1: 99.8, 2: 83.7, 4: 83.1, 8: 83.6, 16: 90.0
    {560, 759, 7039, 4},  // 1: 71.7, 2: 64.7, 4: 61.3, 8: 61.4, 16: 62.5
    {143, 1910, 3628, 2},  // 1: 51.8, 2: 36.3, 4: 36.5, 8: 40.4, 16: 42.3
    {471, 6763, 3812, -2},  // 1: 220.6, 2: 215.0, 4: 214.5, 8: 237.5, 16: 302.2, -2: 206.0, -4: 211.0, -8: 254.8, -16: 259.2
    {201, 316, 7161, 8},  // 1: 41.9, 2: 65.5, 4: 35.6, 8: 22.5, 16: 25.1
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
