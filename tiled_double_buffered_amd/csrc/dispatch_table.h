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
    {128, 128, 128, 5, 13, 7, 6, 6},  // sb 4.74 us, db 4.51 us, ms 4.54 us, ks 4.10 us
    {127, 193, 61, 5, 14, 13, 13, 6},  // sb 4.15 us, db 4.14 us, ms 4.16 us, ks 4.10 us
    {513, 257, 129, 5, 13, 13, 13, 6},  // sb 6.23 us, db 5.84 us, ms 5.92 us, ks 4.91 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.72 us, db 18.61 us, ms 17.99 us, ks 23.56 us
    {256, 1024, 128, 5, 13, 7, 13, 6},  // sb 5.01 us, db 4.60 us, ms 4.74 us, ks 4.21 us
    {1024, 128, 256, 5, 14, 7, 13, 6},  // sb 7.48 us, db 6.42 us, ms 6.49 us, ks 4.52 us
    {4096, 4096, 4096, 2, 0, 9, 0, 3},  // sb 958.42 us, db 902.10 us, ms 911.86 us, ks 1226.76 us
    {8192, 8192, 8192, 2, 0, 9, 0, 8},  // sb 7442.40 us, db 7154.39 us, ms 7255.12 us, ks 9871.22 us
    {256, 256, 256, 5, 14, 7, 13, 6},  // sb 7.41 us, db 6.40 us, ms 6.47 us, ks 4.13 us
    {512, 512, 512, 5, 13, 7, 13, 6},  // sb 12.54 us, db 10.21 us, ms 10.09 us, ks 6.18 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.03 us, db 14.52 us, ms 14.08 us, ks 15.81 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 76.98 us, db 68.98 us, ms 69.03 us, ks 72.48 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 129.61 us, db 118.80 us, ms 121.64 us, ks 161.69 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 436.73 us, db 385.37 us, ms 399.09 us, ks 528.02 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3208.39 us, db 3033.00 us, ms 3071.43 us, ks 4135.36 us
    {64, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.86 us, db 63.77 us, ms 60.78 us, ks 25.07 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 127.60 us, db 123.01 us, ms 125.19 us, ks 213.92 us
    {2048, 8192, 2048, 2, 0, 9, 0, 8},  // sb 484.49 us, db 458.42 us, ms 463.43 us, ks 634.01 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 67.07 us, db 62.06 us, ms 63.69 us, ks 88.45 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.54 us, db 130.77 us, ms 125.55 us, ks 157.16 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.28 us, db 21.16 us, ms 20.65 us, ks 27.54 us
    {4095, 4095, 4095, 2, 0, 9, 0, 0},  // sb 998.65 us, db 915.16 us, ms 917.12 us, ks 1376.02 us
    {16, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.50 us, db 70.13 us, ms 69.46 us, ks 16.27 us
    {32, 4096, 4096, 5, 13, 7, 13, 10},  // sb 98.08 us, db 63.86 us, ms 63.38 us, ks 24.81 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 96.04 us, db 64.42 us, ms 61.35 us, ks 42.00 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 196.42 us, db 128.85 us, ms 123.84 us, ks 48.78 us
    {1, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.16 us, db 70.09 us, ms 69.36 us, ks 14.61 us
    {8, 4096, 4096, 5, 14, 7, 6, 6},  // sb 97.76 us, db 70.23 us, ms 69.48 us, ks 15.26 us
    {16, 11008, 4096, 5, 14, 7, 13, 6},  // sb 100.27 us, db 70.90 us, ms 69.81 us, ks 36.83 us
    {16, 4096, 11008, 5, 14, 7, 6, 6},  // sb 262.24 us, db 182.89 us, ms 181.19 us, ks 37.35 us
    {16, 8192, 8192, 5, 13, 7, 6, 6},  // sb 195.34 us, db 140.57 us, ms 135.87 us, ks 48.21 us
    {4, 1024, 1024, 5, 14, 7, 6, 6},  // sb 23.39 us, db 19.59 us, ms 19.64 us, ks 4.52 us
    {1024, 8192, 8192, 2, 2, 7, 2, 9},  // sb 1037.07 us, db 905.77 us, ms 919.57 us, ks 1231.20 us
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
// squares on relative error, all kept >= 0, to the 81 shapes measured for this file
// (the table's 33 and 48 seeded shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, b_us, g_us, h_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.9902, 0.0000, 4.02965, 0.34624},  // median |error| 2.7%
    {1, 1, 10.1961, 0.0000, 7.74162, 0.44217},  // median |error| 1.4%
    {1, 2, 6.1365, 0.0000, 2.21914, 0.00000},  // median |error| 4.3%
    {1, 3, 4.0052, 0.0000, 1.21453, 0.00000},  // median |error| 9.2%
    {1, 4, 4.1303, 0.0000, 2.22700, 0.00000},  // median |error| 5.0%
    {1, 5, 3.3307, 0.0000, 1.20939, 0.00000},  // median |error| 7.7%
    {1, 6, 2.9604, 0.0000, 0.65766, 0.00000},  // median |error| 11.0%
    {1, 7, 2.9462, 0.0000, 1.21206, 0.00000},  // median |error| 9.5%
    {1, 8, 6.6554, 0.0000, 7.62657, 0.31637},  // median |error| 1.7%
    {1, 9, 4.4125, 0.0000, 4.06030, 0.00000},  // median |error| 2.7%
    {1, 10, 3.0491, 0.0000, 0.68330, 0.00000},  // median |error| 11.9%
    {1, 11, 6.2171, 0.0000, 2.45095, 0.25935},  // median |error| 3.1%
    {1, 12, 6.7376, 0.0000, 4.58778, 0.35526},  // median |error| 1.9%
    {1, 13, 4.4620, 0.0000, 0.18708, 0.00000},  // median |error| 23.1%
    {2, 0, 10.1416, 0.0000, 3.46116, 0.09753},  // median |error| 1.0%
    {2, 1, 10.4371, 0.0000, 6.92948, 0.18472},  // median |error| 1.1%
    {2, 2, 6.7751, 0.0000, 1.74374, 0.06377},  // median |error| 1.6%
    {2, 3, 4.4999, 0.0000, 0.88324, 0.08005},  // median |error| 2.5%
    {2, 4, 4.6340, 0.0000, 1.75001, 0.07914},  // median |error| 1.5%
    {2, 5, 4.1214, 0.0000, 0.91666, 0.04608},  // median |error| 2.1%
    {2, 6, 3.0902, 0.0000, 0.51304, 0.00015},  // median |error| 3.0%
    {2, 7, 3.0868, 0.0000, 1.06827, 0.00000},  // median |error| 2.2%
    {2, 8, 7.2471, 0.0000, 7.07509, 0.19663},  // median |error| 0.9%
    {2, 9, 5.3347, 0.0000, 3.47031, 0.12935},  // median |error| 0.7%
    {2, 10, 3.0701, 0.0000, 0.54655, 0.00000},  // median |error| 3.8%
    {2, 11, 7.0706, 0.0000, 1.98348, 0.05851},  // median |error| 0.5%
    {2, 12, 7.6885, 0.0000, 3.91200, 0.14710},  // median |error| 0.6%
    {2, 13, 4.3398, 0.0000, 0.17482, 0.00000},  // median |error| 20.7%
    {3, 0, 10.6333, 0.0000, 3.54138, 0.13811},  // median |error| 2.0%
    {3, 1, 10.5152, 0.0000, 7.08865, 0.33277},  // median |error| 1.9%
    {3, 2, 6.7574, 0.0000, 1.78870, 0.07587},  // median |error| 1.6%
    {3, 3, 4.6209, 0.0000, 0.91005, 0.01348},  // median |error| 2.1%
    {3, 4, 4.8517, 0.0000, 1.79937, 0.11524},  // median |error| 1.8%
    {3, 5, 4.1586, 0.0000, 0.91930, 0.08627},  // median |error| 1.6%
    {3, 6, 3.1332, 0.0000, 0.50890, 0.00000},  // median |error| 2.8%
    {3, 7, 3.1781, 0.0000, 1.04489, 0.07641},  // median |error| 3.0%
    {3, 8, 7.6761, 0.0000, 7.04847, 0.20644},  // median |error| 0.8%
    {3, 9, 5.3963, 0.0000, 3.51469, 0.13477},  // median |error| 1.0%
    {3, 10, 3.1242, 0.0000, 0.53294, 0.00000},  // median |error| 4.2%
    {3, 11, 7.2991, 0.0000, 2.03471, 0.07332},  // median |error| 2.5%
    {3, 12, 7.7856, 0.0000, 4.02711, 0.21601},  // median |error| 2.6%
    {5, 13, 2.7084, 0.9800, 0.16107, 0.00000},  // median |error| 6.9%
    {5, 14, 2.8045, 0.6159, 0.04812, 0.02323},  // median |error| 9.8%
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
//     3.0899 us (the reduction's launch)
//   + 0.11436 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.5859 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 3.0899;
constexpr double kSplitUsPerMB = 0.11436;
constexpr double kSplitUsPerRound = 0.5859;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 1},  // 1: 16.3, 2: 38.7, 4: 22.9, 8: 17.5, 16: 21.2
    {32, 4096, 4096, 8},  // 1: 24.9, 2: 39.1, 4: 23.3, 8: 17.1, 16: 21.7
    {64, 4096, 4096, 4},  // 1: 25.0, 2: 34.8, 4: 21.1, 8: 24.0, 16: 28.9
    {128, 4096, 4096, 2},  // 1: 39.6, 2: 35.7, 4: 37.2, 8: 39.2, 16: 43.3
    {32, 8192, 8192, 4},  // 1: 48.0, 2: 72.9, 4: 45.0, 8: 46.4, 16: 52.4
    {64, 8192, 8192, 2},  // 1: 79.8, 2: 66.8, 4: 70.4, 8: 74.5, 16: 85.8
    {256, 256, 8192, 16},  // 1: 22.3, 2: 62.9, 4: 34.6, 8: 21.7, 16: 17.1
    {512, 512, 8192, 4},  // 1: 45.9, 2: 63.3, 4: 35.5, 8: 37.5, 16: 40.3
    {1024, 1024, 1024, 1},  // 1: 17.9, 2: 24.9, 4: 29.2, 8: 34.8, 16: 39.1
    {2048, 2048, 2048, 1},  // 1: 118.0, 2: 129.7, 4: 138.7, 8: 157.1, 16: 202.5
    {4096, 4096, 4096, 1},  // 1: 902.9, 2: 945.3, 4: 994.1, 8: 1114.2, 16: 1279.2, -2: 1066.8, -4: 1076.7, -8: 1120.6, -16: 1166.9
    {1536, 1536, 1536, -4},  // 1: 68.3, 2: 66.4, 4: 64.7, 8: 77.6, 16: 88.2, -2: 61.4, -4: 57.0, -8: 58.0, -16: 64.7
    {1536, 1536, 4096, -4},  // 1: 168.0, 2: 154.4, 4: 143.4, 8: 154.8, 16: 176.8, -2: 149.4, -4: 136.5, -8: 136.7, -16: 139.2
    {2560, 2560, 2560, -8},  // 1: 285.5, 2: 271.8, 4: 268.3, 8: 291.6, 16: 365.2, -2: 257.2, -4: 239.9, -8: 233.2, -16: 241.1
    {1280, 1280, 2048, -4},  // 1: 61.9, 2: 65.9, 4: 65.9, 8: 71.2, 16: 82.4, -2: 66.7, -4: 61.2, -8: 62.1, -16: 66.0
    {5000, 5000, 1000, -8},  // 1: 394.1, 2: 441.4, 4: 532.2, 8: 740.4, 16: 1146.7, -2: 405.7, -4: 406.0, -8: 380.2, -16: 386.0
    {1536, 3072, 4096, -4},  // 1: 289.3, 2: 270.1, 4: 280.4, 8: 301.3, 16: 368.5, -2: 267.5, -4: 265.9, -8: 266.2, -16: 269.8
    {39, 432, 6224, 16},  // 1: 17.5, 2: 56.0, 4: 31.7, 8: 20.3, 16: 16.0
    {11, 1640, 2822, 1},  // 1: 9.8, 2: 29.1, 4: 18.4, 8: 13.2, 16: 12.3
    {11, 1486, 1136, 1},  // 1: 5.3, 2: 14.6, 4: 11.1, 8: 9.5, 16: 9.6
    {66, 326, 1317, 1},  // 1: 5.3, 2: 17.5, 4: 12.1, 8: 9.8, 16: 9.7
    {63, 4495, 1443, 2},  // 1: 25.9, 2: 18.8, 4: 20.2, 8: 21.0, 16: 22.3
    {24, 2252, 14173, 8},  // 1: 127.5, 2: 121.6, 4: 64.2, 8: 37.9, 16: 40.2
    {132, 1012, 15340, 16},  // 1: 84.7, 2: 131.3, 4: 69.1, 8: 65.1, 16: 55.2
    {10, 5016, 2286, 4},  // 1: 20.0, 2: 24.5, 4: 16.7, 8: 19.7, 16: 17.0
    {16, 385, 2409, 1},  // 1: 7.0, 2: 24.9, 4: 16.0, 8: 11.9, 16: 11.2
    {420, 479, 5136, 4},  // 1: 32.0, 2: 48.0, 4: 28.5, 8: 31.2, 16: 33.8
    {178, 931, 4676, 4},  // 1: 30.7, 2: 44.7, 4: 26.2, 8: 28.7, 16: 33.3
    {11, 315, 1813, 1},  // 1: 5.9, 2: 20.5, 4: 14.0, 8: 10.6, 16: 10.2
    {217, 1127, 2447, 4},  // 1: 21.1, 2: 26.5, 4: 18.2, 8: 21.5, 16: 23.8
    {137, 1231, 2351, 4},  // 1: 21.2, 2: 25.4, 4: 17.6, 8: 20.1, 16: 24.7
    {378, 2886, 2015, -8},  // 1: 66.3, 2: 55.5, 4: 52.0, 8: 52.1, 16: 68.9, -2: 55.3, -4: 47.9, -8: 45.7, -16: 47.3
    {130, 1580, 11590, 8},  // 1: 95.0, 2: 102.5, 4: 94.2, 8: 73.8, 16: 76.6
    {276, 694, 15508, 8},  // 1: 86.5, 2: 134.5, 4: 69.7, 8: 67.7, 16: 72.5
    {14, 1090, 8356, 16},  // 1: 27.3, 2: 73.5, 4: 39.7, 8: 24.3, 16: 18.6
    {17, 1394, 1142, 1},  // 1: 5.4, 2: 14.6, 4: 10.9, 8: 9.4, 16: 9.2
    {205, 3623, 5015, 4},  // 1: 99.8, 2: 83.6, 4: 82.9, 8: 85.3, 16: 89.1
    {560, 759, 7039, 8},  // 1: 71.7, 2: 64.5, 4: 61.5, 8: 61.3, 16: 61.8
    {143, 1910, 3628, 2},  // 1: 54.0, 2: 36.3, 4: 36.5, 8: 40.2, 16: 44.1
    {471, 6763, 3812, -2},  // 1: 219.9, 2: 226.4, 4: 215.0, 8: 236.1, 16: 279.8, -2: 206.3, -4: 252.6, -8: 252.9, -16: 256.9
    {201, 316, 7161, 8},  // 1: 42.8, 2: 65.6, 4: 35.5, 8: 22.4, 16: 25.1
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
