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
    {128, 128, 128, 5, 13, 7, 13, 6},  // sb 4.75 us, db 4.49 us, ms 4.55 us, ks 3.96 us
    {127, 193, 61, 5, 17, 7, 6, 6},  // sb 4.17 us, db 4.20 us, ms 4.27 us, ks 4.11 us
    {513, 257, 129, 5, 17, 13, 13, 6},  // sb 6.17 us, db 5.82 us, ms 5.96 us, ks 4.27 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.78 us, db 18.57 us, ms 18.04 us, ks 24.14 us
    {256, 1024, 128, 5, 15, 7, 13, 6},  // sb 5.00 us, db 4.63 us, ms 4.76 us, ks 4.18 us
    {1024, 128, 256, 5, 17, 7, 13, 6},  // sb 7.43 us, db 6.45 us, ms 6.50 us, ks 4.21 us
    {4096, 4096, 4096, 2, 0, 9, 0, 3},  // sb 967.42 us, db 906.93 us, ms 916.23 us, ks 1210.85 us
    {8192, 8192, 8192, 2, 0, 4, 0, 3},  // sb 7394.54 us, db 7196.11 us, ms 7226.13 us, ks 9858.91 us
    {256, 256, 256, 5, 15, 7, 13, 6},  // sb 7.41 us, db 6.42 us, ms 6.49 us, ks 4.18 us
    {512, 512, 512, 5, 16, 7, 13, 6},  // sb 12.50 us, db 10.20 us, ms 10.10 us, ks 5.68 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.07 us, db 14.51 us, ms 14.14 us, ks 14.66 us
    {1536, 1536, 1536, 2, 6, 7, 6, 6},  // sb 76.70 us, db 68.93 us, ms 69.09 us, ks 72.30 us
    {2048, 2048, 2048, 2, 3, 6, 3, 3},  // sb 129.46 us, db 117.88 us, ms 121.35 us, ks 161.41 us
    {3072, 3072, 3072, 2, 11, 7, 11, 11},  // sb 426.31 us, db 387.28 us, ms 402.62 us, ks 518.91 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3198.57 us, db 3066.33 us, ms 3076.57 us, ks 4079.98 us
    {64, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.81 us, db 63.47 us, ms 61.11 us, ks 24.96 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 128.43 us, db 123.53 us, ms 125.12 us, ks 202.91 us
    {2048, 8192, 2048, 2, 0, 9, 0, 3},  // sb 490.81 us, db 462.32 us, ms 465.90 us, ks 630.07 us
    {4096, 1024, 1024, 2, 3, 7, 3, 3},  // sb 67.41 us, db 62.15 us, ms 64.09 us, ks 89.46 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.56 us, db 128.89 us, ms 122.53 us, ks 152.49 us
    {512, 4096, 4096, 3, 18, 6, 18, 18},  // sb 136.55 us, db 120.63 us, ms 118.27 us, ks 155.17 us
    {512, 4096, 11008, 3, 18, 6, 18, 18},  // sb 349.38 us, db 318.75 us, ms 311.52 us, ks 400.92 us
    {1023, 1023, 1023, 3, 6, 7, 6, 6},  // sb 25.19 us, db 21.09 us, ms 20.84 us, ks 27.74 us
    {4095, 4095, 4095, 3, 0, 9, 0, 0},  // sb 1005.53 us, db 921.67 us, ms 921.06 us, ks 1344.13 us
    {16, 4096, 4096, 5, 19, 7, 6, 6},  // sb 97.31 us, db 70.38 us, ms 69.53 us, ks 15.22 us
    {32, 4096, 4096, 5, 15, 7, 13, 10},  // sb 97.90 us, db 63.53 us, ms 63.51 us, ks 18.42 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 96.01 us, db 64.41 us, ms 61.64 us, ks 40.93 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 196.54 us, db 128.98 us, ms 124.97 us, ks 48.36 us
    {1, 4096, 4096, 5, 19, 7, 6, 6},  // sb 96.79 us, db 70.32 us, ms 69.42 us, ks 12.31 us
    {8, 4096, 4096, 5, 19, 7, 6, 6},  // sb 97.02 us, db 70.29 us, ms 69.44 us, ks 13.91 us
    {16, 11008, 4096, 5, 16, 7, 6, 6},  // sb 100.10 us, db 71.31 us, ms 70.02 us, ks 30.76 us
    {16, 4096, 11008, 5, 14, 7, 6, 7},  // sb 262.17 us, db 183.96 us, ms 180.70 us, ks 37.50 us
    {16, 8192, 8192, 5, 17, 7, 13, 6},  // sb 194.84 us, db 140.12 us, ms 136.44 us, ks 39.66 us
    {4, 1024, 1024, 5, 19, 7, 6, 6},  // sb 23.30 us, db 19.61 us, ms 19.62 us, ks 4.42 us
    {16, 32000, 4096, 3, 10, 13, 13, 10},  // sb 154.57 us, db 108.74 us, ms 86.80 us, ks 96.31 us
    {1024, 8192, 8192, 2, 2, 18, 2, 3},  // sb 1016.33 us, db 908.71 us, ms 922.85 us, ks 1203.24 us
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
// squares on relative error, all kept >= 0, to the 100 shapes measured for this file
// (the table's 36 and 64 seeded shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, b_us, g_us, h_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.2203, 0.0000, 4.03797, 0.38738},  // median |error| 1.7%
    {1, 1, 9.9725, 0.0000, 7.74228, 0.53882},  // median |error| 1.1%
    {1, 2, 5.5399, 0.0000, 2.25173, 0.00000},  // median |error| 3.9%
    {1, 3, 3.7399, 0.0000, 1.25406, 0.00000},  // median |error| 8.4%
    {1, 4, 3.8334, 0.0000, 2.27332, 0.00000},  // median |error| 4.1%
    {1, 5, 3.3143, 0.0000, 1.24246, 0.00000},  // median |error| 11.0%
    {1, 6, 3.0096, 0.0000, 0.67738, 0.00000},  // median |error| 18.2%
    {1, 7, 2.9674, 0.0000, 1.23808, 0.00000},  // median |error| 11.7%
    {1, 8, 6.6011, 0.0000, 7.62774, 0.41470},  // median |error| 1.6%
    {1, 9, 4.2615, 0.0000, 4.12814, 0.00000},  // median |error| 3.0%
    {1, 10, 3.0595, 0.0000, 0.71059, 0.00000},  // median |error| 22.1%
    {1, 11, 6.3532, 0.0000, 2.45476, 0.30036},  // median |error| 2.9%
    {1, 12, 6.7550, 0.0000, 4.56379, 0.42918},  // median |error| 2.0%
    {1, 13, 4.6025, 0.0000, 0.19635, 0.00000},  // median |error| 32.1%
    {1, 18, 2.8593, 0.0000, 1.23321, 0.00000},  // median |error| 10.0%
    {2, 0, 10.3511, 0.0000, 3.44659, 0.12944},  // median |error| 0.9%
    {2, 1, 10.6552, 0.0000, 6.90450, 0.24646},  // median |error| 0.9%
    {2, 2, 6.4776, 0.0000, 1.74350, 0.06060},  // median |error| 1.1%
    {2, 3, 4.4068, 0.0000, 0.88567, 0.07653},  // median |error| 2.1%
    {2, 4, 4.6366, 0.0000, 1.74895, 0.06769},  // median |error| 1.4%
    {2, 5, 4.0199, 0.0000, 0.92256, 0.01512},  // median |error| 1.8%
    {2, 6, 3.1554, 0.0000, 0.51243, 0.00000},  // median |error| 3.5%
    {2, 7, 3.2257, 0.0000, 1.05191, 0.00000},  // median |error| 3.4%
    {2, 8, 7.2823, 0.0000, 7.01500, 0.29217},  // median |error| 0.6%
    {2, 9, 5.2487, 0.0000, 3.45814, 0.15810},  // median |error| 0.6%
    {2, 10, 3.1308, 0.0000, 0.55388, 0.00000},  // median |error| 3.6%
    {2, 11, 7.2206, 0.0000, 1.97200, 0.06581},  // median |error| 0.6%
    {2, 12, 7.7532, 0.0000, 3.89479, 0.15445},  // median |error| 0.7%
    {2, 13, 4.4856, 0.0000, 0.17813, 0.00000},  // median |error| 24.4%
    {2, 18, 3.3221, 0.0000, 0.94747, 0.02045},  // median |error| 2.2%
    {3, 0, 10.4295, 0.0000, 3.50890, 0.17744},  // median |error| 1.7%
    {3, 1, 10.9631, 0.0000, 7.01996, 0.42503},  // median |error| 1.9%
    {3, 2, 6.9414, 0.0000, 1.77249, 0.08127},  // median |error| 1.5%
    {3, 3, 4.5584, 0.0000, 0.90894, 0.02226},  // median |error| 2.1%
    {3, 4, 4.6774, 0.0000, 1.78215, 0.12054},  // median |error| 1.5%
    {3, 5, 4.2530, 0.0000, 0.92014, 0.06539},  // median |error| 1.6%
    {3, 6, 3.2373, 0.0000, 0.50890, 0.00000},  // median |error| 2.7%
    {3, 7, 3.3037, 0.0000, 1.04689, 0.06374},  // median |error| 2.8%
    {3, 8, 7.7447, 0.0000, 7.03791, 0.27933},  // median |error| 0.7%
    {3, 9, 5.3256, 0.0000, 3.48853, 0.18562},  // median |error| 1.0%
    {3, 10, 3.1964, 0.0000, 0.54370, 0.00000},  // median |error| 4.1%
    {3, 11, 7.3337, 0.0000, 2.01058, 0.09299},  // median |error| 2.2%
    {3, 12, 7.8934, 0.0000, 3.97296, 0.25066},  // median |error| 2.6%
    {3, 18, 3.4710, 0.0000, 0.94438, 0.03880},  // median |error| 1.6%
    {5, 13, 2.9086, 0.9064, 0.16087, 0.00000},  // median |error| 6.2%
    {5, 14, 3.0387, 0.5361, 0.05066, 0.02478},  // median |error| 10.6%
    {5, 15, 2.9305, 0.5093, 0.10016, 0.00000},  // median |error| 11.5%
    {5, 16, 1.7820, 1.7977, 0.16374, 0.01693},  // median |error| 6.8%
    {5, 17, 3.4118, 0.1003, 0.10470, 0.00000},  // median |error| 10.8%
    {5, 19, 3.3759, 0.0000, 0.05938, 0.02055},  // median |error| 11.5%
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
//     3.2197 us (the reduction's launch)
//   + 0.13783 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.2955 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 3.2197;
constexpr double kSplitUsPerMB = 0.13783;
constexpr double kSplitUsPerRound = 0.2955;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 1},  // 1: 15.3, 2: 38.8, 4: 22.9, 8: 17.4, 16: 21.4
    {32, 4096, 4096, 1},  // 1: 17.1, 2: 39.3, 4: 23.4, 8: 17.2, 16: 21.7
    {64, 4096, 4096, 4},  // 1: 24.9, 2: 34.9, 4: 21.6, 8: 23.1, 16: 26.8
    {128, 4096, 4096, 2},  // 1: 40.4, 2: 35.9, 4: 36.9, 8: 39.6, 16: 43.3
    {32, 8192, 8192, 4},  // 1: 48.5, 2: 73.4, 4: 45.1, 8: 46.8, 16: 52.6
    {64, 8192, 8192, 2},  // 1: 81.1, 2: 68.7, 4: 74.5, 8: 77.3, 16: 82.1
    {256, 256, 8192, 16},  // 1: 24.1, 2: 63.2, 4: 34.8, 8: 21.8, 16: 17.3
    {512, 512, 8192, 4},  // 1: 46.1, 2: 63.9, 4: 35.9, 8: 37.2, 16: 40.4
    {1024, 1024, 1024, 1},  // 1: 18.0, 2: 24.5, 4: 28.0, 8: 32.8, 16: 39.9
    {2048, 2048, 2048, 1},  // 1: 117.7, 2: 130.2, 4: 141.2, 8: 159.2, 16: 208.2
    {4096, 4096, 4096, 1},  // 1: 912.6, 2: 955.0, 4: 1005.1, 8: 1131.5, 16: 1295.1, -2: 1078.1, -4: 1093.7, -8: 1125.9, -16: 1179.4
    {1536, 1536, 1536, -4},  // 1: 68.7, 2: 66.9, 4: 65.1, 8: 77.3, 16: 89.1, -2: 62.0, -4: 57.8, -8: 58.2, -16: 64.0
    {1536, 1536, 4096, -8},  // 1: 172.0, 2: 155.4, 4: 143.9, 8: 155.2, 16: 184.3, -2: 150.5, -4: 139.5, -8: 137.5, -16: 140.4
    {2560, 2560, 2560, -8},  // 1: 258.3, 2: 260.8, 4: 272.0, 8: 305.8, 16: 365.5, -2: 245.8, -4: 241.7, -8: 235.5, -16: 241.6
    {1280, 1280, 2048, -4},  // 1: 62.0, 2: 66.2, 4: 66.6, 8: 71.7, 16: 82.8, -2: 67.1, -4: 61.8, -8: 62.9, -16: 66.9
    {5000, 5000, 1000, -8},  // 1: 393.3, 2: 447.6, 4: 528.8, 8: 762.9, 16: 1149.9, -2: 389.0, -4: 390.2, -8: 379.6, -16: 385.3
    {1536, 3072, 4096, -8},  // 1: 291.1, 2: 269.9, 4: 280.3, 8: 320.5, 16: 372.1, -2: 271.6, -4: 267.8, -8: 265.9, -16: 269.8
    {39, 432, 6224, 1},  // 1: 13.9, 2: 56.1, 4: 32.0, 8: 20.5, 16: 16.4
    {11, 1640, 2822, 1},  // 1: 7.5, 2: 29.1, 4: 18.4, 8: 13.1, 16: 12.5
    {11, 1486, 1136, 1},  // 1: 5.3, 2: 14.5, 4: 10.9, 8: 9.6, 16: 9.6
    {66, 326, 1317, 1},  // 1: 5.4, 2: 17.2, 4: 12.0, 8: 9.9, 16: 9.8
    {63, 4495, 1443, 1},  // 1: 17.6, 2: 18.8, 4: 19.3, 8: 19.0, 16: 19.8
    {24, 2252, 14173, 8},  // 1: 55.3, 2: 120.9, 4: 64.1, 8: 38.0, 16: 40.5
    {132, 1012, 15340, 16},  // 1: 84.7, 2: 131.3, 4: 69.2, 8: 65.5, 16: 56.1
    {10, 5016, 2286, 1},  // 1: 10.6, 2: 24.4, 4: 16.9, 8: 19.8, 16: 17.1
    {16, 385, 2409, 1},  // 1: 7.0, 2: 25.0, 4: 15.9, 8: 11.8, 16: 11.0
    {420, 479, 5136, 4},  // 1: 32.0, 2: 48.2, 4: 28.5, 8: 30.9, 16: 33.3
    {178, 931, 4676, 4},  // 1: 29.8, 2: 44.3, 4: 26.3, 8: 28.4, 16: 30.2
    {11, 315, 1813, 1},  // 1: 5.9, 2: 20.6, 4: 13.9, 8: 10.6, 16: 10.2
    {217, 1127, 2447, 1},  // 1: 18.4, 2: 26.7, 4: 18.5, 8: 21.4, 16: 22.8
    {137, 1231, 2351, 1},  // 1: 17.6, 2: 25.4, 4: 17.6, 8: 19.8, 16: 22.4
    {378, 2886, 2015, -8},  // 1: 56.3, 2: 57.2, 4: 52.4, 8: 56.9, 16: 64.9, -2: 52.3, -4: 47.0, -8: 44.5, -16: 45.5
    {130, 1580, 11590, 1},  // 1: 65.8, 2: 101.0, 4: 94.2, 8: 74.3, 16: 71.5
    {276, 694, 15508, 8},  // 1: 88.3, 2: 132.5, 4: 70.4, 8: 68.1, 16: 70.7
    {14, 1090, 8356, 16},  // 1: 25.0, 2: 73.9, 4: 40.1, 8: 24.5, 16: 18.7
    {17, 1394, 1142, 1},  // 1: 5.4, 2: 14.5, 4: 10.9, 8: 9.5, 16: 9.3
    {205, 3623, 5015, 4},  // 1: 87.1, 2: 83.5, 4: 83.3, 8: 84.6, 16: 92.8
    {560, 759, 7039, 4},  // 1: 72.8, 2: 64.8, 4: 61.8, 8: 61.8, 16: 67.4
    {143, 1910, 3628, 2},  // 1: 41.7, 2: 35.8, 4: 35.9, 8: 40.3, 16: 38.2
    {471, 6763, 3812, -8},  // 1: 222.6, 2: 217.9, 4: 216.7, 8: 243.6, 16: 302.4, -2: 208.7, -4: 206.6, -8: 203.0, -16: 205.2
    {201, 316, 7161, 8},  // 1: 29.7, 2: 64.5, 4: 35.7, 8: 22.6, 16: 24.6
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
