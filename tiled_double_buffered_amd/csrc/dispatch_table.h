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
    {128, 128, 128, 5, 15, 7, 6, 6},  // sb 4.79 us, db 4.49 us, ms 4.39 us, ks 4.09 us
    {127, 193, 61, 2, 7, 7, 7, 7},  // sb 4.21 us, db 4.17 us, ms 4.20 us, ks 4.16 us
    {513, 257, 129, 5, 16, 13, 13, 6},  // sb 6.16 us, db 5.78 us, ms 5.94 us, ks 4.22 us
    {1024, 1024, 1024, 3, 6, 7, 6, 6},  // sb 23.78 us, db 18.59 us, ms 17.74 us, ks 24.07 us
    {256, 1024, 128, 5, 13, 7, 13, 6},  // sb 4.99 us, db 4.61 us, ms 4.62 us, ks 4.21 us
    {1024, 128, 256, 5, 15, 7, 13, 6},  // sb 7.41 us, db 6.42 us, ms 6.30 us, ks 4.21 us
    {4096, 4096, 4096, 2, 0, 18, 0, 3},  // sb 951.74 us, db 906.42 us, ms 914.13 us, ks 1180.96 us
    {8192, 8192, 8192, 2, 0, 4, 0, 3},  // sb 7351.59 us, db 7167.92 us, ms 7190.38 us, ks 9420.21 us
    {256, 256, 256, 5, 15, 7, 13, 6},  // sb 7.38 us, db 6.38 us, ms 6.27 us, ks 4.17 us
    {512, 512, 512, 5, 16, 7, 13, 6},  // sb 12.54 us, db 10.21 us, ms 9.88 us, ks 5.66 us
    {768, 768, 768, 3, 6, 7, 6, 6},  // sb 18.05 us, db 14.53 us, ms 13.72 us, ks 14.66 us
    {1536, 1536, 1536, 3, 6, 7, 6, 6},  // sb 76.38 us, db 68.24 us, ms 68.08 us, ks 70.19 us
    {2048, 2048, 2048, 2, 3, 6, 3, 18},  // sb 126.42 us, db 117.49 us, ms 119.26 us, ks 156.18 us
    {3072, 3072, 3072, 2, 11, 7, 11, 6},  // sb 416.03 us, db 386.68 us, ms 395.58 us, ks 507.44 us
    {6144, 6144, 6144, 2, 11, 4, 11, 3},  // sb 3169.38 us, db 3038.76 us, ms 3055.43 us, ks 3924.60 us
    {64, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.60 us, db 63.48 us, ms 60.31 us, ks 24.94 us
    {4096, 4096, 512, 2, 2, 9, 2, 3},  // sb 128.21 us, db 122.96 us, ms 124.63 us, ks 202.97 us
    {2048, 8192, 2048, 2, 0, 18, 0, 8},  // sb 481.16 us, db 460.73 us, ms 466.15 us, ks 614.07 us
    {4096, 1024, 1024, 2, 3, 7, 3, 18},  // sb 66.53 us, db 61.72 us, ms 62.93 us, ks 88.36 us
    {1024, 1024, 8192, 3, 6, 7, 6, 6},  // sb 190.87 us, db 128.35 us, ms 119.72 us, ks 147.46 us
    {512, 4096, 4096, 3, 18, 6, 18, 18},  // sb 135.59 us, db 118.72 us, ms 116.87 us, ks 149.69 us
    {512, 4096, 11008, 3, 18, 6, 18, 18},  // sb 342.88 us, db 310.52 us, ms 305.49 us, ks 387.60 us
    {1023, 1023, 1023, 2, 6, 7, 6, 6},  // sb 25.18 us, db 20.66 us, ms 20.71 us, ks 27.17 us
    {4095, 4095, 4095, 3, 0, 9, 0, 0},  // sb 1003.92 us, db 920.15 us, ms 919.77 us, ks 1308.88 us
    {16, 4096, 4096, 5, 19, 7, 6, 6},  // sb 97.44 us, db 70.47 us, ms 67.71 us, ks 15.19 us
    {32, 4096, 4096, 5, 15, 7, 13, 10},  // sb 97.54 us, db 63.41 us, ms 62.44 us, ks 18.45 us
    {128, 4096, 4096, 5, 13, 7, 13, 6},  // sb 95.88 us, db 64.23 us, ms 60.75 us, ks 40.05 us
    {32, 8192, 8192, 5, 13, 7, 13, 10},  // sb 196.65 us, db 128.87 us, ms 122.64 us, ks 48.21 us
    {128, 11008, 4096, 5, 13, 6, 18, 18},  // sb 127.41 us, db 117.33 us, ms 115.60 us, ks 109.81 us
    {128, 4096, 11008, 5, 13, 7, 13, 6},  // sb 257.70 us, db 167.76 us, ms 158.42 us, ks 101.42 us
    {1, 4096, 4096, 5, 19, 7, 6, 6},  // sb 96.66 us, db 70.27 us, ms 67.56 us, ks 12.22 us
    {8, 4096, 4096, 5, 19, 7, 6, 6},  // sb 97.24 us, db 70.24 us, ms 67.39 us, ks 13.90 us
    {16, 11008, 4096, 5, 16, 7, 13, 6},  // sb 100.02 us, db 70.74 us, ms 67.71 us, ks 30.87 us
    {16, 4096, 11008, 5, 14, 7, 6, 6},  // sb 262.03 us, db 184.03 us, ms 176.39 us, ks 37.50 us
    {16, 8192, 8192, 5, 17, 7, 13, 6},  // sb 195.27 us, db 140.34 us, ms 132.41 us, ks 39.66 us
    {4, 1024, 1024, 5, 19, 7, 6, 6},  // sb 23.36 us, db 19.66 us, ms 19.20 us, ks 4.39 us
    {16, 32000, 4096, 3, 10, 13, 13, 10},  // sb 154.81 us, db 108.84 us, ms 92.27 us, ks 96.62 us
    {1024, 8192, 8192, 2, 2, 7, 2, 18},  // sb 998.21 us, db 906.38 us, ms 912.22 us, ks 1173.89 us
    {1, 11008, 4096, 5, 14, 7, 13, 6},  // sb 99.87 us, db 70.62 us, ms 67.90 us, ks 30.24 us
    {1, 4096, 11008, 5, 19, 7, 6, 6},  // sb 255.99 us, db 183.83 us, ms 176.11 us, ks 27.65 us
    {1, 8192, 8192, 5, 17, 7, 13, 6},  // sb 192.57 us, db 138.39 us, ms 132.17 us, ks 39.47 us
    {1, 32000, 4096, 3, 10, 13, 13, 10},  // sb 154.25 us, db 107.58 us, ms 92.96 us, ks 94.13 us
    {4, 4096, 4096, 5, 19, 7, 6, 6},  // sb 97.02 us, db 70.26 us, ms 67.45 us, ks 12.74 us
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
// squares on relative error, all kept >= 0, to the 107 shapes measured for this file
// (the table's 43 and 64 seeded shapes outside it).
struct ModelRow {
  int variant, cfg;
  double a_us, b_us, g_us, h_us;
};

static const ModelRow kModel[] = {
    {1, 0, 9.2158, 0.0000, 4.03658, 0.39670},  // median |error| 1.7%
    {1, 1, 9.9696, 0.0000, 7.73859, 0.54805},  // median |error| 1.1%
    {1, 2, 5.5172, 0.0000, 2.25607, 0.00000},  // median |error| 3.8%
    {1, 3, 3.6759, 0.0000, 1.26270, 0.00000},  // median |error| 7.2%
    {1, 4, 3.8023, 0.0000, 2.28078, 0.00000},  // median |error| 3.7%
    {1, 5, 3.2466, 0.0000, 1.25129, 0.00000},  // median |error| 10.8%
    {1, 6, 2.9643, 0.0000, 0.67840, 0.00000},  // median |error| 19.4%
    {1, 7, 2.9295, 0.0000, 1.24135, 0.00000},  // median |error| 13.1%
    {1, 8, 6.5773, 0.0000, 7.63221, 0.40494},  // median |error| 1.5%
    {1, 9, 4.2517, 0.0000, 4.12865, 0.00000},  // median |error| 3.1%
    {1, 10, 3.0176, 0.0000, 0.70893, 0.00000},  // median |error| 24.6%
    {1, 11, 6.3457, 0.0000, 2.45524, 0.30305},  // median |error| 2.5%
    {1, 12, 6.7563, 0.0000, 4.56054, 0.43298},  // median |error| 1.6%
    {1, 13, 4.5144, 0.0000, 0.19718, 0.00000},  // median |error| 35.3%
    {1, 18, 2.8351, 0.0000, 1.24059, 0.00000},  // median |error| 10.5%
    {2, 0, 10.3266, 0.0000, 3.44961, 0.11529},  // median |error| 0.7%
    {2, 1, 10.6272, 0.0000, 6.90987, 0.21794},  // median |error| 0.7%
    {2, 2, 6.4632, 0.0000, 1.74671, 0.05148},  // median |error| 1.0%
    {2, 3, 4.3894, 0.0000, 0.88486, 0.07767},  // median |error| 2.1%
    {2, 4, 4.6245, 0.0000, 1.75071, 0.05992},  // median |error| 1.2%
    {2, 5, 3.9870, 0.0000, 0.92607, 0.00296},  // median |error| 1.9%
    {2, 6, 3.1224, 0.0000, 0.50790, 0.00000},  // median |error| 3.7%
    {2, 7, 3.1530, 0.0000, 1.04853, 0.00000},  // median |error| 3.5%
    {2, 8, 7.2576, 0.0000, 7.02091, 0.25303},  // median |error| 0.5%
    {2, 9, 5.2373, 0.0000, 3.45889, 0.14232},  // median |error| 0.5%
    {2, 10, 3.1369, 0.0000, 0.54827, 0.00000},  // median |error| 4.2%
    {2, 11, 7.2089, 0.0000, 1.97277, 0.05849},  // median |error| 0.5%
    {2, 12, 7.7493, 0.0000, 3.89577, 0.13389},  // median |error| 0.5%
    {2, 13, 4.4367, 0.0000, 0.17631, 0.00000},  // median |error| 27.0%
    {2, 18, 3.3110, 0.0000, 0.94837, 0.00789},  // median |error| 2.3%
    {3, 0, 10.3561, 0.0000, 3.52032, 0.15600},  // median |error| 1.8%
    {3, 1, 10.8666, 0.0000, 7.04727, 0.38331},  // median |error| 2.0%
    {3, 2, 6.9024, 0.0000, 1.78025, 0.07063},  // median |error| 1.6%
    {3, 3, 4.5288, 0.0000, 0.91101, 0.01843},  // median |error| 2.3%
    {3, 4, 4.6383, 0.0000, 1.79127, 0.10820},  // median |error| 1.6%
    {3, 5, 4.2181, 0.0000, 0.92197, 0.06016},  // median |error| 1.5%
    {3, 6, 3.1937, 0.0000, 0.49881, 0.00000},  // median |error| 4.0%
    {3, 7, 3.2232, 0.0000, 1.03592, 0.06087},  // median |error| 3.6%
    {3, 8, 7.7219, 0.0000, 7.04374, 0.24121},  // median |error| 0.6%
    {3, 9, 5.2917, 0.0000, 3.49651, 0.16310},  // median |error| 1.0%
    {3, 10, 3.1687, 0.0000, 0.53028, 0.00000},  // median |error| 5.9%
    {3, 11, 7.2833, 0.0000, 2.01835, 0.08208},  // median |error| 2.4%
    {3, 12, 7.8262, 0.0000, 3.99216, 0.22613},  // median |error| 2.9%
    {3, 18, 3.4730, 0.0000, 0.94459, 0.02560},  // median |error| 1.8%
    {5, 13, 2.8632, 0.9138, 0.15826, 0.00000},  // median |error| 7.1%
    {5, 14, 2.9625, 0.5305, 0.05039, 0.02583},  // median |error| 10.4%
    {5, 15, 2.8759, 0.5092, 0.10059, 0.00000},  // median |error| 11.7%
    {5, 16, 1.6633, 1.8113, 0.16249, 0.01855},  // median |error| 7.0%
    {5, 17, 3.3667, 0.0914, 0.10552, 0.00000},  // median |error| 10.6%
    {5, 19, 3.3011, 0.0000, 0.06077, 0.01946},  // median |error| 11.1%
};
constexpr int kModelRows = (int)(sizeof(kModel) / sizeof(kModel[0]));
constexpr int kVariantMS = 3;
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
    // with a K tail the multi-stage kernel runs the double-buffered loop in its larger LDS
    // allocation, never ahead of the double-buffered kernel: not a candidate then
    if (variant == 0 && kModel[i].variant == kVariantMS && K % kConfigs[kModel[i].cfg].bk != 0)
      continue;
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
//     3.3486 us (the reduction's launch)
//   + 0.13897 us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + 0.2572 us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the 41 shapes of the split study below.
constexpr double kSplitFixedUs = 3.3486;
constexpr double kSplitUsPerMB = 0.13897;
constexpr double kSplitUsPerRound = 0.2572;
constexpr int kSplitChoices[] = {1, 2, 4, 8, 16};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {
  int64_t m, n, k;
  int splits;
};

static const SplitRow kSplitK[] = {
    {16, 4096, 4096, 1},  // 1: 14.9, 2: 37.9, 4: 22.5, 8: 17.6, 16: 21.2
    {32, 4096, 4096, 1},  // 1: 17.0, 2: 38.3, 4: 22.9, 8: 17.2, 16: 21.3
    {64, 4096, 4096, 4},  // 1: 24.6, 2: 34.5, 4: 21.6, 8: 23.1, 16: 26.8
    {128, 4096, 4096, 2},  // 1: 40.1, 2: 35.5, 4: 36.7, 8: 39.3, 16: 43.4
    {32, 8192, 8192, 4},  // 1: 48.2, 2: 70.6, 4: 45.0, 8: 46.2, 16: 52.7
    {64, 8192, 8192, 2},  // 1: 80.4, 2: 67.6, 4: 73.7, 8: 75.8, 16: 81.7
    {256, 256, 8192, 16},  // 1: 24.1, 2: 62.4, 4: 34.5, 8: 21.8, 16: 16.9
    {512, 512, 8192, 4},  // 1: 45.8, 2: 63.1, 4: 35.3, 8: 37.0, 16: 40.3
    {1024, 1024, 1024, 1},  // 1: 17.7, 2: 24.4, 4: 28.0, 8: 32.7, 16: 39.8
    {2048, 2048, 2048, 1},  // 1: 117.5, 2: 129.2, 4: 140.3, 8: 158.7, 16: 207.1
    {4096, 4096, 4096, 1},  // 1: 903.5, 2: 944.8, 4: 996.8, 8: 1128.4, 16: 1291.0, -2: 1071.4, -4: 1085.1, -8: 1120.3, -16: 1172.8
    {1536, 1536, 1536, -4},  // 1: 68.2, 2: 65.4, 4: 64.7, 8: 77.0, 16: 89.2, -2: 61.4, -4: 57.5, -8: 58.0, -16: 63.6
    {1536, 1536, 4096, -8},  // 1: 171.6, 2: 153.1, 4: 142.6, 8: 154.6, 16: 184.0, -2: 148.8, -4: 137.5, -8: 136.8, -16: 139.5
    {2560, 2560, 2560, -8},  // 1: 255.0, 2: 257.6, 4: 270.5, 8: 305.2, 16: 365.2, -2: 243.4, -4: 240.1, -8: 234.1, -16: 239.9
    {1280, 1280, 2048, -4},  // 1: 61.6, 2: 65.7, 4: 64.2, 8: 69.3, 16: 82.4, -2: 65.9, -4: 60.8, -8: 62.3, -16: 64.3
    {5000, 5000, 1000, -8},  // 1: 390.9, 2: 444.7, 4: 525.0, 8: 760.5, 16: 1147.7, -2: 383.7, -4: 388.9, -8: 379.2, -16: 383.2
    {1536, 3072, 4096, -8},  // 1: 288.1, 2: 269.0, 4: 279.6, 8: 318.9, 16: 370.6, -2: 269.1, -4: 266.0, -8: 264.2, -16: 268.0
    {39, 432, 6224, 1},  // 1: 13.9, 2: 56.0, 4: 31.1, 8: 20.3, 16: 16.2
    {11, 1640, 2822, 1},  // 1: 7.5, 2: 28.5, 4: 18.1, 8: 13.2, 16: 12.3
    {11, 1486, 1136, 1},  // 1: 5.4, 2: 14.6, 4: 11.0, 8: 9.6, 16: 9.6
    {66, 326, 1317, 1},  // 1: 5.4, 2: 16.5, 4: 12.2, 8: 9.9, 16: 9.9
    {63, 4495, 1443, 1},  // 1: 17.7, 2: 18.4, 4: 19.3, 8: 21.0, 16: 19.9
    {24, 2252, 14173, 8},  // 1: 55.1, 2: 120.6, 4: 62.4, 8: 36.8, 16: 41.0
    {132, 1012, 15340, 16},  // 1: 84.8, 2: 130.8, 4: 69.0, 8: 65.1, 16: 55.3
    {10, 5016, 2286, 1},  // 1: 10.7, 2: 24.4, 4: 16.8, 8: 19.6, 16: 17.0
    {16, 385, 2409, 1},  // 1: 7.0, 2: 25.0, 4: 15.9, 8: 11.7, 16: 11.0
    {420, 479, 5136, 4},  // 1: 32.0, 2: 47.2, 4: 27.8, 8: 30.9, 16: 33.2
    {178, 931, 4676, 4},  // 1: 29.8, 2: 44.1, 4: 25.7, 8: 28.4, 16: 30.0
    {11, 315, 1813, 1},  // 1: 6.0, 2: 20.2, 4: 13.9, 8: 10.8, 16: 10.5
    {217, 1127, 2447, 4},  // 1: 18.3, 2: 26.1, 4: 18.1, 8: 21.3, 16: 22.8
    {137, 1231, 2351, 1},  // 1: 17.6, 2: 24.9, 4: 17.6, 8: 20.0, 16: 22.1
    {378, 2886, 2015, -8},  // 1: 56.1, 2: 55.6, 4: 51.3, 8: 55.5, 16: 67.5, -2: 51.4, -4: 46.3, -8: 44.0, -16: 45.2
    {130, 1580, 11590, 1},  // 1: 65.5, 2: 100.7, 4: 93.9, 8: 73.1, 16: 69.3
    {276, 694, 15508, 8},  // 1: 87.7, 2: 132.0, 4: 69.0, 8: 67.5, 16: 70.2
    {14, 1090, 8356, 16},  // 1: 25.0, 2: 73.3, 4: 39.1, 8: 23.9, 16: 18.1
    {17, 1394, 1142, 1},  // 1: 5.4, 2: 14.6, 4: 10.8, 8: 9.4, 16: 9.1
    {205, 3623, 5015, 4},  // 1: 86.8, 2: 83.6, 4: 83.0, 8: 86.6, 16: 90.8
    {560, 759, 7039, 4},  // 1: 72.3, 2: 64.4, 4: 61.4, 8: 61.6, 16: 63.9
    {143, 1910, 3628, 8},  // 1: 41.7, 2: 35.3, 4: 35.9, 8: 32.5, 16: 37.4
    {471, 6763, 3812, -8},  // 1: 221.5, 2: 216.1, 4: 215.4, 8: 242.6, 16: 301.6, -2: 208.0, -4: 206.1, -8: 202.2, -16: 204.7
    {201, 316, 7161, 8},  // 1: 29.6, 2: 64.5, 4: 35.5, 8: 22.1, 16: 24.5
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
