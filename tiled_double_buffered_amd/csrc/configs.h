// The tile configurations of gemmf32 and the host-side record of each configuration's
// kernels.  Every configuration's kernels are compiled in a translation unit of their own
// (cfg_kernels.hip, built once per configuration id), which exports cfg_entry_<id>().
#pragma once

#include "gemm_common.h"
#include "kernels_ks16.h"

namespace gemmf32 {

// Configuration ids are part of the ABI (gemm_f32_ex, gemm_f32_config_info).
template <int ID>
struct CfgById;
template <> struct CfgById<0> { using type = TileCfg<256, 256, 16, 2, 2>; };   // wave 128x128 (16 blocks)
template <> struct CfgById<1> { using type = TileCfg<256, 256, 32, 2, 2>; };   // wave 128x128, deeper K tile
template <> struct CfgById<2> { using type = TileCfg<256, 128, 16, 2, 2>; };   // wave 128x64
template <> struct CfgById<3> { using type = TileCfg<128, 128, 16, 2, 2>; };   // wave 64x64
template <> struct CfgById<4> { using type = TileCfg<128, 128, 32, 2, 2>; };   // wave 64x64, deeper K tile
template <> struct CfgById<5> { using type = TileCfg<128, 64, 32, 2, 2>; };    // wave 64x32
template <> struct CfgById<6> { using type = TileCfg<64, 64, 32, 2, 2>; };     // wave 32x32
template <> struct CfgById<7> { using type = TileCfg<64, 64, 64, 2, 2>; };     // wave 32x32, deeper K tile
template <> struct CfgById<8> { using type = TileCfg<256, 256, 32, 2, 4>; };   // 8 waves of 128x64: two per SIMD
template <> struct CfgById<9> { using type = TileCfg<128, 256, 32, 2, 4>; };   // 8 waves of 64x64
template <> struct CfgById<10> { using type = TileCfg<32, 128, 32, 1, 4>; };   // 4 waves of 32x32 side by side: skinny M
template <> struct CfgById<11> { using type = TileCfg<192, 192, 16, 2, 2>; };  // wave 96x96: 16x16 tiles for 3072-wide C
template <> struct CfgById<12> { using type = TileCfg<192, 192, 32, 2, 2>; };  // wave 96x96, deeper K tile
template <> struct CfgById<13> { using type = TileCfg<32, 32, 32, 1, 1>; };    // one wave: few rows, long K (K-split kernel)
template <> struct CfgById<14> { using type = Ks16Cfg<16, 2>; };               // 16 x 16 tile, 16 waves over K in 32-deep groups: decode rows (K-split only)
template <> struct CfgById<15> { using type = Ks16Cfg<8, 2, false, 2>; };      // 16 x 32 tile, 8 waves over K: 128-byte rows of B
template <> struct CfgById<16> { using type = Ks16Cfg<8, 2, false, 4>; };      // 16 x 64 tile, 8 waves over K: wide layers
template <> struct CfgById<17> { using type = Ks16Cfg<4, 2, false, 2>; };      // 16 x 32 tile, 4 waves over K: several workgroups per CU
template <> struct CfgById<18> { using type = TileCfg<64, 128, 32, 2, 4>; };   // 8 waves of 32x32, two per SIMD: one round of tiles at a few hundred rows
template <> struct CfgById<19> { using type = Ks16Cfg<4, 2, true>; };         // 16 x 16 tile, 4 waves taking alternate K groups: the workgroup reads B in one front (few rows, 4096-wide layers)
constexpr int kNumConfigs = 20;

typedef void (*KernelFn)(int, int, int, const float*, int64_t, const float*, int64_t, float*,
                         int64_t, int, SplitArgs);

// ms: the multi-stage kernel, where the configuration has one (its swizzle needs tiles
// of B at least 64 wide; stages 0 otherwise); ks: the K-split kernel and its wave groups,
// where it has one (groups 1 otherwise).  The 16-row configurations have only a K-split
// kernel (sb, db and sb3 null, no LDS slots).
struct CfgEntry {
  int bm, bn, bk, nt;
  int lds_sb, lds_db;
  int ms_stages, lds_ms;
  KernelFn sb, db, ms, sb3;
  KernelFn ks;
  int ks_groups;
};

#define GEMMF32_CFG_ENTRY_DECL(ID) CfgEntry cfg_entry_##ID();
GEMMF32_CFG_ENTRY_DECL(0) GEMMF32_CFG_ENTRY_DECL(1) GEMMF32_CFG_ENTRY_DECL(2)
GEMMF32_CFG_ENTRY_DECL(3) GEMMF32_CFG_ENTRY_DECL(4) GEMMF32_CFG_ENTRY_DECL(5)
GEMMF32_CFG_ENTRY_DECL(6) GEMMF32_CFG_ENTRY_DECL(7) GEMMF32_CFG_ENTRY_DECL(8)
GEMMF32_CFG_ENTRY_DECL(9) GEMMF32_CFG_ENTRY_DECL(10) GEMMF32_CFG_ENTRY_DECL(11)
GEMMF32_CFG_ENTRY_DECL(12) GEMMF32_CFG_ENTRY_DECL(13) GEMMF32_CFG_ENTRY_DECL(14)
GEMMF32_CFG_ENTRY_DECL(15) GEMMF32_CFG_ENTRY_DECL(16) GEMMF32_CFG_ENTRY_DECL(17)
GEMMF32_CFG_ENTRY_DECL(18) GEMMF32_CFG_ENTRY_DECL(19)
#undef GEMMF32_CFG_ENTRY_DECL

}  // namespace gemmf32
