// The kernels of one tile configuration of gemmf32 and its host-side record.  This file is
// compiled once per configuration, with GEMMF32_CFG_ID set to the configuration's id, so
// that the configurations build in parallel; the library links all of them.
#include <hip/hip_runtime.h>

#include "configs.h"
#include "kernels_ks.h"
#include "kernels_ks16.h"
#include "kernels_ms.h"
#include "kernels_sb_db.h"

#ifndef GEMMF32_CFG_ID
#error "compile with -DGEMMF32_CFG_ID=<configuration id>"
#endif

namespace gemmf32 {

template <class C>
constexpr bool has_ms() {
  return C::BN % 64 == 0;
}

template <class C>
CfgEntry make_entry() {
  constexpr int S = has_ms<C>() ? ms_stages<C>() : 0;
  constexpr int KS = ks_groups<C>();
  KernelFn ms = nullptr, ks = nullptr;
  int lds_ms = 0;
  if constexpr (has_ms<C>()) {
    ms = &gemm_f32_ms_kernel<C, S>;
    lds_ms = (int)(MsCfg<C, S>::LDS_FLOATS * sizeof(float));
  }
  if constexpr (KS > 1) ks = &gemm_f32_ks_kernel<C, KS>;
  return CfgEntry{C::BM,
                  C::BN,
                  C::BK,
                  C::NT,
                  (int)(C::SLOT * sizeof(float)),
                  (int)(2 * C::SLOT * sizeof(float)),
                  S,
                  lds_ms,
                  &gemm_f32_tile_kernel<C, kLoopSB>,
                  &gemm_f32_tile_kernel<C, kLoopDB>,
                  ms,
                  &gemm_f32_tile_kernel<C, kLoopSB3>,
                  ks,
                  KS};
}

// The 16-row decode configurations: the K-split kernel only.
template <class D>
CfgEntry make_ks16_entry() {
  return CfgEntry{D::BM, D::BN, D::KG, 64, 0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr,
                  &gemm_f32_ks16_kernel<D>, D::WAVES};
}

template <class T>
struct EntryOf {
  static CfgEntry get() { return make_entry<T>(); }
};
template <int WAVES, int BLOCKS, bool STRIDED, int CB>
struct EntryOf<Ks16Cfg<WAVES, BLOCKS, STRIDED, CB>> {
  static CfgEntry get() { return make_ks16_entry<Ks16Cfg<WAVES, BLOCKS, STRIDED, CB>>(); }
};

#define GEMMF32_CAT2(a, b) a##b
#define GEMMF32_CAT(a, b) GEMMF32_CAT2(a, b)
CfgEntry GEMMF32_CAT(cfg_entry_, GEMMF32_CFG_ID)() {
  return EntryOf<typename CfgById<GEMMF32_CFG_ID>::type>::get();
}

}  // namespace gemmf32
