// gemmf32: FP32 GEMM C = A.B for gfx950 (MI355X), tiled through LDS, with a
// single-buffered and a double-buffered K-loop, an FP32 matrix-core micro-kernel,
// a guarded path for ragged or misaligned operands, and a per-shape dispatcher.
//
// What the K-loop does comes from two pages on the technique:
//   "Double Buffering" (metalworking glossary), code figure: two staging buffers per
//     operand; each iteration opens with one barrier, loads tile l+1 into the idle
//     buffer when there is one, computes on the current buffer and swaps.
//   "Case Study: The Double-Buffered GEMM", code figure: a prologue loads tile 0 into
//     buffer 0 before the loop; its second paragraph: the sibling (single-buffered)
//     kernel has one buffer set and two barriers per iteration.
//   Same case study, paragraph after the figure: the one barrier serves both as "the
//     prefetch has landed" and as "every wave is done reading the buffer about to be
//     overwritten", because the buffers alternate.
// The pages' own kernels target Apple GPUs; everything here is written for CDNA4:
// 64-lane waves, v_mfma_f32_32x32x2_f32 on the matrix cores, LDS with padded rows,
// 16-byte buffer loads from scalar tile bases (and direct-to-LDS copies in the
// multi-stage loop), and an XCD-aware ordering of workgroups.
//
// Files: gemm_common.h (tile configurations, copy, micro-kernel, epilogue),
// kernels_sb_db.h (single- and double-buffered loops), kernels_ms.h (multi-stage
// direct-to-LDS loop), kernels_ks.h (K split inside the workgroup), configs.h (the
// configuration list), cfg_kernels.hip (one configuration's kernels, compiled once per
// configuration), splitk_reduce.h (split-K reduction), dispatch_table.h (measured
// per-shape choices); this file holds the configuration table, argument validation,
// dispatch and the C ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gemmf32.h"
#include "configs.h"
#include "gemm_common.h"
#include "mfma_peak.h"
#include "splitk_reduce.h"

namespace gemmf32 {

// The table of tile configurations (configs.h); each entry's kernels live in the
// configuration's own translation unit.
static const CfgEntry kConfigs[] = {
    cfg_entry_0(),  cfg_entry_1(),  cfg_entry_2(),  cfg_entry_3(),  cfg_entry_4(),
    cfg_entry_5(),  cfg_entry_6(),  cfg_entry_7(),  cfg_entry_8(),  cfg_entry_9(),
    cfg_entry_10(), cfg_entry_11(), cfg_entry_12(), cfg_entry_13(), cfg_entry_14(),
    cfg_entry_15(), cfg_entry_16(), cfg_entry_17(), cfg_entry_18(), cfg_entry_19(),
};
static_assert(sizeof(kConfigs) / sizeof(kConfigs[0]) == kNumConfigs, "configuration table");

constexpr int kMaxSplits = 64;
constexpr int kSplitGranule = 64;  // K chunks are whole K tiles of every configuration

// K chunk of one split and the number of splits actually used.
static inline void splitk_plan(int64_t K, int splits, int64_t* k_chunk, int* used) {
  int64_t kc = (K + splits - 1) / splits;
  kc = (kc + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  if (kc < kSplitGranule) kc = kSplitGranule;
  *k_chunk = kc;
  *used = (int)((K + kc - 1) / kc);
}

}  // namespace gemmf32

#include "dispatch_table.h"

namespace gemmf32 {

// ------------------------------------------------------------------------------------
// Host side: validation, dispatch, launch.
// ------------------------------------------------------------------------------------
static thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = 2147483647LL - 1024;  // keeps tile-end arithmetic in int32
constexpr int64_t kMaxLd = kMaxDim * 64;           // leading dimensions (elements)
constexpr int64_t kMaxExtent = (int64_t)1 << 61;   // bytes one operand may span

// Byte extent ((rows - 1) * ld + cols) * 4 of a rows x cols operand with row stride ld
// (rows, cols >= 1), computed without signed overflow.  False when it passes kMaxExtent.
static bool extent_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t* bytes) {
  int64_t e;
  if (__builtin_mul_overflow(rows - 1, ld, &e) || __builtin_add_overflow(e, cols, &e) ||
      __builtin_mul_overflow(e, (int64_t)4, &e) || e > kMaxExtent)
    return false;
  *bytes = e;
  return true;
}

// [p, p + bytes) as addresses; false when it wraps around the address space.
static bool byte_range(const void* p, int64_t bytes, uintptr_t* lo, uintptr_t* hi) {
  *lo = (uintptr_t)p;
  if (__builtin_add_overflow(*lo, (uintptr_t)bytes, hi)) return false;
  return true;
}

static bool overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

// Byte ranges of the operands of a validated, non-empty call (A and B only when K > 0).
struct Extents {
  uintptr_t a0, a1, b0, b1, c0, c1;
};

static int validate(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                    const float* B, int64_t ldb, const float* C, int64_t ldc,
                    Extents* ext = nullptr) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  const int64_t min_lda = K > 1 ? K : 1;
  const int64_t min_ldb = N > 1 ? N : 1;
  if (lda < min_lda || ldb < min_ldb || ldc < min_ldb) return GEMMF32_ERR_BAD_LD;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMMF32_ERR_TOO_LARGE;
  if (lda > kMaxLd || ldb > kMaxLd || ldc > kMaxLd) return GEMMF32_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return GEMMF32_OK;
  if (C == nullptr) return GEMMF32_ERR_NULL_PTR;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMMF32_ERR_NULL_PTR;
  if (((uintptr_t)C & 3u) != 0) return GEMMF32_ERR_MISALIGNED;
  if (K > 0 && ((((uintptr_t)A) & 3u) != 0 || (((uintptr_t)B) & 3u) != 0))
    return GEMMF32_ERR_MISALIGNED;
  // Byte extents [begin, end) of the three operands, each at most kMaxExtent and not
  // wrapping; C must be disjoint from A and B.
  Extents x{0, 0, 0, 0, 0, 0};
  int64_t cb;
  if (!extent_bytes(M, N, ldc, &cb) || !byte_range(C, cb, &x.c0, &x.c1))
    return GEMMF32_ERR_TOO_LARGE;
  if (K > 0) {
    int64_t ab, bb;
    if (!extent_bytes(M, K, lda, &ab) || !byte_range(A, ab, &x.a0, &x.a1) ||
        !extent_bytes(K, N, ldb, &bb) || !byte_range(B, bb, &x.b0, &x.b1))
      return GEMMF32_ERR_TOO_LARGE;
    if (overlap(x.c0, x.c1, x.a0, x.a1) || overlap(x.c0, x.c1, x.b0, x.b1))
      return GEMMF32_ERR_ALIAS;
  }
  if (ext) *ext = x;
  return GEMMF32_OK;
}

// GEMMF32_RASTER=<group_m>[,noxcd] changes the workgroup order of every launch (for
// measurement); group_m in 1..255.
static int env_raster_flags() {
  const char* v = std::getenv("GEMMF32_RASTER");
  if (v == nullptr || *v == 0) return 0;
  char* end = nullptr;
  long gm = std::strtol(v, &end, 10);
  int flags = 0;
  if (gm >= 1 && gm <= 255) flags |= (int)gm << kRasterGroupShift;
  if (end && std::strstr(end, "noxcd")) flags |= kRasterNoXcdRemap;
  return flags;
}

// How one launch divides the product (the host side of SplitArgs).  split_from: the first
// split tile in launch order (0: every tile is split).
struct SplitPlan {
  float* ws;
  int64_t plane;
  int64_t k_chunk;
  int chunks;
  int64_t split_from;
};

// Kernel flags of a launch with tile configuration e.
static int launch_flags(const CfgEntry& e, int64_t K, int64_t lda, int64_t ldb) {
  int flags = 0;
  // 16-byte copies address a tile with 32-bit per-thread byte offsets (rows x leading
  // dimension), which must stay below the buffer range; rows need only the 4-byte
  // alignment that validation already demands.
  if (K > 0 && (int64_t)e.bm * lda * 4 <= (int64_t)kBufferRange) flags |= kVecA;
  if (K > 0 && (int64_t)e.bk * ldb * 4 <= (int64_t)kBufferRange) flags |= kVecB;
  return flags | env_raster_flags();
}

// One launch of a GEMM kernel: every tile over the whole K range into C, or with `plan`,
// the tiles from plan->split_from on in plan->chunks K chunks into the workspace.
static int launch(int variant, int cfg_id, int64_t M, int64_t N, int64_t K, const float* A,
                  int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                  void* stream, const SplitPlan* plan = nullptr) {
  const CfgEntry& e = kConfigs[cfg_id];
  KernelFn fn = variant == GEMMF32_VARIANT_SB    ? e.sb
                : variant == GEMMF32_VARIANT_MS  ? e.ms
                : variant == GEMMF32_VARIANT_SB3 ? e.sb3
                : variant == GEMMF32_VARIANT_KS  ? e.ks
                                                 : e.db;
  // a configuration without this variant's kernel; the K-split kernel divides K itself
  if (fn == nullptr || (variant == GEMMF32_VARIANT_KS && plan != nullptr))
    return GEMMF32_ERR_BAD_CONFIG;
  const int threads = variant == GEMMF32_VARIANT_KS ? e.nt * e.ks_groups : e.nt;
  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
  const int64_t from = plan ? std::min(plan->split_from, tiles) : tiles;
  const int64_t chunks = plan ? plan->chunks : 1;
  const int64_t wgs = from + (tiles - from) * chunks;
  if (wgs * threads > 0xFFFFFFFFLL) return GEMMF32_ERR_TOO_LARGE;
  int flags = launch_flags(e, K, lda, ldb);
  int m = (int)M, n = (int)N, k = (int)K;
  SplitArgs sp{plan ? plan->ws : nullptr, plan ? plan->plane : 0,
               plan ? (int)plan->k_chunk : k, (int)chunks, (int)from, (int)tiles};
  void* args[] = {&m, &n, &k, (void*)&A, &lda, (void*)&B, &ldb, &C, &ldc, &flags, &sp};
  hipError_t err = hipLaunchKernel((const void*)fn, dim3((unsigned)wgs), dim3(threads), args,
                                   0, (hipStream_t)stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return GEMMF32_ERR_HIP;
  }
  return GEMMF32_OK;
}

static bool has_variant(int cfg_id, int variant) {
  const CfgEntry& e = kConfigs[cfg_id];
  switch (variant) {
    case GEMMF32_VARIANT_SB: return e.sb != nullptr;
    case GEMMF32_VARIANT_DB: return e.db != nullptr;
    case GEMMF32_VARIANT_MS: return e.ms != nullptr;
    case GEMMF32_VARIANT_SB3: return e.sb3 != nullptr;
    case GEMMF32_VARIANT_KS: return e.ks != nullptr;
    default: return false;
  }
}

// The first configuration with a kernel for `variant` (the measured tables name one for
// every variant they timed; this covers a table without the variant).
static int first_cfg_with(int variant) {
  for (int c = 0; c < kNumConfigs; ++c)
    if (has_variant(c, variant)) return c;
  return 0;
}

static int env_variant() {
  const char* v = std::getenv("GEMMF32_VARIANT");
  if (v == nullptr) return GEMMF32_VARIANT_AUTO;
  if (std::strcmp(v, "sb") == 0) return GEMMF32_VARIANT_SB;
  if (std::strcmp(v, "db") == 0) return GEMMF32_VARIANT_DB;
  if (std::strcmp(v, "ms") == 0) return GEMMF32_VARIANT_MS;
  if (std::strcmp(v, "ks") == 0) return GEMMF32_VARIANT_KS;
  return GEMMF32_VARIANT_AUTO;
}

static int run(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
               int64_t ldb, float* C, int64_t ldc, int variant, int cfg_id, void* stream) {
  if (variant != GEMMF32_VARIANT_AUTO && variant != GEMMF32_VARIANT_SB &&
      variant != GEMMF32_VARIANT_DB && variant != GEMMF32_VARIANT_MS &&
      variant != GEMMF32_VARIANT_SB3 && variant != GEMMF32_VARIANT_KS)
    return GEMMF32_ERR_BAD_CONFIG;
  if (cfg_id < -1 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  if (cfg_id >= 0 && variant != GEMMF32_VARIANT_AUTO && !has_variant(cfg_id, variant))
    return GEMMF32_ERR_BAD_CONFIG;
  int rc = validate(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != GEMMF32_OK) return rc;
  if (M == 0 || N == 0) return GEMMF32_OK;
  if (variant == GEMMF32_VARIANT_AUTO) {
    int v = 0, c = 0;
    select_shape(M, N, K, &v, &c);
    variant = v;
    if (cfg_id < 0) {
      cfg_id = c;
    } else if (!has_variant(cfg_id, variant)) {
      // a forced configuration without the picked variant: its double-buffered kernel, or
      // its K-split one where it has no other
      variant = has_variant(cfg_id, GEMMF32_VARIANT_DB) ? GEMMF32_VARIANT_DB
                                                        : GEMMF32_VARIANT_KS;
    }
  } else if (cfg_id < 0) {
    cfg_id = select_for_variant(M, N, K, variant == GEMMF32_VARIANT_SB3 ? GEMMF32_VARIANT_SB
                                                                        : variant);
    if (!has_variant(cfg_id, variant)) cfg_id = first_cfg_with(variant);
  }
  return launch(variant, cfg_id, M, N, K, A, lda, B, ldb, C, ldc, stream);
}


// The plan of a split-K call with `splits` (> 0: every tile split; < 0: only the tail tiles
// split into -splits chunks, or every tile when the product has no tail): the chunks, the
// tile configuration, the first split tile and the workspace floats.  used <= 1: no split.
struct SplitLayout {
  int64_t kc;
  int used;
  int variant, cfg;
  int64_t split_from;
  int64_t need;  // workspace floats; -1 when the workspace would pass kMaxExtent bytes
};

// a * b * c as workspace floats, or -1 when its byte size would pass kMaxExtent.
static int64_t checked_product(int64_t a, int64_t b, int64_t c) {
  int64_t r;
  if (__builtin_mul_overflow(a, b, &r) || __builtin_mul_overflow(r, c, &r) ||
      r > kMaxExtent / 4)
    return -1;
  return r;
}

static SplitLayout splitk_layout(int64_t M, int64_t N, int64_t K, int splits) {
  SplitLayout L{0, 1, 0, 0, 0, 0};
  if (K > 0) splitk_plan(K, splits < 0 ? -splits : splits, &L.kc, &L.used);
  if (L.used <= 1) return L;
  const TailPick tp = splits < 0 ? tail_pick(M, N, K, L.used, L.kc) : TailPick{};
  if (tp.found) {
    // Full rounds run whole; the split tiles' chunks go to packed tile blocks.
    const CfgEntry& e = kConfigs[tp.cfg];
    const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
    L.variant = tp.variant;
    L.cfg = tp.cfg;
    L.split_from = tp.split_from;
    L.need = checked_product(L.used, tiles - tp.split_from, (int64_t)e.bm * e.bn);
  } else {
    // Every tile split: its chunks run side by side in one grid, so the tile is chosen for
    // `used` times the workgroups of one chunk's product; partial products are M x N planes.
    const ModelRow& pick = model_pick(M, N, L.kc, 0, L.used);
    L.variant = pick.variant;
    L.cfg = pick.cfg;
    L.need = checked_product(L.used, M, N);
  }
  return L;
}

// The two launches of a split product whose workspace `ws` holds L.need floats: the GEMM
// kernel writes every chunk's partial product into it (each element of each partial is
// stored, so nothing needs clearing first), then a reduction sums the chunks into C.
static int splitk_launch(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                         const float* B, int64_t ldb, float* C, int64_t ldc,
                         const SplitLayout& L, float* ws, void* stream) {
  const SplitPlan plan{ws, M * N, L.kc, L.used, L.split_from};
  int rc = launch(L.variant, L.cfg, M, N, K, A, lda, B, ldb, C, ldc, stream, &plan);
  if (rc != GEMMF32_OK) return rc;
  int m = (int)M, n = (int)N, used = L.used;
  const float* p = ws;
  hipError_t err;
  if (L.split_from > 0) {
    const CfgEntry& e = kConfigs[L.cfg];
    const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
    int bm = e.bm, bn = e.bn, from = (int)L.split_from, nt = (int)tiles;
    int flags = env_raster_flags();
    void* args[] = {&m, &n, &used, (void*)&p, &C, &ldc, &bm, &bn, &from, &nt, &flags};
    const dim3 grid((unsigned)(tiles - L.split_from), (unsigned)((bm * bn + 255) / 256));
    err = hipLaunchKernel((const void*)&gemm_f32_splitk_reduce_tiles, grid, dim3(256), args, 0,
                          (hipStream_t)stream);
  } else {
    const bool vec = (N % 4) == 0 && (ldc % 4) == 0 && ((uintptr_t)ws & 15u) == 0 &&
                     ((uintptr_t)C & 15u) == 0;
    const int64_t items = vec ? M * (N / 4) : M * N;
    const int64_t blocks64 = (items + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 4096 ? blocks64 : 4096);
    void* args[] = {&m, &n, &used, (void*)&p, &C, &ldc};
    const void* fn = vec ? (const void*)&gemm_f32_splitk_reduce<true>
                         : (const void*)&gemm_f32_splitk_reduce<false>;
    err = hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, (hipStream_t)stream);
  }
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return GEMMF32_ERR_HIP;
  }
  return GEMMF32_OK;
}

// Validation and layout shared by both split entry points.  Returns GEMMF32_OK with
// *plain set when the call is an unsplit product (or empty), otherwise the layout in *L.
static int splitk_prepare(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                          const float* B, int64_t ldb, const float* C, int64_t ldc,
                          int splits, Extents* x, SplitLayout* L, bool* plain) {
  if (splits == 0 && M >= 0 && N >= 0 && K >= 0) splits = select_splits(M, N, K);
  if (splits == 0 || splits == -1 || splits < -kMaxSplits || splits > kMaxSplits)
    return GEMMF32_ERR_BAD_CONFIG;
  const int rc = validate(M, N, K, A, lda, B, ldb, C, ldc, x);
  if (rc != GEMMF32_OK) return rc;
  *plain = true;
  if (M == 0 || N == 0) return GEMMF32_OK;
  *L = splitk_layout(M, N, K, splits);
  if (L->used <= 1) return GEMMF32_OK;
  if (L->need < 0) return GEMMF32_ERR_TOO_LARGE;
  *plain = false;
  return GEMMF32_OK;
}

static int run_splitk(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                      const float* B, int64_t ldb, float* C, int64_t ldc, int splits,
                      float* ws, int64_t ws_floats, void* stream) {
  Extents x;
  SplitLayout L;
  bool plain = true;
  int rc = splitk_prepare(M, N, K, A, lda, B, ldb, C, ldc, splits, &x, &L, &plain);
  if (rc != GEMMF32_OK) return rc;
  if (plain) {
    if (M == 0 || N == 0) return GEMMF32_OK;
    return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_AUTO, -1, stream);
  }
  if (ws == nullptr) return GEMMF32_ERR_NULL_PTR;
  if (((uintptr_t)ws & 3u) != 0) return GEMMF32_ERR_MISALIGNED;
  if (ws_floats < L.need) return GEMMF32_ERR_BAD_LD;
  // The workspace must not overlap A, B or C (K > 0 here: a split needs K chunks).
  uintptr_t w0, w1;
  if (!byte_range(ws, L.need * 4, &w0, &w1)) return GEMMF32_ERR_TOO_LARGE;
  if (overlap(w0, w1, x.a0, x.a1) || overlap(w0, w1, x.b0, x.b1) ||
      overlap(w0, w1, x.c0, x.c1))
    return GEMMF32_ERR_ALIAS;
  return splitk_launch(M, N, K, A, lda, B, ldb, C, ldc, L, ws, stream);
}

// ------------------------------------------------------------------------------------
// The static scratch of gemm_f32_splitk_noalloc.  Each device the library runs on holds
// its own copy of this array from the module's load until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and is kept in g_scratch.
// ------------------------------------------------------------------------------------
static __device__ __align__(256) float scratch[GEMMF32_SCRATCH_FLOATS];

constexpr int kMaxDevices = 64;
static std::atomic<float*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The device address of `scratch` on the device `stream` belongs to (the current device
// for the NULL stream).
static int scratch_address(void* stream, float** out) {
  int dev = -1;
  hipError_t err = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return GEMMF32_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = (int)hipErrorInvalidDevice;
    return GEMMF32_ERR_HIP;
  }
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      err = hipGetDevice(&cur);
      if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
      void* addr = nullptr;
      if (err == hipSuccess) err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (cur >= 0 && cur != dev) {
        const hipError_t back = hipSetDevice(cur);
        if (err == hipSuccess) err = back;
      }
      if (err != hipSuccess || addr == nullptr) {
        g_last_hip_error = (int)(err != hipSuccess ? err : hipErrorInvalidSymbol);
        return GEMMF32_ERR_HIP;
      }
      p = static_cast<float*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GEMMF32_OK;
}

static int run_splitk_noalloc(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                              const float* B, int64_t ldb, float* C, int64_t ldc, int splits,
                              void* stream) {
  Extents x;
  SplitLayout L;
  bool plain = true;
  int rc = splitk_prepare(M, N, K, A, lda, B, ldb, C, ldc, splits, &x, &L, &plain);
  if (rc != GEMMF32_OK) return rc;
  if (plain) {
    if (M == 0 || N == 0) return GEMMF32_OK;
    return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_AUTO, -1, stream);
  }
  if (L.need > (int64_t)GEMMF32_SCRATCH_FLOATS) return GEMMF32_ERR_SCRATCH_LIMIT;
  float* ws = nullptr;
  rc = scratch_address(stream, &ws);
  if (rc != GEMMF32_OK) return rc;
  return splitk_launch(M, N, K, A, lda, B, ldb, C, ldc, L, ws, stream);
}

}  // namespace gemmf32

using namespace gemmf32;

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
             int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, env_variant(), -1, stream);
}

int gemm_f32_sb(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_SB, -1, stream);
}

int gemm_f32_db(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_DB, -1, stream);
}

int gemm_f32_ms(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, GEMMF32_VARIANT_MS, -1, stream);
}

int gemm_f32_ex(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc, int variant, int cfg_id, void* stream) {
  return run(M, N, K, A, lda, B, ldb, C, ldc, variant, cfg_id, stream);
}

int gemm_f32_splitk(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                    const float* B, int64_t ldb, float* C, int64_t ldc, int splits,
                    float* workspace, int64_t workspace_floats, void* stream) {
  return run_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_floats,
                    stream);
}

int gemm_f32_splitk_noalloc(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                            const float* B, int64_t ldb, float* C, int64_t ldc, int splits,
                            void* stream) {
  return run_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, splits, stream);
}

int gemm_f32_splitk_select(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  return select_splits(M, N, K);
}

int64_t gemm_f32_splitk_workspace(int64_t M, int64_t N, int64_t K, int splits) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  if (splits == 0) splits = select_splits(M, N, K);
  if (splits == 0 || splits == -1 || splits < -kMaxSplits || splits > kMaxSplits)
    return GEMMF32_ERR_BAD_CONFIG;
  if (M == 0 || N == 0 || K == 0) return 0;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMMF32_ERR_TOO_LARGE;
  const SplitLayout L = splitk_layout(M, N, K, splits);
  if (L.used <= 1) return 0;
  return L.need < 0 ? GEMMF32_ERR_TOO_LARGE : L.need;
}

int gemm_f32_splitk_plan(int64_t M, int64_t N, int64_t K, int splits, int* variant,
                         int* cfg_id, int* chunks, int64_t* split_from) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  if (splits == 0) splits = select_splits(M, N, K);
  if (splits == 0 || splits == -1 || splits < -kMaxSplits || splits > kMaxSplits)
    return GEMMF32_ERR_BAD_CONFIG;
  const SplitLayout L = splitk_layout(M, N, K, splits);
  int v = L.variant, c = L.cfg, used = L.used;
  int64_t from = L.split_from;
  if (L.used <= 1) {  // the plain product
    select_shape(M, N, K, &v, &c);
    used = 1;
    const CfgEntry& e = kConfigs[c];
    from = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
  }
  if (variant) *variant = v;
  if (cfg_id) *cfg_id = c;
  if (chunks) *chunks = used;
  if (split_from) *split_from = from;
  return GEMMF32_OK;
}

int gemm_f32_select(int64_t M, int64_t N, int64_t K, int* variant, int* cfg_id) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  int v = 0, c = 0;
  select_shape(M, N, K, &v, &c);
  if (variant) *variant = v;
  if (cfg_id) *cfg_id = c;
  return GEMMF32_OK;
}

int gemm_f32_select_cfg(int64_t M, int64_t N, int64_t K, int variant) {
  if (M < 0 || N < 0 || K < 0) return GEMMF32_ERR_NEGATIVE_DIM;
  if (variant != GEMMF32_VARIANT_SB && variant != GEMMF32_VARIANT_DB &&
      variant != GEMMF32_VARIANT_MS && variant != GEMMF32_VARIANT_KS)
    return GEMMF32_ERR_BAD_CONFIG;
  const int c = select_for_variant(M, N, K, variant);
  return has_variant(c, variant) ? c : first_cfg_with(variant);
}

int gemm_f32_num_configs(void) { return kNumConfigs; }

int gemm_f32_config_info(int cfg_id, int* BM, int* BN, int* BK, int* threads, int* lds_sb,
                         int* lds_db) {
  if (cfg_id < 0 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  const CfgEntry& e = kConfigs[cfg_id];
  if (BM) *BM = e.bm;
  if (BN) *BN = e.bn;
  if (BK) *BK = e.bk;
  if (threads) *threads = e.nt;
  if (lds_sb) *lds_sb = e.lds_sb;
  if (lds_db) *lds_db = e.lds_db;
  return GEMMF32_OK;
}

int gemm_f32_config_ms(int cfg_id, int* stages, int* lds_bytes) {
  if (cfg_id < 0 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  const CfgEntry& e = kConfigs[cfg_id];
  if (stages) *stages = e.ms_stages;
  if (lds_bytes) *lds_bytes = e.lds_ms;
  return GEMMF32_OK;
}

int gemm_f32_config_variants(int cfg_id) {
  if (cfg_id < 0 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  int mask = 0;
  for (int v : {GEMMF32_VARIANT_SB, GEMMF32_VARIANT_DB, GEMMF32_VARIANT_MS, GEMMF32_VARIANT_SB3,
                GEMMF32_VARIANT_KS})
    if (has_variant(cfg_id, v)) mask |= 1 << v;
  return mask;
}

int gemm_f32_config_ks(int cfg_id) {
  if (cfg_id < 0 || cfg_id >= kNumConfigs) return GEMMF32_ERR_BAD_CONFIG;
  return kConfigs[cfg_id].ks_groups;
}

int gemm_f32_last_hip_error(void) { return g_last_hip_error; }

const char* gemm_f32_strerror(int code) {
  switch (code) {
    case GEMMF32_OK: return "success";
    case GEMMF32_ERR_NEGATIVE_DIM: return "negative matrix dimension";
    case GEMMF32_ERR_BAD_LD: return "leading dimension smaller than the row length";
    case GEMMF32_ERR_NULL_PTR: return "null pointer for a non-empty operand";
    case GEMMF32_ERR_MISALIGNED: return "operand pointer not 4-byte aligned";
    case GEMMF32_ERR_ALIAS: return "C overlaps A or B";
    case GEMMF32_ERR_TOO_LARGE: return "dimension or grid too large for one launch";
    case GEMMF32_ERR_BAD_CONFIG: return "unknown variant or tile configuration";
    case GEMMF32_ERR_HIP: return "HIP kernel launch failed";
    case GEMMF32_ERR_SCRATCH_LIMIT: return "split needs more than the static scratch holds";
    default: return "unknown error code";
  }
}

const char* gemm_f32_version(void) {
  return GEMMF32_LDS_POISON ? "gemmf32 0.1.0 gfx950 lds-poison" : "gemmf32 0.1.0 gfx950";
}

int gemm_f32_peak_probe(int blocks, int iters, float* out, uint64_t* rec, void* stream) {
  if (blocks < 1 || blocks > kPeakMaxBlocks || iters < 0 || iters > kPeakMaxIters)
    return GEMMF32_ERR_TOO_LARGE;
  if (out == nullptr || rec == nullptr) return GEMMF32_ERR_NULL_PTR;
  if (((uintptr_t)out & 3u) != 0 || ((uintptr_t)rec & 7u) != 0) return GEMMF32_ERR_MISALIGNED;
  void* args[] = {&iters, &out, &rec};
  hipError_t err = hipLaunchKernel((const void*)&gemm_f32_peak_kernel, dim3(blocks),
                                   dim3(kPeakThreads), args, 0, (hipStream_t)stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return GEMMF32_ERR_HIP;
  }
  return GEMMF32_OK;
}

}  // extern "C"
