"""Measure every (variant, tile configuration) per shape on the GPU and regenerate the
dispatch table csrc/dispatch_table.h from the measurements.

    python -m tiled_double_buffered_amd.tune [--out results.json] [--write-header]

Protocol (after the repeated, counterbalanced timing of the LuisaCompute note "Dependence-
aware group synchronization on M1 Max", section "Controlled implementation comparison"):
for each shape, `rounds` rounds visit every (variant, configuration) pair in an order that
rotates from round to round; each visit times `batches` batches of back-to-back launches
(each batch at least `batch_ms` of GPU time) with HIP events on the launch stream; a pair's
time is the median over rounds of the per-round median batch.  The fastest configuration
of each variant and the overall winner go into the table (within 0.5% of the fastest, the
larger tile, then the smaller LDS footprint).  The same measurements, plus those of seeded
shapes outside the table, fit the cost model that picks for every other shape.

    python -m tiled_double_buffered_amd.tune --holdout 40   # dispatcher regret on 40 seeded
                                                            # shapes outside the table
    python -m tiled_double_buffered_amd.tune --holdout-decode 16   # ... on decode products

After shapes are added to the table or the training set, --fill measures only the ones an
earlier --out file lacks and writes the merged file (the split study is kept as it was):

    python -m tiled_double_buffered_amd.tune --fill full.json --out full2.json   # GPU

The split-count study times the unsplit product through gemm_f32, that is through the
dispatch table the library was built with.  After a change of the configurations, measure
in two steps so that it sees the new table:

    python -m tiled_double_buffered_amd.tune --no-split --out base.json   # GPU
    python -m tiled_double_buffered_amd.tune --from-json base.json        # header; rebuild
    python -m tiled_double_buffered_amd.tune --split-only base.json --out full.json   # GPU
    python -m tiled_double_buffered_amd.tune --from-json full.json        # header; rebuild

Timing does not depend on the values multiplied, so inputs are seeded uniform values.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

from . import _binding as tdb
from .build import CSRC

VARIANTS = (tdb.VARIANT_SB, tdb.VARIANT_DB, tdb.VARIANT_MS, tdb.VARIANT_KS)
NAMES = {tdb.VARIANT_SB: "sb", tdb.VARIANT_DB: "db", tdb.VARIANT_MS: "ms",
         tdb.VARIANT_KS: "ks"}
IDS = {v: k for k, v in NAMES.items()}


def available_pairs():
    """(variant, cfg) pairs that have a kernel, in configuration order."""
    out = []
    for c in range(tdb.gemm_f32_num_configs()):
        mask = tdb.gemm_f32_config_variants(c)
        out += [(v, c) for v in VARIANTS if mask & (1 << v)]
    return out

SHAPES = [
    # the workloads
    (128, 128, 128), (127, 193, 61), (513, 257, 129), (1024, 1024, 1024),
    (256, 1024, 128), (1024, 128, 256), (4096, 4096, 4096), (8192, 8192, 8192),
    # more measured points, also fitted by the cost model; the squares trace the SB / DB
    # regimes from 256 to 8192
    (256, 256, 256), (512, 512, 512), (768, 768, 768), (1536, 1536, 1536),
    (2048, 2048, 2048), (3072, 3072, 3072), (6144, 6144, 6144),
    (64, 4096, 4096), (4096, 4096, 512), (2048, 8192, 2048), (4096, 1024, 1024),
    (1024, 1024, 8192),
    # a few hundred rows against a layer: one round of workgroups
    (512, 4096, 4096), (512, 4096, 11008),
    # odd sizes: edge tiles, a K tail and leading dimensions that are not multiples of 4
    (1023, 1023, 1023), (4095, 4095, 4095),
    # skinny shapes (a small batch of rows against a wide layer)
    (16, 4096, 4096), (32, 4096, 4096), (128, 4096, 4096), (32, 8192, 8192),
    (128, 11008, 4096), (128, 4096, 11008),
    # decode rows (1 to 16) against 4096- to 32000-wide layers, and a small one
    (1, 4096, 4096), (8, 4096, 4096), (16, 11008, 4096), (16, 4096, 11008),
    (16, 8192, 8192), (4, 1024, 1024), (16, 32000, 4096),
    (1, 11008, 4096), (1, 4096, 11008), (1, 8192, 8192), (1, 32000, 4096), (4, 4096, 4096),
    # one GPU's share of 8192^3 split by rows over eight GPUs
    (1024, 8192, 8192),
]

# Shapes for the split-count table: skinny, tall-K and square.
SPLIT_SHAPES = [(16, 4096, 4096), (32, 4096, 4096), (64, 4096, 4096), (128, 4096, 4096),
                (32, 8192, 8192), (64, 8192, 8192), (256, 256, 8192), (512, 512, 8192),
                (1024, 1024, 1024), (2048, 2048, 2048), (4096, 4096, 4096)]
# Shapes whose tiles leave the last round of workgroups partly filled (the tail split).
TAIL_SHAPES = [(1536, 1536, 1536), (1536, 1536, 4096), (2560, 2560, 2560), (1280, 1280, 2048),
               (5000, 5000, 1000), (1536, 3072, 4096)]
SPLIT_CHOICES = (1, 2, 4, 8, 16)
# Skinny shapes measured only to fit the split model.
SPLIT_TRAIN_SEED = 7
SPLIT_TRAIN_COUNT = 24

HEADER_TEMPLATE = """// Per-shape dispatch table: (M, N, K) -> variant and tile configuration.
//
// The pages' central measured lesson is that double buffering wins at some sizes and
// loses or ties at others, so a library has to pick a variant per shape ("Double
// Buffering", last two paragraphs; "Case Study: The Double-Buffered GEMM", paragraph on
// the three regimes).  The rows below were measured on {device} by
// tiled_double_buffered_amd/tune.py ({rounds} rotated rounds x {batches} batches of >= {batch_ms} ms
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

namespace gemmf32 {{

struct DispatchRow {{
  int64_t m, n, k;
  int variant, cfg, sb_cfg, db_cfg, ms_cfg;
}};

static const DispatchRow kDispatch[] = {{
{rows}
}};
constexpr int kDispatchRows = (int)(sizeof(kDispatch) / sizeof(kDispatch[0]));

static inline double dispatch_log2(int64_t x) {{ return x > 0 ? std::log2((double)x) : -1.0; }}

static inline const DispatchRow* dispatch_exact(int64_t M, int64_t N, int64_t K) {{
  for (int i = 0; i < kDispatchRows; ++i)
    if (kDispatch[i].m == M && kDispatch[i].n == N && kDispatch[i].k == K) return &kDispatch[i];
  return nullptr;
}}

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
// squares on relative error, all kept >= 0, to the {nfit} shapes measured for this file
// (the table's {ntable} and {ntrain} seeded shapes outside it).
struct ModelRow {{
  int variant, cfg;
  double a_us, b_us, g_us, h_us;
}};

static const ModelRow kModel[] = {{
{model_rows}
}};
constexpr int kModelRows = (int)(sizeof(kModel) / sizeof(kModel[0]));
constexpr int kVariantMS = 3;
constexpr int kVariantKS = 5;
constexpr int64_t kModelCUs = 256;

// Modelled microseconds of one launch; wg_factor multiplies the workgroup count (the K
// chunks of a split-K launch run side by side in one grid).
static inline double model_us(const ModelRow& r, int64_t M, int64_t N, int64_t K,
                              int64_t wg_factor) {{
  const CfgEntry& e = kConfigs[r.cfg];
  const int64_t tiles = ((M + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn) * wg_factor;
  const int64_t rounds = (tiles + kModelCUs - 1) / kModelCUs;
  const int64_t k_tiles = (K + e.bk - 1) / e.bk;
  return r.a_us + r.b_us * (double)rounds + r.g_us * (double)rounds * (double)k_tiles +
         r.h_us * (double)tiles * (double)k_tiles / (double)kModelCUs;
}}

// The row with the least modelled time (variant 0: any variant), first row on ties.
static inline const ModelRow& model_pick(int64_t M, int64_t N, int64_t K, int variant,
                                         int64_t wg_factor) {{
  int best = 0;
  double best_t = 0.0;
  bool found = false;
  for (int i = 0; i < kModelRows; ++i) {{
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
    if (!found || t < best_t) {{
      best = i;
      best_t = t;
      found = true;
    }}
  }}
  return kModel[best];
}}

static inline void select_shape(int64_t M, int64_t N, int64_t K, int* variant, int* cfg) {{
  if (const DispatchRow* r = dispatch_exact(M, N, K)) {{
    *variant = r->variant;
    *cfg = r->cfg;
    return;
  }}
  const ModelRow& m = model_pick(M, N, K, 0, 1);
  *variant = m.variant;
  *cfg = m.cfg;
}}

static inline int select_for_variant(int64_t M, int64_t N, int64_t K, int variant) {{
  const DispatchRow* r = variant != kVariantKS ? dispatch_exact(M, N, K) : nullptr;
  if (r) return variant == 1 ? r->sb_cfg : variant == 3 ? r->ms_cfg : r->db_cfg;
  return model_pick(M, N, K, variant, 1).cfg;
}}

// Split-K: the number of K chunks (1 = do not split) with the least modelled time among
// the counts the split study measured.  A split launch costs the GEMM of its chunks, all in
// one grid (the model above, with the workgroups multiplied by the chunks), plus
//     {split_fixed:.4f} us (the reduction's launch)
//   + {split_us_per_mb:.5f} us per MB of (2 * chunks + 1) * M * N * 4 bytes (partial products,
//     written once and read once by the reduction, and C)
//   + {split_us_per_round:.4f} us per round of workgroups of the split grid (each workgroup's
//     first copy and partial-tile store, which short chunks no longer hide),
// the constants fitted (>= 0, least squares) to the {nsplit} shapes of the split study below.
constexpr double kSplitFixedUs = {split_fixed:.4f};
constexpr double kSplitUsPerMB = {split_us_per_mb:.5f};
constexpr double kSplitUsPerRound = {split_us_per_round:.4f};
constexpr int kSplitChoices[] = {{{split_choices}}};

// The split study: trailing comments hold the measured microseconds of each count.
struct SplitRow {{
  int64_t m, n, k;
  int splits;
}};

static const SplitRow kSplitK[] = {{
{split_rows}
}};

static inline double model_best_us(int64_t M, int64_t N, int64_t K, int64_t wg_factor) {{
  return model_us(model_pick(M, N, K, 0, wg_factor), M, N, K, wg_factor);
}}

static inline double split_model_us(int64_t M, int64_t N, int64_t K, int splits) {{
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
}}

// Tail split: only the tiles of the last, partly filled round of workgroups are split (the
// full rounds run whole), priced like a split launch whose overhead covers just those
// tiles.  The pick with the least modelled time among the configurations whose tiles make
// at least one full round and a partly filled one; found = false when there is none.
struct TailPick {{
  bool found;
  int variant, cfg;
  int64_t split_from;
  double us;
}};

static inline TailPick tail_pick(int64_t M, int64_t N, int64_t K, int used, int64_t kc) {{
  TailPick best{{false, 0, 0, 0, 0.0}};
  for (int i = 0; i < kModelRows; ++i) {{
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
    if (!best.found || t < best.us) best = TailPick{{true, r.variant, r.cfg, full, t}};
  }}
  return best;
}}

// The split count: > 1 splits every tile, 1 does not split, -s splits only the tail tiles
// into s chunks.
static inline int select_splits(int64_t M, int64_t N, int64_t K) {{
  int best = 1;
  double best_t = 0.0;
  for (int i = 0; i < (int)(sizeof(kSplitChoices) / sizeof(kSplitChoices[0])); ++i) {{
    const double t = split_model_us(M, N, K, kSplitChoices[i]);
    if (i == 0 || t < best_t) {{
      best = kSplitChoices[i];
      best_t = t;
    }}
  }}
  for (int i = 0; i < (int)(sizeof(kSplitChoices) / sizeof(kSplitChoices[0])); ++i) {{
    const int s = kSplitChoices[i];
    if (s < 2 || K <= 0) continue;
    int64_t kc = 0;
    int used = 1;
    splitk_plan(K, s, &kc, &used);
    if (used <= 1) continue;
    const TailPick tp = tail_pick(M, N, K, used, kc);
    if (tp.found && tp.us < best_t) {{
      best = -s;
      best_t = tp.us;
    }}
  }}
  return best;
}}

}}  // namespace gemmf32
"""


def measure(shapes, rounds=2, batches=5, batch_ms=20.0, log=print):
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    s_ptr = stream.cuda_stream
    pairs = available_pairs()
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    results = []
    for (M, N, K) in shapes:
        A = torch.rand((M, K), device=dev, generator=gen) * 2 - 1
        B = torch.rand((K, N), device=dev, generator=gen) * 2 - 1
        C = torch.empty((M, N), device=dev)
        pa, pb, pc = A.data_ptr(), B.data_ptr(), C.data_ptr()

        def call(v, c):
            rc = tdb.gemm_f32_ex(M, N, K, pa, K, pb, N, pc, N, v, c, s_ptr)
            if rc != tdb.OK:
                raise tdb.GemmError(rc, "gemm_f32_ex")

        reps = {}
        for (v, c) in pairs:  # calibrate launches per batch
            call(v, c)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(3):
                call(v, c)
            e1.record(stream)
            torch.cuda.synchronize()
            one = e0.elapsed_time(e1) / 3
            reps[(v, c)] = int(min(20000, max(2, batch_ms / max(one, 1e-4))))
        per_round = {p: [] for p in pairs}
        for r in range(rounds):
            shift = (r * len(pairs)) // max(rounds, 1)
            order = pairs[shift:] + pairs[:shift]
            if r % 2:
                order = order[::-1]
            for p in order:
                n = reps[p]
                for _ in range(2):
                    call(*p)
                ts = []
                for _ in range(batches):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(n):
                        call(*p)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3 / n)
                per_round[p].append(statistics.median(ts))
        row = {"M": M, "N": N, "K": K, "us": {}}
        for (v, c), xs in per_round.items():
            row["us"][f"{NAMES[v]}{c}"] = statistics.median(xs)
        results.append(row)
        best = min(row["us"].items(), key=lambda kv: kv[1])
        log(f"{M}x{N}x{K}: best {best[0]} {best[1]:.2f} us "
            f"({2.0 * M * N * K / best[1] / 1e6:.2f} TFLOP/s)")
        del A, B, C
    return results


def time_calls(calls, rounds=2, batches=5, batch_ms=20.0):
    """Median-of-round-medians microseconds per launch for each named callable, with the
    visiting order rotated (and reversed on odd rounds) from round to round."""
    import torch

    stream = torch.cuda.current_stream()
    names = list(calls)
    reps = {}
    for n in names:
        calls[n]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            calls[n]()
        e1.record(stream)
        torch.cuda.synchronize()
        reps[n] = int(min(20000, max(2, batch_ms / max(e0.elapsed_time(e1) / 3, 1e-4))))
    per_round = {n: [] for n in names}
    for r in range(rounds):
        shift = (r * len(names)) // max(rounds, 1)
        order = names[shift:] + names[:shift]
        if r % 2:
            order = order[::-1]
        for n in order:
            for _ in range(2):
                calls[n]()
            ts = []
            for _ in range(batches):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps[n]):
                    calls[n]()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / reps[n])
            per_round[n].append(statistics.median(ts))
    return {n: statistics.median(v) for n, v in per_round.items()}


def _operands(M, N, K, seed=99):
    import torch

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    A = torch.rand((M, K), device=dev, generator=gen) * 2 - 1
    B = torch.rand((K, N), device=dev, generator=gen) * 2 - 1
    C = torch.empty((M, N), device=dev)
    return A, B, C


def _caller(M, N, K, A, B, C, variant, cfg):
    import torch

    s_ptr = torch.cuda.current_stream().cuda_stream
    pa, pb, pc = A.data_ptr(), B.data_ptr(), C.data_ptr()

    def call():
        rc = tdb.gemm_f32_ex(M, N, K, pa, K, pb, N, pc, N, variant, cfg, s_ptr)
        if rc != tdb.OK:
            raise tdb.GemmError(rc, "gemm_f32_ex")
    return call


BARRIER_SHAPES = [(1024, 1024, 1024), (2048, 2048, 2048), (4096, 4096, 4096),
                  (8192, 8192, 8192), (513, 257, 129)]


def barrier_study(shapes=BARRIER_SHAPES, rounds=2, batches=5, batch_ms=20.0, log=print):
    """Single-buffered with 3 barriers per K tile (copy A | copy B | multiply), with 2
    (copies coalesced) and double-buffered with 1, all at the same tile configuration
    (the single- and the double-buffered column of the table for the shape)."""
    out = []
    for (M, N, K) in shapes:
        A, B, C = _operands(M, N, K)
        cfgs = sorted({tdb.gemm_f32_select_cfg(M, N, K, tdb.VARIANT_SB),
                       tdb.gemm_f32_select_cfg(M, N, K, tdb.VARIANT_DB)})
        for cfg in cfgs:
            _, info = tdb.gemm_f32_config_info(cfg)
            calls = {n: _caller(M, N, K, A, B, C, v, cfg)
                     for n, v in (("sb3", tdb.VARIANT_SB3), ("sb", tdb.VARIANT_SB),
                                  ("db", tdb.VARIANT_DB))}
            us = time_calls(calls, rounds, batches, batch_ms)
            k_tiles = -(-K // info["BK"])
            row = {"M": M, "N": N, "K": K, "cfg": cfg,
                   "tile": f"{info['BM']}x{info['BN']}x{info['BK']}", "k_tiles": k_tiles,
                   "us": us,
                   "barriers": {"sb3": 3 * k_tiles, "sb": 2 * k_tiles, "db": k_tiles},
                   "us_per_removed_barrier_sb3_to_sb": (us["sb3"] - us["sb"]) / k_tiles,
                   "sb_over_db": us["sb"] / us["db"]}
            out.append(row)
            log(f"{M}x{N}x{K} cfg{cfg} {row['tile']}: sb3 {us['sb3']:.2f} us, "
                f"sb {us['sb']:.2f} us, db {us['db']:.2f} us; "
                f"{row['us_per_removed_barrier_sb3_to_sb'] * 1e3:.1f} ns per removed barrier")
        del A, B, C
    return out


def _has_tail(M, N, cus=256):
    """Some configuration a split launch may take (not a one-wave one) cuts M x N into at
    least one full round of tiles plus a partly filled one."""
    for c, (bm, bn, _bk, _lds) in config_dims().items():
        if not _one_wave(c):
            tiles = -(-M // bm) * -(-N // bn)
            if tiles >= cus and tiles % cus:
                return True
    return False


def split_study(shapes=SPLIT_SHAPES, choices=SPLIT_CHOICES, rounds=2, batches=5,
                batch_ms=20.0, log=print):
    """Time gemm_f32_splitk for each split count (1 = the plain dispatched product; -s = the
    tail split into s chunks, where the product has a tail)."""
    import torch

    out = []
    for (M, N, K) in shapes:
        A, B, C = _operands(M, N, K)
        s_ptr = torch.cuda.current_stream().cuda_stream
        # a tail split (-s) is timed where some configuration's tiles make a full round
        # of workgroups and a partly filled one (whichever the model then prefers)
        wsz = tdb.gemm_f32_splitk_workspace
        counts = list(choices)
        if _has_tail(M, N):
            counts += [-sp for sp in choices if sp > 1]
        need = max(wsz(M, N, K, sp) for sp in counts)
        ws = torch.empty(max(need, 1), device=A.device)

        def caller(sp):
            def call():
                rc = tdb.gemm_f32_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                         C.data_ptr(), N, sp, ws.data_ptr(), ws.numel(), s_ptr)
                if rc != tdb.OK:
                    raise tdb.GemmError(rc, "gemm_f32_splitk")
            return call
        us = time_calls({str(sp): caller(sp) for sp in counts}, rounds, batches, batch_ms)
        out.append({"M": M, "N": N, "K": K, "us": us})
        best = min(us, key=us.get)
        log(f"{M}x{N}x{K}: " + ", ".join(f"s{k} {v:.1f}" for k, v in us.items())
            + f" -> splits {best}")
        del A, B, C, ws
    return out


RASTER_SHAPES = [(4096, 4096, 4096), (8192, 8192, 8192), (6144, 6144, 6144)]
RASTER_SETTINGS = ["", "1", "2", "3", "8", "16", "32", "4,noxcd", "8,noxcd", "1,noxcd"]


def raster_study(shapes=RASTER_SHAPES, settings=RASTER_SETTINGS, rounds=2, batches=5,
                 batch_ms=20.0, log=print):
    """The dispatched kernel of each shape under different workgroup orders
    (GEMMF32_RASTER; "" is the built-in default: group 4 with XCD renumbering)."""
    out = []
    for (M, N, K) in shapes:
        A, B, C = _operands(M, N, K)
        _, v, cfg = tdb.gemm_f32_select(M, N, K)
        base = _caller(M, N, K, A, B, C, v, cfg)

        def with_raster(setting):
            def call():
                os.environ["GEMMF32_RASTER"] = setting
                base()
            return call
        calls = {st or "default": with_raster(st) for st in settings}
        try:
            us = time_calls(calls, rounds, batches, batch_ms)
        finally:
            os.environ.pop("GEMMF32_RASTER", None)
        out.append({"M": M, "N": N, "K": K, "variant": v, "cfg": cfg, "us": us})
        best = min(us, key=us.get)
        log(f"{M}x{N}x{K} v{v} cfg{cfg}: " + ", ".join(f"{k} {t:.1f}" for k, t in us.items())
            + f" -> best {best}")
        del A, B, C
    return out


def holdout_shapes(n, seed=2024, lo=5.0, hi=13.0, max_flop=2.0 * 4096 ** 3, exclude=()):
    """n shapes drawn with each of M, N, K log-uniform in [2**lo, 2**hi] (so sizes are
    mostly not multiples of any tile), redrawn while 2MNK exceeds max_flop.  Seeded; none
    of them is a row of the table or in `exclude`."""
    import random

    rng = random.Random(seed)
    out = []
    while len(out) < n:
        m, n_, k = (int(round(2.0 ** rng.uniform(lo, hi))) for _ in range(3))
        if (2.0 * m * n_ * k <= max_flop and (m, n_, k) not in SHAPES
                and (m, n_, k) not in exclude and (m, n_, k) not in out):
            out.append((m, n_, k))
    return out


def decode_shapes(n, seed, exclude=()):
    """n seeded decode products: M uniform in 1..16, N log-uniform in [2**11, 2**15], K
    log-uniform in [2**10, 2**14]; none of them a row of the table or in `exclude`."""
    import random

    rng = random.Random(seed)
    out = []
    while len(out) < n:
        m = rng.randint(1, 16)
        n_ = int(round(2.0 ** rng.uniform(11, 15)))
        k = int(round(2.0 ** rng.uniform(10, 14)))
        s = (m, n_, k)
        if s not in SHAPES and s not in exclude and s not in out:
            out.append(s)
    return out


def train_shapes():
    """The seeded shapes outside the table that the cost model is also fitted to: general
    shapes, and decode products (1-16 rows)."""
    return (holdout_shapes(TRAIN_COUNT, TRAIN_SEED)
            + decode_shapes(DECODE_TRAIN_COUNT, DECODE_TRAIN_SEED))


def holdout_study(n=40, seed=2024, rounds=2, batches=5, batch_ms=20.0, log=print,
                  decode=False):
    """How far the dispatcher's pick is from the best measured (variant, configuration) on
    shapes it was not tuned on: per shape, the time of the dispatched pair over the time of
    the fastest pair (1.0 = the dispatcher found the best).  decode: seeded decode products
    (decode_shapes) instead of general ones."""
    if decode:
        shapes = decode_shapes(n, seed, exclude=set(train_shapes()))
    else:
        shapes = holdout_shapes(n, seed, exclude=set(train_shapes()))
    results = measure(shapes, rounds, batches, batch_ms, log=log)
    out = []
    for r in results:
        M, N, K = r["M"], r["N"], r["K"]
        _, v, cfg = tdb.gemm_f32_select(M, N, K)
        pick = f"{NAMES[v]}{cfg}"
        best = min(r["us"], key=r["us"].get)
        regret = r["us"][pick] / r["us"][best]
        out.append({"M": M, "N": N, "K": K, "pick": pick, "pick_us": r["us"][pick],
                    "best": best, "best_us": r["us"][best], "regret": regret,
                    "us": r["us"]})
        log(f"{M}x{N}x{K}: dispatched {pick} {r['us'][pick]:.2f} us, best {best} "
            f"{r['us'][best]:.2f} us, regret {regret:.3f}")
    regrets = sorted(o["regret"] for o in out)
    summary = {"shapes": len(out), "median": statistics.median(regrets),
               "p90": regrets[int(0.9 * (len(regrets) - 1))], "max": regrets[-1],
               "within_5pct": sum(1 for x in regrets if x <= 1.05) / len(regrets)}
    log(("dispatcher regret on held-out decode shapes: " if decode else
         "dispatcher regret on held-out shapes: ") + json.dumps(summary))
    return {"summary": summary, "rows": out}


# Shapes measured only to fit the cost model (never table rows).
TRAIN_SEED = 1
TRAIN_COUNT = 48
DECODE_TRAIN_SEED = 3
DECODE_TRAIN_COUNT = 16


def model_features(M, N, K, cfg_dims, wg_factor=1, cus=256):
    """rounds * k_tiles of the cost model for a configuration of tile BM x BN x BK."""
    bm, bn, bk = cfg_dims
    tiles = -(-M // bm) * -(-N // bn) * wg_factor
    return -(-tiles // cus) * -(-K // bk)


def model_rounds(M, N, cfg_dims, wg_factor=1, cus=256):
    bm, bn = cfg_dims[0], cfg_dims[1]
    return -(-(-(-M // bm) * -(-N // bn) * wg_factor) // cus)


def model_work(M, N, K, cfg_dims, wg_factor=1, cus=256):
    """workgroups * k_tiles / 256: the launch's tile work spread over every compute unit."""
    bm, bn, bk = cfg_dims[:3]
    return -(-M // bm) * -(-N // bn) * wg_factor * -(-K // bk) / cus


def model_time(row, M, N, K, cfg_dims, wg_factor=1):
    """a + b * rounds + g * rounds * k_tiles + h * work of one fitted row."""
    _v, _c, a, b, g, h = row[:6]
    return (a + b * model_rounds(M, N, cfg_dims, wg_factor)
            + g * model_features(M, N, K, cfg_dims, wg_factor)
            + h * model_work(M, N, K, cfg_dims, wg_factor))


def fit_model(rows, cfg_dims):
    """Per (variant, configuration): (variant id, cfg, a_us, b_us, g_us, h_us, median
    |relative error|) of the cost model a + b * rounds + g * rounds * k_tiles + h * work over
    the measured rows, by non-negative least squares on relative error.  b is fitted for
    the K-split kernels only, whose every round of workgroups ends in a hand-off through LDS
    and a store; it is 0 for the others."""
    import numpy as np
    from scipy.optimize import nnls

    out = []
    ids = IDS
    keys = sorted({k for r in rows for k in r["us"]}, key=lambda k: (ids[k[:2]], int(k[2:])))
    for key in keys:
        cfg = int(key[2:])
        dims = cfg_dims[cfg][:3]
        have = [r for r in rows if key in r["us"]]
        ks = ids[key[:2]] == tdb.VARIANT_KS
        X, ys = [], []
        for r in have:
            y = r["us"][key]
            f = [1.0, model_rounds(r["M"], r["N"], dims),
                 model_features(r["M"], r["N"], r["K"], dims),
                 model_work(r["M"], r["N"], r["K"], dims)]
            if not ks:
                f.pop(1)
            X.append([v / y for v in f])
            ys.append(y)
        coef, _ = nnls(np.array(X), np.ones(len(ys)))
        coef = [float(c) for c in coef]
        if not ks:
            coef.insert(1, 0.0)
        a, b, g, h = coef
        err = statistics.median(abs(model_time((0, cfg, a, b, g, h), r["M"], r["N"], r["K"],
                                               dims) / r["us"][key] - 1.0) for r in have)
        out.append((ids[key[:2]], cfg, a, b, g, h, err))
    return out


def _one_wave(cfg):
    return tdb.gemm_f32_config_info(cfg)[1]["threads"] == 64


def _model_pick_py(M, N, K, model, dims, wg_factor=1):
    """Least modelled (us, variant, cfg) over the fitted rows, as the header computes it
    (a split launch never takes the K-split kernel; with a K tail the multi-stage kernel
    runs the double-buffered loop in a larger LDS allocation and is no candidate)."""
    best = None
    for row in model:
        v, c = row[0], row[1]
        if wg_factor != 1 and (v == tdb.VARIANT_KS or _one_wave(c)):
            continue
        if v == tdb.VARIANT_MS and K % dims[c][2] != 0:
            continue
        t = model_time(row, M, N, K, dims[c][:3], wg_factor)
        if best is None or t < best[0]:
            best = (t, v, c)
    return best


def split_plan(K, splits, granule=64):
    """(K chunk, chunks used) of a split launch, as the library plans it."""
    kc = -(-K // splits)
    kc = max(granule, -(-kc // granule) * granule)
    return kc, -(-K // kc)


def split_extra_mb(M, N, used):
    return (2 * used + 1) * M * N * 4 / 1e6


def split_features(M, N, K, splits, model, dims):
    """(chunks used, modelled GEMM us, [1, extra MB, rounds]) of a split launch; the
    overhead model is the dot product of fitted constants with the list.  splits < 0: the
    tail split (full rounds whole, the tail tiles' chunks priced), with the configuration of
    least modelled GEMM time among those that have a tail; None when none has."""
    kc, used = split_plan(K, abs(splits))
    if splits > 0:
        t, _v, c = _model_pick_py(M, N, kc, model, dims, used)
        bm, bn = dims[c][0], dims[c][1]
        rounds = -(-(-(-M // bm) * -(-N // bn) * used) // 256)
        return used, t, [1.0, split_extra_mb(M, N, used), float(rounds)]
    best = None
    for (v, c, a, b, g, h, _e) in model:
        if v == tdb.VARIANT_KS or _one_wave(c):
            continue
        bm, bn, bk = dims[c][:3]
        tiles = -(-M // bm) * -(-N // bn)
        full = tiles // 256 * 256
        rest = tiles - full
        if full == 0 or rest == 0:
            continue
        tr = -(-(rest * used) // 256)
        kt, kct = -(-K // bk), -(-kc // bk)
        t = (a + b * (full // 256 + tr) + g * (full // 256 * kt + tr * kct)
             + h * (full * kt + rest * used * kct) / 256)
        if best is None or t < best[0]:
            best = (t, [1.0, (2 * used + 1) * rest * bm * bn * 4 / 1e6, float(tr)])
    return (used, best[0], best[1]) if best else None


def fit_split_model(split_results, model, dims):
    """(fixed us, us per extra MB, us per round of workgroups) >= 0 of the split overhead:
    least squares, on error relative to each launch's measured time, of what the measured
    split launches (full and tail) took beyond the modelled GEMM of their chunks.  Relative
    error weighs a small product's second launch as much as a large one's extra traffic:
    the count is chosen by comparing times, whatever their size."""
    import numpy as np
    from scipy.optimize import nnls

    X, y = [], []
    for r in split_results:
        M, N, K = r["M"], r["N"], r["K"]
        for sp, us in r["us"].items():
            f = split_features(M, N, K, int(sp), model, dims)
            if f is not None and f[0] > 1:
                X.append([v / us for v in f[2]])
                y.append((us - f[1]) / us)
    coef, _ = nnls(np.array(X), np.array(y))
    return tuple(float(c) for c in coef)


def config_dims():
    """cfg -> (BM, BN, BK, LDS bytes of the double-buffered loop)."""
    dims = {}
    for c in range(tdb.gemm_f32_num_configs()):
        _, info = tdb.gemm_f32_config_info(c)
        dims[c] = (info["BM"], info["BN"], info["BK"], info["lds_bytes_db"])
    return dims


# Pairs whose times differ by less than this are within run-to-run noise (two tunes on two
# boxes ordered the 256x256 and 256x128 tiles at 8192^3 both ways, 0.2% apart).
TIE_TOLERANCE = 0.005


def _pick(cands, dims):
    """Fastest (name, us) of cands, except that among those within TIE_TOLERANCE of it the
    largest tile wins (fewest bytes fetched per FLOP), then the smallest LDS footprint, then
    the faster: a choice that noise between runs does not flip."""
    fastest = min(v for _, v in cands)
    close = [(k, v) for k, v in cands if v <= fastest * (1.0 + TIE_TOLERANCE)]

    def key(kv):
        bm, bn, _bk, lds = dims[int(kv[0][2:])]
        return (-bm * bn, lds, kv[1])
    return min(close, key=key)


def skinny_shapes(n, seed=2025, max_flop=2.0 * 2048 * 4096 * 4096, exclude=()):
    """n seeded shapes of the split-K regime: few rows against long K (M log-uniform in
    [8, 1024], N in [256, 8192], K in [1024, 16384])."""
    import random

    rng = random.Random(seed)
    out = []
    while len(out) < n:
        m = int(round(2.0 ** rng.uniform(3, 10)))
        n_ = int(round(2.0 ** rng.uniform(8, 13)))
        k = int(round(2.0 ** rng.uniform(10, 14)))
        if 2.0 * m * n_ * k <= max_flop and (m, n_, k) not in SPLIT_SHAPES \
                and (m, n_, k) not in out and (m, n_, k) not in exclude:
            out.append((m, n_, k))
    return out


def _nearest_split_row(M, N, K, split_results):
    """The split count of the nearest measured row in (log2 M, log2 N, log2 K): the rule the
    split model replaced, kept here to measure against."""
    import math

    def d(r):
        return sum((math.log2(a) - math.log2(b)) ** 2
                   for a, b in ((M, r["M"]), (N, r["N"]), (K, r["K"])))
    r = min(split_results, key=d)
    return int(min(r["us"], key=r["us"].get))


def holdout_splitk_study(n=24, seed=2025, rounds=2, batches=5, batch_ms=20.0, log=print,
                         split_results=None):
    """Every split count on n seeded skinny shapes: the time of gemm_f32_splitk_select's
    count over the fastest count (and, given the split study, the same for the nearest-row
    rule)."""
    shapes = skinny_shapes(n, seed, exclude=set(skinny_shapes(SPLIT_TRAIN_COUNT,
                                                              SPLIT_TRAIN_SEED)))
    meas = split_study(shapes, rounds=rounds, batches=batches, batch_ms=batch_ms, log=log)
    rows = []
    for r in meas:
        M, N, K = r["M"], r["N"], r["K"]
        best = min(r["us"], key=r["us"].get)
        pick = str(tdb.gemm_f32_splitk_select(M, N, K))
        row = {"M": M, "N": N, "K": K, "pick": int(pick), "best": int(best),
               "regret": r["us"][pick] / r["us"][best], "us": r["us"]}
        if split_results:
            old = str(_nearest_split_row(M, N, K, split_results))
            row["nearest_row_pick"] = int(old)
            row["nearest_row_regret"] = r["us"][old] / r["us"][best]
        rows.append(row)
        log(f"{M}x{N}x{K}: model picks {pick} ({row['regret']:.3f} of best {best})"
            + (f", nearest row picks {row['nearest_row_pick']} "
               f"({row['nearest_row_regret']:.3f})" if split_results else ""))

    def summ(key):
        xs = sorted(x[key] for x in rows)
        return {"median": statistics.median(xs), "p90": xs[int(0.9 * (len(xs) - 1))],
                "max": xs[-1], "within_5pct": sum(1 for x in xs if x <= 1.05) / len(xs)}
    summary = {"shapes": len(rows), "model": summ("regret")}
    if split_results:
        summary["nearest_row"] = summ("nearest_row_regret")
    log("split-count regret on held-out skinny shapes: " + json.dumps(summary))
    return {"summary": summary, "rows": rows}


def table_rows(results, dims=None):
    dims = dims or config_dims()
    rows = []
    for r in results:
        best = {}
        for name in ("sb", "db", "ms", "ks"):
            cands = [(k, v) for k, v in r["us"].items() if k[:2] == name]
            if cands:
                k, v = _pick(cands, dims)
                best[name] = (int(k[2:]), v)
        win = _pick([(n + str(c), v) for n, (c, v) in best.items()], dims)[0][:2]
        vid = IDS[win]
        ms = best.get("ms", best["db"])
        ks = best.get("ks", (None, None))[1]
        rows.append((r["M"], r["N"], r["K"], vid, best[win][0], best["sb"][0], best["db"][0],
                     ms[0], best["sb"][1], best["db"][1], ms[1], ks))
    return rows


def split_rows(split_results):
    lines = []
    for r in split_results:
        best = min(r["us"], key=lambda k: r["us"][k])
        times = ", ".join(f"{k}: {v:.1f}" for k, v in r["us"].items())
        lines.append(f"    {{{r['M']}, {r['N']}, {r['K']}, {int(best)}}},  // {times}")
    return lines


def write_header(results, device, rounds, batches, batch_ms, path=None, split_results=None,
                 train=None):
    path = path or os.path.join(CSRC, "dispatch_table.h")
    lines = []
    for (m, n, k, v, c, s, d, ms, sb_us, db_us, ms_us, ks_us) in table_rows(results):
        lines.append(f"    {{{m}, {n}, {k}, {v}, {c}, {s}, {d}, {ms}}},  // sb {sb_us:.2f} us, "
                     f"db {db_us:.2f} us, ms {ms_us:.2f} us"
                     + (f", ks {ks_us:.2f} us" if ks_us is not None else ""))
    srows = split_rows(split_results) if split_results else ["    {1024, 1024, 1024, 1},"]
    fit_rows = list(results) + list(train or [])
    dims = config_dims()
    model = fit_model(fit_rows, dims)
    # round as written, so that the split fit sees the model the library will use
    model = [(v, c, round(a, 4), round(b, 4), round(g, 5), round(h, 5), e)
             for (v, c, a, b, g, h, e) in model]
    mrows = [f"    {{{v}, {c}, {a:.4f}, {b:.4f}, {g:.5f}, {h:.5f}}},  "
             f"// median |error| {100 * e:.1f}%"
             for (v, c, a, b, g, h, e) in model]
    r0, per_mb, per_round = (fit_split_model(split_results, model, dims) if split_results
                             else (3.0, 0.3, 1.0))
    choices = sorted({int(k) for r in (split_results or []) for k in r["us"] if int(k) > 0}) or [1]
    text = HEADER_TEMPLATE.format(device=device, rounds=rounds, batches=batches,
                                  batch_ms=int(batch_ms), rows="\n".join(lines),
                                  split_rows="\n".join(srows), model_rows="\n".join(mrows),
                                  nfit=len(fit_rows), ntable=len(results),
                                  ntrain=len(fit_rows) - len(results), split_fixed=r0,
                                  split_us_per_mb=per_mb, split_us_per_round=per_round,
                                  nsplit=len(split_results or []),
                                  split_choices=", ".join(str(c) for c in choices))
    with open(path, "w") as f:
        f.write(text)
    return path


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default=None, help="write the raw measurements (JSON)")
    ap.add_argument("--write-header", action="store_true",
                    help="regenerate csrc/dispatch_table.h from the measurements")
    ap.add_argument("--from-json", default=None,
                    help="regenerate the header from an earlier --out file, no GPU")
    ap.add_argument("--rounds", type=int, default=2)
    ap.add_argument("--batches", type=int, default=5)
    ap.add_argument("--batch-ms", type=float, default=20.0)
    ap.add_argument("--barrier-study", action="store_true",
                    help="time 3-, 2- and 1-barrier loops at equal tile configurations")
    ap.add_argument("--raster-study", action="store_true",
                    help="time the dispatched kernels under different workgroup orders")
    ap.add_argument("--holdout", type=int, default=0, metavar="N",
                    help="time every pair on N seeded shapes outside the table and report "
                         "how far the dispatcher's pick is from the fastest")
    ap.add_argument("--holdout-seed", type=int, default=2024)
    ap.add_argument("--holdout-decode", type=int, default=0, metavar="N",
                    help="as --holdout, on N seeded decode products (1-16 rows)")
    ap.add_argument("--fill", default=None, metavar="BASE_JSON",
                    help="measure the table and training shapes that an earlier --out file "
                         "lacks; write the merged file to --out")
    ap.add_argument("--holdout-splitk", type=int, default=0, metavar="N",
                    help="time every split count on N seeded skinny shapes and report how "
                         "far gemm_f32_splitk_select is from the fastest")
    ap.add_argument("--no-split", action="store_true",
                    help="measure the table and training shapes only (the split study can "
                         "follow with --split-only on the --out file)")
    ap.add_argument("--split-only", default=None, metavar="BASE_JSON",
                    help="re-measure only the split study; the table and training rows "
                         "come from an earlier --out file")
    ap.add_argument("--split-json", default=None,
                    help="an earlier --out file whose split study the nearest-row rule of "
                         "--holdout-splitk is measured against")
    args = ap.parse_args(argv)
    if (args.barrier_study or args.raster_study or args.holdout or args.holdout_splitk
            or args.holdout_decode):
        import torch

        props = torch.cuda.get_device_properties(0)
        res = {"device": f"{props.name} ({getattr(props, 'gcnArchName', '?')})",
               "library": tdb.gemm_f32_version(), "rounds": args.rounds,
               "batches": args.batches, "batch_ms": args.batch_ms}
        if args.barrier_study:
            res["barrier_study"] = barrier_study(rounds=args.rounds, batches=args.batches,
                                                 batch_ms=args.batch_ms,
                                                 log=lambda *a: print(*a, flush=True))
        if args.raster_study:
            res["raster_study"] = raster_study(rounds=args.rounds, batches=args.batches,
                                               batch_ms=args.batch_ms,
                                               log=lambda *a: print(*a, flush=True))
        if args.holdout:
            res["holdout"] = holdout_study(args.holdout, args.holdout_seed, args.rounds,
                                           args.batches, args.batch_ms,
                                           log=lambda *a: print(*a, flush=True))
        if args.holdout_decode:
            res["holdout_decode"] = holdout_study(args.holdout_decode, args.holdout_seed,
                                                  args.rounds, args.batches, args.batch_ms,
                                                  log=lambda *a: print(*a, flush=True),
                                                  decode=True)
        if args.holdout_splitk:
            prior = None
            if args.split_json:
                with open(args.split_json) as f:
                    prior = json.load(f).get("splits")
            res["holdout_splitk"] = holdout_splitk_study(
                args.holdout_splitk, rounds=args.rounds, batches=args.batches,
                batch_ms=args.batch_ms, log=lambda *a: print(*a, flush=True),
                split_results=prior)
        if args.out:
            with open(args.out, "w") as f:
                json.dump(res, f, indent=1)
        return 0
    if args.from_json:
        with open(args.from_json) as f:
            data = json.load(f)
        print(write_header(data["results"], data["device"], data["rounds"], data["batches"],
                           data["batch_ms"], split_results=data.get("splits"),
                           train=data.get("train")))
        return 0
    if args.fill:
        with open(args.fill) as f:
            data = json.load(f)
        have = {(r["M"], r["N"], r["K"]) for r in data["results"] + (data.get("train") or [])}
        log = lambda *a: print(*a, flush=True)  # noqa: E731
        data["results"] = [r for r in data["results"] if (r["M"], r["N"], r["K"]) in SHAPES] + \
            measure([s for s in SHAPES if s not in have], args.rounds, args.batches,
                    args.batch_ms, log=log)
        train_set = set(train_shapes())
        data["train"] = [r for r in (data.get("train") or [])
                         if (r["M"], r["N"], r["K"]) in train_set] + measure(
            [s for s in train_shapes() if s not in have], args.rounds, args.batches,
            args.batch_ms, log=log)
        data["library"] = tdb.gemm_f32_version()
        if args.out:
            with open(args.out, "w") as f:
                json.dump(data, f, indent=1)
        return 0
    import torch

    props = torch.cuda.get_device_properties(0)
    device = f"{props.name} ({getattr(props, 'gcnArchName', '?')})"
    t0 = time.time()
    if args.split_only:
        with open(args.split_only) as f:
            base = json.load(f)
        results, train = base["results"], base.get("train")
    else:
        results = measure(SHAPES, args.rounds, args.batches, args.batch_ms,
                          log=lambda *a: print(*a, flush=True))
        train = measure(train_shapes(), args.rounds, args.batches, args.batch_ms,
                        log=lambda *a: print(*a, flush=True))
    splits = [] if args.no_split else split_study(
        SPLIT_SHAPES + TAIL_SHAPES + skinny_shapes(SPLIT_TRAIN_COUNT, SPLIT_TRAIN_SEED),
        rounds=args.rounds, batches=args.batches, batch_ms=args.batch_ms,
        log=lambda *a: print(*a, flush=True))
    data = {"device": device, "rounds": args.rounds, "batches": args.batches,
            "batch_ms": args.batch_ms, "library": tdb.gemm_f32_version(),
            "seconds": time.time() - t0, "results": results, "train": train,
            "splits": splits}
    if args.out:
        with open(args.out, "w") as f:
            json.dump(data, f, indent=1)
    if args.write_header:
        print(write_header(results, device, args.rounds, args.batches, args.batch_ms,
                           split_results=splits, train=train))
    return 0


if __name__ == "__main__":
    sys.exit(main())
