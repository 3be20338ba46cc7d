#!/usr/bin/env python3
"""Benchmark of the FP32 GEMM C = A.B on one MI355X.

One step = one 8192 x 8192 x 8192 product through the dispatched C-ABI entry point
(gemm_f32): dispatcher -> tiled kernel (global -> LDS copy, LDS ping-pong or single slot,
FP32 MFMA micro-kernel, guarded epilogue).  Inputs are the seeded uniform grid values of
tdb_inputs, resident in HBM before timing starts; C is preallocated.

Prints ONE JSON line:
  value         whole-job TFLOP/s = 2*M*N*K / (host-wall time per step), K timed steps
                bracketed by torch.cuda.synchronize()
  roofline      FP32 MFMA bound: algorithmic FLOP per launch / average launch duration
                from HIP events on the launch stream, against the 157.3 TFLOP/s peak;
                `traffic` = HBM bytes per launch from the committed rocprofv3 counter
                summary (null if the kernel source changed since it was taken)
  cpu_baseline  the CPU oracle timed on a bounded row sample of the same product
  mfma_ceiling  the matrix-core ceiling at the clock the device sustains (a kernel of
                nothing but FP32 MFMAs) and the headline's fraction of it
  per_shape     single-buffered, double-buffered, multi-stage and dispatched time for
                every workload shape, with torch.matmul (FP32, black box) as context
  parity        the 8192^3 result checked on 4096 seeded positions against the oracle

Also:
  python bench.py --oracle-table             the CPU oracle's time per workload on all host
                                             threads and on one (no GPU needed)
  python bench.py --summarize-trace DIR      per-(kernel, grid) average durations from a
                                             rocprofv3 kernel trace (kernel_trace.csv)
  python bench.py --summarize-counters DIR   per-(kernel, grid) average counter values
                                             from rocprofv3 --pmc runs (counter_collection.csv)
  --copy-calibration MIB                     first run one streaming elementwise kernel
                                             (negate) that reads MIB MiB and writes MIB MiB;
                                             its FETCH_SIZE / WRITE_SIZE readings calibrate
                                             the GEMM's HBM byte counts
  python bench.py --counter-run              a few SB, DB and MS launches per
                                             metric shape (1024^3, 4096^3, 8192^3) plus the
                                             calibration kernel: the program that the
                                             rocprofv3 --pmc passes profile
  python bench.py --counter-run-skinny       the K-split kernel at 16x4096x4096 and, with
                                             the same per-wave work, the 64x64x32 DB tile at
                                             1024^3 (three launches each), plus the
                                             calibration kernel: the program of the K-split
                                             kernel's counter passes
  python bench.py --write-traffic FETCH_DIR WRITE_DIR
                                             HBM bytes per launch of the headline kernel from
                                             a FETCH_SIZE pass and a WRITE_SIZE pass of
                                             --counter-run, scaled by the calibration
                                             kernel's readings; writes
                                             profiles/traffic_square_8192.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3          # MI355X dense FP32 matrix peak (AMD specification)
METRIC = "FP32 GEMM TFLOP/s and % of MFMA FP32 peak at 1024³/4096³/8192³, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_square_8192.json")
HEADLINE = "square_8192"
VARIANT_NAMES = {1: "sb", 2: "db", 3: "ms", 5: "ks"}


def kernel_source_hash() -> str:
    """SHA-256 over the library's sources and headers (the files its build compiles)."""
    from tiled_double_buffered_amd import build
    h = hashlib.sha256()
    for p in build.DEPS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def summarize_trace(d: str) -> int:
    """Average kernel duration per (kernel name, grid size) from rocprofv3's CSV trace."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        print(f"no kernel_trace.csv under {d}", file=sys.stderr)
        return 1
    groups = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                grid = row.get("Grid_Size", row.get("Grid_Size_X", ""))
                dur = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
                groups.setdefault((name, grid), []).append(dur)
    print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  grid  kernel")
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"{len(v):6d} {statistics.mean(v)/1e3:10.2f} {min(v)/1e3:10.2f} "
              f"{max(v)/1e3:10.2f}  {grid}  {name[:150]}")
    return 0


def summarize_counters(d: str) -> int:
    """Average counter value per (kernel name, grid size, counter) from rocprofv3 --pmc."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        print(f"no counter_collection.csv under {d}", file=sys.stderr)
        return 1
    groups = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                key = (row.get("Kernel_Name", ""), row.get("Grid_Size", ""),
                       row.get("Counter_Name", ""))
                groups.setdefault(key, {}).setdefault(row.get("Dispatch_Id", ""), 0.0)
                groups[key][row.get("Dispatch_Id", "")] += float(row["Counter_Value"])
    print(f"{'dispatches':>10} {'avg_value':>16}  counter  grid  kernel")
    for (name, grid, ctr), per in sorted(groups.items()):
        vals = list(per.values())
        print(f"{len(vals):10d} {statistics.mean(vals):16.4f}  {ctr}  {grid}  {name[:140]}")
    return 0


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for fn in files:
        with open(fn) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter, match):
    """Average over dispatches of one counter (summed over its instances) for the
    dispatches whose (kernel name, grid size) satisfy `match`."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not match(r.get("Kernel_Name", ""),
                                                         r.get("Grid_Size", "")):
            continue
        per[r.get("Dispatch_Id")] = per.get(r.get("Dispatch_Id"), 0.0) + float(r["Counter_Value"])
    return (statistics.mean(per.values()), len(per)) if per else (None, 0)


def write_traffic(fetch_dir: str, write_dir: str, calib_mib: int = 512) -> int:
    import tdb_inputs as ti
    import tiled_double_buffered_amd as tdb

    M, N, K, _ = ti.WORKLOADS[HEADLINE]
    _, variant, cfg = tdb.gemm_f32_select(M, N, K)
    _, info = tdb.gemm_f32_config_info(cfg)
    grid = str(((M + info["BM"] - 1) // info["BM"]) * ((N + info["BN"] - 1) // info["BN"])
               * info["threads"])
    tag = f"TileCfg<{info['BM']}, {info['BN']}, {info['BK']},"
    if variant == tdb.VARIANT_MS:
        kname, flag = "gemm_f32_ms_kernel", ">, %d>" % tdb.gemm_f32_config_ms(cfg)[1]["stages"]
    else:
        kname, flag = "gemm_f32_tile_kernel", ", %d>" % variant  # loop kind = variant id

    def is_gemm(name, g):
        return kname in name and tag in name and flag in name and g == grid

    def is_calib(name, g):
        return "neg" in name.lower() and "gemm" not in name

    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    g_fetch, nf = _per_dispatch(fr, "FETCH_SIZE", is_gemm)
    g_write, nw = _per_dispatch(wr, "WRITE_SIZE", is_gemm)
    c_fetch, _ = _per_dispatch(fr, "FETCH_SIZE", is_calib)
    c_write, _ = _per_dispatch(wr, "WRITE_SIZE", is_calib)
    if None in (g_fetch, g_write, c_fetch, c_write):
        print("missing counter rows (gemm fetch/write, calibration fetch/write): "
              f"{g_fetch} {g_write} {c_fetch} {c_write}", file=sys.stderr)
        return 1
    kib = calib_mib * 1024.0
    sf, sw = kib / c_fetch, kib / c_write
    fetch_b = g_fetch * sf * 1024.0
    write_b = g_write * sw * 1024.0
    algo = 4.0 * (M * K + K * N + M * N)
    out = {
        "workload": HEADLINE,
        "kernel": f"{VARIANT_NAMES[variant]} cfg{cfg} "
                  f"{info['BM']}x{info['BN']}x{info['BK']}",
        "kernel_source_sha256": kernel_source_hash(),
        "fetch_kib_per_launch_raw": g_fetch, "write_kib_per_launch_raw": g_write,
        "dispatches": [nf, nw],
        "calibration": {"kernel": "torch negate, reads and writes %d MiB" % calib_mib,
                        "fetch_kib_raw": c_fetch, "write_kib_raw": c_write,
                        "fetch_scale": sf, "write_scale": sw},
        "hbm_fetch_bytes_per_launch": fetch_b,
        "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": (fetch_b + write_b) / algo,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -f csv -d <FETCH_DIR> -o run -- "
            "python3 bench.py --counter-run --copy-calibration %d" % calib_mib,
            "rocprofv3 --pmc WRITE_SIZE -f csv -d <WRITE_DIR> -o run -- "
            "python3 bench.py --counter-run --copy-calibration %d" % calib_mib,
            "python3 bench.py --write-traffic <FETCH_DIR> <WRITE_DIR>"],
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def counter_run(calib_mib: int) -> int:
    """A short program for counter passes: a few launches of each variant (dispatch-table
    configurations) at the three metric shapes."""
    import torch

    import tdb_inputs as ti
    import tiled_double_buffered_amd as tdb

    dev = torch.device("cuda:0")
    if calib_mib > 0:
        n = calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    s_ptr = torch.cuda.current_stream(dev).cuda_stream
    for name in ("square_1024", "square_4096", "square_8192"):
        M, N, K, seed = ti.WORKLOADS[name]
        a, b = ti.workload_inputs(M, N, K, seed)
        A, B = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
        C = torch.empty((M, N), device=dev)
        for fn in (tdb.gemm_f32_sb, tdb.gemm_f32_db, tdb.gemm_f32_ms):
            for _ in range(3):
                rc = fn(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N, s_ptr)
                if rc != tdb.OK:
                    raise tdb.GemmError(rc, fn.__name__)
        torch.cuda.synchronize()
        print(f"[counter-run] {name} done", file=sys.stderr, flush=True)
        del A, B, C
    return 0


def counter_run_skinny(calib_mib: int) -> int:
    """A short program for counter passes of the K-split kernel: three launches at
    16 x 4096 x 4096 (variant KS, configuration 13) and three of the 64 x 64 x 32 DB tile
    (configuration 6) at 1024^3, whose four waves each walk the same 32 K tiles of one
    32 x 32 block."""
    import torch

    import tdb_inputs as ti
    import tiled_double_buffered_amd as tdb

    dev = torch.device("cuda:0")
    if calib_mib > 0:
        n = calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    s_ptr = torch.cuda.current_stream(dev).cuda_stream
    for (M, N, K, variant, cfg, seed) in [(16, 4096, 4096, tdb.VARIANT_KS, 13, 7101),
                                          (1024, 1024, 1024, tdb.VARIANT_DB, 6, 7102)]:
        a, b = ti.workload_inputs(M, N, K, seed)
        A, B = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
        C = torch.empty((M, N), device=dev)
        for _ in range(3):
            rc = tdb.gemm_f32_ex(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                                 variant, cfg, s_ptr)
            if rc != tdb.OK:
                raise tdb.GemmError(rc, "gemm_f32_ex")
        torch.cuda.synchronize()
        print(f"[counter-run-skinny] {M}x{N}x{K} variant {variant} cfg {cfg} done",
              file=sys.stderr, flush=True)
        del A, B, C
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--per-shape", choices=("all", "metric", "none"), default="all",
                    help="which workload shapes get the SB/DB/dispatch comparison")
    ap.add_argument("--rounds", type=int, default=2,
                    help="per-shape timing: rounds, each visiting the variants in rotated order")
    ap.add_argument("--batches", type=int, default=5, help="per-shape timing: batches per round")
    ap.add_argument("--batch-ms", type=float, default=25.0,
                    help="per-shape timing: minimum milliseconds of launches per batch")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 = skip)")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--counter-run", action="store_true")
    ap.add_argument("--counter-run-skinny", action="store_true")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--oracle-table", action="store_true")
    args = ap.parse_args()

    if args.oracle_table:
        return oracle_table()

    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.counter_run:
        return counter_run(args.copy_calibration)
    if args.counter_run_skinny:
        return counter_run_skinny(args.copy_calibration)

    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tdb_inputs as ti
    import tiled_double_buffered_amd as tdb

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    lib_version = tdb.gemm_f32_version()
    torch.backends.cuda.matmul.allow_tf32 = False  # the torch.matmul context stays FP32

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # reads and writes exactly MIB MiB each
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration} MiB done")
        del src, dst

    # ------------------------------------------------------------------ headline
    M, N, K, seed = ti.WORKLOADS[HEADLINE]
    log(f"[bench] generating {M}x{N}x{K} inputs (seed {seed}) ...")
    A_h, B_h = ti.workload_inputs(M, N, K, seed)
    A = torch.from_numpy(A_h).to(dev)
    B = torch.from_numpy(B_h).to(dev)
    C = torch.zeros((M, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    s_ptr = stream.cuda_stream
    flop = 2.0 * M * N * K
    _, variant, cfg = tdb.gemm_f32_select(M, N, K)

    def step():
        rc = tdb.gemm_f32(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N, s_ptr)
        if rc != tdb.OK:
            raise tdb.GemmError(rc, "gemm_f32")

    log(f"[bench] warmup {args.warmup} steps (variant {variant}, cfg {cfg}) ...")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = e0.elapsed_time(e1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    log(f"[bench] {HEADLINE}: {ms_per_step:.3f} ms/step wall, {kernel_ms:.3f} ms/launch "
        f"(events) -> {value:.2f} TFLOP/s")

    # parity of the timed output on the workload's seeded positions
    parity = None
    try:
        import oracle
        ri, rj = ti.sample_positions(seed, M, N, 4096)
        c64, bnd = oracle.gemm_f64_sampled(A_h, B_h, ri, rj)
        got = C[torch.from_numpy(ri).to(dev), torch.from_numpy(rj).to(dev)].cpu().numpy()
        r = oracle.tolerance_ratio(got, c64, bnd)
        parity = {"positions": 4096, "max_err_over_bound": r, "pass": bool(r <= 1.0)}
        log(f"[bench] parity on 4096 positions: max |C-C64|/(1e-5*Bnd+1e-6) = {r:.3g}")
    except Exception as exc:  # the oracle is test infrastructure; report, do not fail
        parity = {"error": repr(exc)}

    # traffic from the committed counter summary, if it describes this kernel source
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256") == kernel_source_hash() and \
                tr.get("workload") == HEADLINE:
            traffic = tr["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    roofline = {"bound": "mfma", "achieved": round(achieved, 3),
                "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": traffic,
                "kernel": f"{VARIANT_NAMES[variant]} cfg{cfg}",
                "launch_ms": round(kernel_ms, 4)}

    # the matrix-core ceiling at the clock this device sustains, measured right after the
    # headline so that both run warm
    try:
        from tiled_double_buffered_amd import peak
        ceiling = peak.mfma_ceiling(stream=stream)
        ceiling["headline_frac"] = round(achieved / ceiling["value"], 4)
        log(f"[bench] matrix-core ceiling {ceiling['value']} TFLOP/s at "
            f"{ceiling['clock_ghz']} GHz; headline at {ceiling['headline_frac']:.3f} of it")
    except Exception as exc:
        ceiling = {"error": repr(exc)}

    # power, clocks and temperatures while the headline kernel runs (amd-smi, sampled once)
    telemetry = telemetry_under_load(step, torch)
    log(f"[bench] telemetry under load: {telemetry}")

    # ------------------------------------------------------------------ per shape
    def time_call(fn, target_ms=args.batch_ms, batches=args.batches):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        one = max(time.perf_counter() - t, 1e-6)
        reps = int(min(5000, max(3, target_ms * 1e-3 / one)))
        for _ in range(min(reps, 10)):
            fn()
        res = []
        for _ in range(batches):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            h0 = time.perf_counter()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            h1 = time.perf_counter()
            res.append((a.elapsed_time(b) * 1e3 / reps, (h1 - h0) * 1e6 / reps))
        ev = statistics.median(x[0] for x in res)
        wall_us = statistics.median(x[1] for x in res)
        return ev, wall_us, min(x[0] for x in res), max(x[0] for x in res)

    # the oracle for each per-shape workload, to check every timed variant once per round
    def shape_checker(name, m, n, k, s, a_h, b_h):
        try:
            import oracle
        except Exception as exc:  # the oracle is test infrastructure; report, do not fail
            return lambda C: {"error": repr(exc)}
        if m * n * k <= 4096 ** 3:
            c64, bnd = oracle.gemm_f64(a_h, b_h)
            return lambda C: oracle.tolerance_ratio(C.cpu().numpy(), c64, bnd)
        ri, rj = ti.sample_positions(s, m, n, 4096)
        c64, bnd = oracle.gemm_f64_sampled(a_h, b_h, ri, rj)
        ii, jj = torch.from_numpy(ri).to(dev), torch.from_numpy(rj).to(dev)
        return lambda C: oracle.tolerance_ratio(C[ii, jj].cpu().numpy(), c64, bnd)

    per_shape = {}
    names = {"all": list(ti.WORKLOADS), "none": [],
             "metric": ["square_1024", "square_4096", "square_8192"]}[args.per_shape]
    rounds = args.rounds
    for name in names:
        m, n, k, s = ti.WORKLOADS[name]
        if name == HEADLINE:
            Ad, Bd, Cd = A, B, C
            a_h, b_h = A_h, B_h
        else:
            a_h, b_h = ti.workload_inputs(m, n, k, s)
            Ad, Bd = torch.from_numpy(a_h).to(dev), torch.from_numpy(b_h).to(dev)
            Cd = torch.zeros((m, n), dtype=torch.float32, device=dev)
        check = shape_checker(name, m, n, k, s, a_h, b_h)
        pa, pb, pc = Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr()
        fns = {
            "sb": lambda: tdb.gemm_f32_sb(m, n, k, pa, k, pb, n, pc, n, s_ptr),
            "db": lambda: tdb.gemm_f32_db(m, n, k, pa, k, pb, n, pc, n, s_ptr),
            "ms": lambda: tdb.gemm_f32_ms(m, n, k, pa, k, pb, n, pc, n, s_ptr),
            "dispatch": lambda: tdb.gemm_f32(m, n, k, pa, k, pb, n, pc, n, s_ptr),
            # context only: the vendor library through torch, timed as a black box
            "torch": lambda: torch.matmul(Ad, Bd, out=Cd),
        }
        order = list(fns)
        samples = {v: [] for v in fns}
        checks = {v: [] for v in fns if v != "torch"}
        for r in range(rounds):  # rotate the variant order between rounds
            rot = r % len(order)
            for v in order[rot:] + order[:rot]:
                samples[v].append(time_call(fns[v]))
            for v in checks:  # every timed variant of the library, once per round
                Cd.fill_(float("nan"))
                fns[v]()
                torch.cuda.synchronize()
                checks[v].append(check(Cd))
        f = 2.0 * m * n * k
        entry = {"M": m, "N": n, "K": k}
        for v, xs in samples.items():
            ev = statistics.median(x[0] for x in xs)  # median of the per-round medians
            wl = statistics.median(x[1] for x in xs)
            entry[v] = {"us": round(ev, 2), "host_wall_us": round(wl, 2),
                        "us_range": [round(min(x[2] for x in xs), 2),
                                     round(max(x[3] for x in xs), 2)],
                        "tflops": round(f / (ev * 1e-6) / 1e12, 2),
                        "frac_peak": round(f / (ev * 1e-6) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4)}
            if v in checks:
                cs = checks[v]
                entry[v]["max_err_over_bound"] = (max(cs) if all(isinstance(c, float)
                                                                   for c in cs) else cs[0])
        entry["sb_cfg"] = tdb.gemm_f32_select_cfg(m, n, k, tdb.VARIANT_SB)
        entry["db_cfg"] = tdb.gemm_f32_select_cfg(m, n, k, tdb.VARIANT_DB)
        entry["ms_cfg"] = tdb.gemm_f32_select_cfg(m, n, k, tdb.VARIANT_MS)
        _, dv, dc = tdb.gemm_f32_select(m, n, k)
        entry["dispatch_choice"] = f"{VARIANT_NAMES[dv]} cfg{dc}"
        entry["db_over_sb_speedup"] = round(entry["sb"]["us"] / entry["db"]["us"], 3)
        entry["ms_over_db_speedup"] = round(entry["db"]["us"] / entry["ms"]["us"], 3)
        entry["dispatch_over_torch_speedup"] = round(entry["torch"]["us"] /
                                                     entry["dispatch"]["us"], 3)
        per_shape[name] = entry
        log(f"[bench] {name}: sb {entry['sb']['us']} us, db {entry['db']['us']} us, "
            f"ms {entry['ms']['us']} us, dispatch {entry['dispatch']['us']} us "
            f"({entry['dispatch']['tflops']} TFLOP/s), torch.matmul {entry['torch']['us']} us")
        if name != HEADLINE:
            del Ad, Bd, Cd
        del check

    # ------------------------------------------------------------------ CPU baseline
    cpu_baseline = None
    if args.cpu_seconds > 0:
        try:
            import oracle
            threads = oracle.max_threads()
            # successive row blocks of the product until the time budget is spent; the
            # block size comes from a pilot block so that the last one overshoots little
            t = time.perf_counter()
            oracle.gemm_f64(A_h[:threads], B_h)
            pilot = time.perf_counter() - t
            block = int(min(M, max(threads, threads * round(args.cpu_seconds / 8 / pilot))))
            rows, dt = 0, 0.0
            while rows < M and dt < args.cpu_seconds:
                r1 = min(M, rows + block)
                t = time.perf_counter()
                oracle.gemm_f64(A_h[rows:r1], B_h)
                dt += time.perf_counter() - t
                rows = r1
            cpu_tflops = 2.0 * rows * N * K / dt / 1e12
            cpu_baseline = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s",
                            "cores": threads, "kind": "oracle",
                            "sample": f"first {rows} rows of the {M}x{N}x{K} product "
                                      f"(C64 and Bnd in FP64, {dt:.1f} s); full product "
                                      f"extrapolates to {flop / (cpu_tflops * 1e12):.0f} s",
                            "cpu": _cpu_model()}
            log(f"[bench] CPU oracle: {rows} rows in {dt:.1f} s on {threads} threads")
        except Exception as exc:
            cpu_baseline = {"error": repr(exc)}

    metric_shapes = {}
    for name in ("square_1024", "square_4096", "square_8192"):
        if name in per_shape:
            d = per_shape[name]["dispatch"]
            metric_shapes[name] = {"tflops": d["tflops"], "frac_peak": d["frac_peak"]}

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "M": M, "N": N, "K": K, "seed": seed,
                   "inputs": "uniform grid values in [-1, 1) (SplitMix64)",
                   "dispatch": roofline["kernel"], "library": lib_version},
        "frac_peak": round(value / PEAK_FP32_MFMA_TFLOPS, 4),
        "roofline": roofline,
        "mfma_ceiling": ceiling,
        "telemetry": telemetry,
        "cpu_baseline": cpu_baseline,
        "metric_shapes": metric_shapes,
        "per_shape": per_shape,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)
    return 0


def oracle_table() -> int:
    """Time the CPU oracle (C64 and Bnd in FP64) on every workload, in full up to 4096^3
    and on the 4096 seeded positions at 8192^3, on all host threads and on one thread.
    Prints one JSON object; needs no GPU."""
    import oracle
    import tdb_inputs as ti
    threads = oracle.max_threads()
    rows = []
    for name, (m, n, k, seed) in ti.WORKLOADS.items():
        a, b = ti.workload_inputs(m, n, k, seed)
        full = m * n * k <= 4096 ** 3
        row = {"workload": name, "M": m, "N": n, "K": k,
               "what": "full product" if full else "4096 seeded positions"}
        for t in (threads, 1):
            oracle.set_threads(t)
            t0 = time.perf_counter()
            if full:
                oracle.gemm_f64(a, b)
            else:
                ri, rj = ti.sample_positions(seed, m, n, 4096)
                oracle.gemm_f64_sampled(a, b, ri, rj)
            row[f"seconds_{t}_threads"] = round(time.perf_counter() - t0, 4)
        rows.append(row)
        print(f"[oracle] {row}", file=sys.stderr, flush=True)
    oracle.set_threads(threads)
    print(json.dumps({"cpu": _cpu_model(), "threads": threads, "rows": rows}), flush=True)
    return 0


def telemetry_under_load(step, torch, timeout_s: float = 20.0) -> dict:
    """One amd-smi sample of socket power, shader clocks (per XCD) and temperatures, taken
    while `step` keeps the GPU busy.  amd-smi runs as a child process; nothing is timed
    meanwhile.  Returns {"error": ...} when amd-smi is missing or fails."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi")
    if exe is None:
        return {"error": "amd-smi not found"}
    try:
        proc = subprocess.Popen([exe, "metric", "-g", "0", "-p", "-c", "-t", "--json"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL)
    except OSError as exc:
        return {"error": repr(exc)}
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < timeout_s:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    try:
        out, _ = proc.communicate(timeout=5)
    except subprocess.TimeoutExpired:
        proc.kill()
        proc.communicate()
        return {"error": "amd-smi timed out"}
    try:
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clocks = [v["clk"]["value"] for k, v in sorted(g["clock"].items())
                  if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        temps = {k: v["value"] for k, v in g.get("temperature", {}).items()
                 if isinstance(v, dict) and "value" in v}
        return {"socket_power_w": g["power"]["socket_power"]["value"],
                "gfx_clock_mhz_per_xcd": clocks, "temperature_c": temps,
                "source": "amd-smi metric -g 0 -p -c -t, sampled during headline launches"}
    except (ValueError, KeyError, IndexError, TypeError) as exc:
        return {"error": "unparsed amd-smi output: " + repr(exc)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())
