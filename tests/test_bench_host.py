"""bench.py on the host: the parity gate that keeps a wrong product from publishing a
throughput, the trace summary the roofline figure is read from, and the refusal of
more than one GPU.  No GPU needed."""
import io
import json
import os
import sys
from contextlib import redirect_stdout

import numpy as np
import pytest

import bench


def _entry(r=0.01):
    return {v: {"us": 1.0, "max_err_over_bound": r}
            for v in ("sb", "db", "ms", "dispatch", "pair_sb", "pair_db")} | \
        {"torch": {"us": 1.0}}


def _line(**per_shape):
    return {"parity": {"positions": 4096, "max_err_over_bound": 0.02, "pass": True},
            "per_shape": per_shape}


def test_gate_passes_only_when_every_check_passed():
    assert bench.line_parity_ok(_line(a=_entry(), b=_entry(1.0)))
    assert not bench.line_parity_ok(_line(a=_entry(), b=_entry(1.0000001)))
    assert not bench.line_parity_ok(_line(a=_entry(float("inf"))))
    assert not bench.line_parity_ok(_line(a=_entry(float("nan"))))
    # a check that could not run (an error record, or one error among the rounds)
    assert not bench.line_parity_ok(_line(a=_entry({"error": "no oracle"})))
    assert not bench.line_parity_ok(_line(a=_entry([0.01, {"error": "x"}])))
    # a column without its recorded check
    e = _entry()
    del e["pair_db"]["max_err_over_bound"]
    assert not bench.line_parity_ok(_line(a=e))
    # the headline check failed, or never ran
    line = _line(a=_entry())
    line["parity"] = {"positions": 4096, "max_err_over_bound": 3.0, "pass": False}
    assert not bench.line_parity_ok(line)
    line["parity"] = {"error": "RuntimeError()", "pass": False}
    assert not bench.line_parity_ok(line)
    del line["parity"]
    assert not bench.line_parity_ok(line)
    # torch.matmul is context, never checked
    assert bench.line_parity_ok(_line(a=_entry()))


class _FakeOracle:
    """Stands in for the oracle module: every comparison returns a fixed ratio."""

    def __init__(self, ratio):
        self.ratio = ratio

    def gemm_f64(self, a, b):
        return np.zeros((a.shape[0], b.shape[1])), np.ones((a.shape[0], b.shape[1]))

    def gemm_f64_sampled(self, a, b, ri, rj):
        return np.zeros(len(ri)), np.ones(len(ri))

    def tolerance_ratio(self, C, c64, bnd):
        return self.ratio


class _FakeTensor:
    def __init__(self, shape):
        self.shape = shape

    def cpu(self):
        return self

    def numpy(self):
        return np.zeros(self.shape, dtype=np.float32)


@pytest.mark.parametrize("ratio,ok", [(0.5, True), (1.0, True), (1.5, False),
                                      (float("inf"), False)])
def test_cpu_leg_checker_feeds_the_gate(ratio, ok):
    """The checkers the bench builds report the oracle's ratio unchanged, and a line built
    from them passes the gate exactly when every ratio is at most 1."""
    leg = bench.CpuLeg()
    leg.oracle, leg.error = _FakeOracle(ratio), None
    a = np.zeros((8, 4), dtype=np.float32)
    b = np.zeros((4, 8), dtype=np.float32)
    check = leg.full_or_sampled(None, None, None, 8, 8, 4, 1, a, b)
    r = check(_FakeTensor((8, 8)))
    assert r == ratio
    assert bench.line_parity_ok(_line(a=_entry(r))) is ok


def test_missing_oracle_fails_the_gate():
    leg = bench.CpuLeg()
    leg.oracle, leg.error = None, "ModuleNotFoundError('oracle')"
    r = leg.full_or_sampled(None, None, None, 8, 8, 4, 1, None, None)(None)
    assert isinstance(r, dict) and "error" in r
    assert not bench.line_parity_ok(_line(a=_entry(r)))
    assert "error" in leg.baseline(None, None, 1.0)


def test_trace_summary_reports_median_and_steady_launches(tmp_path):
    """Median and minimum per (kernel, grid), and the median without the first tenth of the
    launches (the clock ramps over those): one slow first launch moves the mean, not them."""
    rows = ["Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp"]
    t = 0
    for i in range(20):
        dur = 9000 if i == 0 else 7000 + (i % 3)
        rows.append(f"\"k<1>\",65536,{t},{t + dur}")
        t += dur + 5
    (tmp_path / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    groups, found = bench.trace_groups(str(tmp_path))
    assert found and len(groups[("k<1>", "65536")]) == 20
    out = io.StringIO()
    with redirect_stdout(out):
        assert bench.summarize_trace(str(tmp_path)) == 0
    fields = out.getvalue().splitlines()[1].split()
    calls, median, steady_med, mn, mean, mx = fields[:6]
    assert int(calls) == 20
    assert float(median) == pytest.approx(7.0, abs=0.01)
    assert float(steady_med) == pytest.approx(7.0, abs=0.01)
    assert float(mn) == pytest.approx(7.0)
    assert float(mx) == pytest.approx(9.0)
    assert float(mean) > float(median)
    assert bench.steady([5, 1, 1, 1]) == [1, 1, 1]
    assert bench.steady([5, 1]) == [5, 1]


def test_more_than_one_gpu_is_refused(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2


def test_layer_shapes_are_decode_and_layer_products():
    assert all(m in (1, 8, 16, 128, 512, 4096) for m, _, _ in bench.LAYER_SHAPES)
    assert (16, 4096, 4096) in bench.LAYER_SHAPES and (1, 4096, 4096) in bench.LAYER_SHAPES


def test_timed_headline_summary_takes_exactly_the_timed_steps(tmp_path):
    """The traced run's line says how many headline launches precede its timed steps; the
    summary takes those steps only, not the warm-up and the later per-shape launches."""
    import tiled_double_buffered_amd as tdb
    _, v, c = tdb.gemm_f32_select(8192, 8192, 8192)
    if v not in (tdb.VARIANT_SB, tdb.VARIANT_DB):
        pytest.skip("the headline is not a register-staged kernel")
    _, i = tdb.gemm_f32_config_info(c)
    name = (f"void gemmf32::gemm_f32_tile_kernel<gemmf32::TileCfg<{i['BM']}, {i['BN']}, "
            f"{i['BK']}, 2, 2>, {v}>(int, int, int)")
    grid = (8192 // i["BM"]) * (8192 // i["BN"]) * i["threads"]
    first, steps = 7, 5
    durs = [9000] * first + [7000, 7002, 7001, 7003, 7004] + [8000] * 20
    rows = ["Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp"]
    t = 0
    for d in durs:
        rows.append(f"\"{name}\",{grid},{t},{t + d * 1000}")
        t += d * 1000 + 10
    rows.append(f"\"other\",256,{t},{t + 5}")
    # the other loop kind of the same tile, same grid: its name differs only after the
    # closing ">" of TileCfg (the tile's own fields end in "2, 2>", as ", 2>" does)
    twin = name.replace(f"2, 2>, {v}>", f"2, 2>, {3 - v}>")
    assert twin != name
    for d in (8500, 8600, 8700):
        rows.append(f"\"{twin}\",{grid},{t + 100 + d},{t + 100 + 2 * d}")
    (tmp_path / "run_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    line = {"config": {"M": 8192, "N": 8192, "K": 8192}, "steps": steps,
            "protocol": {"headline_launches_before_timed": first}, "ms_per_step": 7.01,
            "roofline": {"launch_ms": 7.005, "frac": 0.998}}
    lf = tmp_path / "line.json"
    lf.write_text("[bench] log line\n" + json.dumps(line) + "\n")
    out = io.StringIO()
    with redirect_stdout(out):
        assert bench.summarize_timed_headline(str(tmp_path), str(lf)) == 0
    text = out.getvalue()
    assert "launches 7 .. 11 of 32" in text
    assert "mean 7002.00 us, median 7002.00 us, min 7000.00 us, max 7004.00 us" in text
    assert "2*M*N*K / mean" in text and "2*M*N*K / median" in text


def test_counter_table_ratios_from_fake_passes(tmp_path):
    """Counter passes holding one dispatch of the 8192^3 kernel (the numbers chosen so each
    ratio has a known value) and of the calibration kernel: the table's row for that kernel
    shows those ratios, and rows with no counters show dashes."""
    import tiled_double_buffered_amd as tdb
    M = N = K = 8192
    desc, match = bench._kernel_match(tdb, M, N, K)
    _, v, c = tdb.gemm_f32_select(M, N, K)
    _, i = tdb.gemm_f32_config_info(c)
    name = (f"void gemmf32::gemm_f32_tile_kernel<gemmf32::TileCfg<{i['BM']}, {i['BN']}, "
            f"{i['BK']}, 2, 2>, {v}>(int)")
    grid = str((M // i["BM"]) * (N // i["BN"]) * i["threads"])
    assert match(name, grid)
    cyc = 1_000_000
    flop = 2.0 * M * N * K
    algo = 4.0 * (M * K + K * N + M * N)
    vals = {
        "mfma": {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.9 * cyc * 1024,
                 "SQ_INSTS_VALU_MFMA_MOPS_F32": flop / 512, "SQ_BUSY_CYCLES": 32 * cyc,
                 "SQ_WAVE_CYCLES": 1.0},
        "lds": {"SQ_LDS_BANK_CONFLICT": 5.0, "SQ_LDS_IDX_ACTIVE": 1000.0,
                "SQ_WAIT_INST_ANY": 40.0, "SQ_ACTIVE_INST_LDS": 3.0, "SQ_WAVE_CYCLES": 100.0},
        # 200 busy CUs: sum(BUSY_CU) / (sum(BUSY_CYCLES) / 32) = 200
        "busy": {"SQ_BUSY_CU_CYCLES": 200 * cyc, "SQ_BUSY_CYCLES": 32 * cyc},
        # 2 KiB counted per 1 KiB moved by the negate kernel for reads, 1 for writes
        "fetch": {"FETCH_SIZE": 3 * algo / 1024 / 2},
        "write": {"WRITE_SIZE": algo / 1024},
    }
    dirs = {}
    for kind, ctrs in vals.items():
        d = tmp_path / kind
        d.mkdir()
        lines = ["Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value"]
        for ctr, x in ctrs.items():
            lines.append(f'1,"{name}",{grid},{ctr},{x!r}')
        if kind == "fetch":
            lines.append(f'2,"void at::native::neg_kernel",1024,FETCH_SIZE,{512 * 1024 / 2}')
        if kind == "write":
            lines.append(f'2,"void at::native::neg_kernel",1024,WRITE_SIZE,{512 * 1024}')
        (d / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
        dirs[kind] = str(d)
    out = io.StringIO()
    with redirect_stdout(out):
        assert bench.counter_table(dirs) == 0
    rows = [ln for ln in out.getvalue().splitlines() if ln.startswith("square_8192")]
    disp = [ln for ln in rows if ln.split()[1] == "gemm_f32"]
    assert len(disp) == 1
    f = disp[0].split()
    # workload entry kind cfg tile grid cyc mfma mops lds wait ldsi busy read write algo ratio
    assert f[5] == grid and float(f[6]) == cyc
    assert float(f[7]) == pytest.approx(0.9, abs=1e-3)
    assert float(f[8]) == pytest.approx(1.0, abs=1e-3)
    assert float(f[9]) == pytest.approx(0.005, abs=1e-4)
    assert float(f[10]) == pytest.approx(0.40, abs=1e-2)
    assert float(f[11]) == pytest.approx(0.03, abs=1e-3)
    assert float(f[12]) == pytest.approx(200.0, abs=0.1)
    assert float(f[13]) == pytest.approx(3 * algo / 1e6, rel=1e-3)
    assert float(f[14]) == pytest.approx(algo / 1e6, rel=1e-3)
    assert float(f[16]) == pytest.approx(4.0, abs=0.01)
    other = [ln for ln in out.getvalue().splitlines() if ln.startswith("control_")]
    assert len(other) == 1 and other[0].split()[6] == "-"
