"""bench.py on the host: the parity gate that keeps a wrong product from publishing a
throughput, the trace summary the roofline figure is read from, and the refusal of
more than one GPU.  No GPU needed."""
import io
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
