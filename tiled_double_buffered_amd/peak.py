"""The FP32 matrix-core ceiling of this device at the clock it sustains, measured with
gemm_f32_peak_probe (a kernel of nothing but v_mfma_f32_32x32x2_f32 on registers).

The specification peak (157.3 TFLOP/s) assumes the 2.4 GHz peak shader clock.  Under a
sustained matrix load the clock settles where power management puts it, and it takes
tens of milliseconds of load to ramp up from idle; this measures both the attainable
rate and the clock behind it, after a warm-up long enough for the ramp.

    python -m tiled_double_buffered_amd.peak       # prints one JSON object
"""
from __future__ import annotations

import json
import statistics
import sys

from . import _binding as b

MFMA_FLOP = 32 * 32 * 2 * 2      # one v_mfma_f32_32x32x2_f32
WAVES_PER_BLOCK = 4
MFMA_PER_ITER = 16
CUS = 256                        # MI355X compute units, 4 SIMDs each
FLOP_PER_CLOCK = CUS * 4 * MFMA_FLOP // 64   # each SIMD retires one such MFMA per 64 clocks


def mfma_ceiling(blocks: int = 768, iters: int = 6144, warm_s: float = 0.3,
                 launches: int = 5, stream=None) -> dict:
    """Time `launches` probe launches after `warm_s` seconds of warm-up on `stream`
    (default: torch's current stream) and return the attained rate, the shader clock and
    the rate that one instruction per SIMD per 64 clocks gives at that clock.

    The default of 768 workgroups is three waves per SIMD, all resident at once (the probe
    needs 132 registers per lane, so a SIMD holds three of its waves); 6144 iterations
    make one launch about 8 ms, so that launch and ramp overheads stay near 0.3%."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    rec = torch.zeros(blocks * WAVES_PER_BLOCK * 2, dtype=torch.int64, device=dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    s = st.cuda_stream

    def launch():
        rc = b.gemm_f32_peak_probe(blocks, iters, out.data_ptr(), rec.data_ptr(), s)
        if rc != b.OK:
            raise b.GemmError(rc, "gemm_f32_peak_probe")

    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    launch()
    e1.record(st)
    torch.cuda.synchronize()
    one_ms = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(max(1, int(warm_s * 1e3 / one_ms))):
        launch()
    times = []
    for _ in range(launches):
        e0.record(st)
        launch()
        e1.record(st)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    r = rec.view(-1, 2).cpu().numpy().astype("float64")
    cycles, ticks = r[:, 0], r[:, 1]
    clock_ghz = float(cycles.sum() / ticks.sum() * 0.1)
    ms = statistics.median(times)
    flop = float(blocks) * WAVES_PER_BLOCK * MFMA_PER_ITER * iters * MFMA_FLOP
    return {
        "value": round(flop / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "clock_ghz": round(clock_ghz, 4),
        "at_clock_tflops": round(FLOP_PER_CLOCK * clock_ghz * 1e9 / 1e12, 3),
        "launch_ms": round(ms, 4),
        "probe": f"{blocks} workgroups x 4 waves x {MFMA_PER_ITER * iters} "
                 f"v_mfma_f32_32x32x2_f32, after {warm_s:.1f} s of warm-up",
    }


def main() -> int:
    print(json.dumps(mfma_ceiling()), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
