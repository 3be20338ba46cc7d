"""Seeded synthetic inputs for the FP32 GEMM C = A.B (shared by tests, bench and smoke).

This module only draws numbers.  It holds none of the product's arithmetic, so both the
CPU oracle's tests and the GPU path's tests can take their inputs from it without sharing
any code of the method itself.

Generator
---------
SplitMix64 (Steele, Lea & Flood, "Fast Splittable Pseudorandom Number Generators",
OOPSLA 2014; the 64-bit output function used here is the widely published SplitMix64
variant with D. Stafford's "Mix13" finalizer, as in S. Vigna's splitmix64.c).  Output
number e (e = 0, 1, ...) of the stream whose state starts at s0 is
    mix(s0 + (e + 1) * GAMMA)   (mod 2**64),
so any element can be produced from its index alone.

Matrix entries (the "uniform[-1, 1] from a fixed seed" of the workloads)
-----------------------------------------------------------------------
Element e (row-major linear index over the logical rows x cols matrix, independent of
any leading dimension) of matrix X in {A: 1, B: 2} under seed s takes
    u  = splitmix64 output e of the stream with s0 = (s << 8) | X
    ia = (u >> 40) - 2**23                 an integer in [-2**23, 2**23)
    v  = ia * 2**-23                       in [-1, 1 - 2**-23], exact in FP32
The values sit on a uniform grid of 2**24 points, so host, device and oracle see the same
bits and the integer ia gives an exact integer check of the product.

Sampled output positions (for the 8192^3 workload) use stream X = 3:
    i = u mod M,  j = (u >> 32) mod N,  duplicates allowed.
Seeds: workload index c uses s = 1000 * c + 1.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_A = 1
STREAM_B = 2
STREAM_SAMPLE = 3

# Workloads: (name, M, N, K, seed).  Seeds follow s = 1000 * c + 1 for workload group c.
WORKLOADS = {
    "square_128": (128, 128, 128, 1001),
    "ragged_127x193x61": (127, 193, 61, 2001),
    "ragged_513x257x129": (513, 257, 129, 2002),
    "square_1024": (1024, 1024, 1024, 3001),
    "rect_256x1024x128": (256, 1024, 128, 3002),
    "rect_1024x128x256": (1024, 128, 256, 3003),
    "square_4096": (4096, 4096, 4096, 4001),
    "square_8192": (8192, 8192, 8192, 5001),
    # one GPU's share of the 8192^3 product split by rows over eight GPUs
    "shard_1024x8192x8192": (1024, 8192, 8192, 6001),
}

_CHUNK = 1 << 23


def splitmix64(state0: int, index: np.ndarray) -> np.ndarray:
    """SplitMix64 output number `index` (uint64 array) of the stream starting at state0."""
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(state0 & 0xFFFFFFFFFFFFFFFF) + (idx + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def stream_state(seed: int, stream: int) -> int:
    return ((int(seed) << 8) | int(stream)) & 0xFFFFFFFFFFFFFFFF


def grid_ints(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    """Integers ia in [-2**23, 2**23) for elements start .. start+count-1 (int32)."""
    s0 = stream_state(seed, stream)
    out = np.empty(count, dtype=np.int32)
    for off in range(0, count, _CHUNK):
        n = min(_CHUNK, count - off)
        u = splitmix64(s0, np.arange(start + off, start + off + n, dtype=np.uint64))
        out[off:off + n] = (u >> np.uint64(40)).astype(np.int64) - (1 << 23)
    return out


def grid_matrix_ints(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    return grid_ints(seed, stream, rows * cols).reshape(rows, cols)


def grid_matrix(seed: int, stream: int, rows: int, cols: int, ld: int | None = None,
                pad_value: float = np.nan) -> np.ndarray:
    """FP32 rows x cols matrix of grid values; with ld > cols the result is a rows x ld
    buffer whose columns cols..ld-1 hold pad_value (the caller slices [:, :cols])."""
    ld = cols if ld is None else int(ld)
    if ld < cols:
        raise ValueError("ld < cols")
    vals = grid_ints(seed, stream, rows * cols).astype(np.float32)
    vals *= np.float32(2.0 ** -23)
    vals = vals.reshape(rows, cols)
    if ld == cols:
        return vals
    buf = np.full((rows, ld), pad_value, dtype=np.float32)
    buf[:, :cols] = vals
    return buf


def workload_inputs(M: int, N: int, K: int, seed: int):
    """(A, B) for a workload: A is M x K (stream 1), B is K x N (stream 2), FP32."""
    return grid_matrix(seed, STREAM_A, M, K), grid_matrix(seed, STREAM_B, K, N)


def sample_positions(seed: int, M: int, N: int, count: int = 4096):
    """Seeded output positions (i, j) for sampled checks; duplicates allowed."""
    u = splitmix64(stream_state(seed, STREAM_SAMPLE), np.arange(count, dtype=np.uint64))
    i = (u % np.uint64(M)).astype(np.int64)
    j = ((u >> np.uint64(32)) % np.uint64(N)).astype(np.int64)
    return i, j
