"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The oracle computes C64 = sum_k A[i][k] * B[k][j] in FP64 and Bnd = sum_k |A[i][k] B[k][j]|.
It is pinned by:
  * hand-worked products (tests/golden/worked_examples.json);
  * exact rational brute force (fractions.Fraction) on every tiny shape up to 4 x 4 x 4;
  * an exact integer cross-check: grid inputs are ia * 2**-23 with integer ia, so
    C_exact = (ia @ ib) * 2**-46 with the integer product taken in int64 (no rounding);
  * closed forms: identity, all-ones (C = K), rank-1, constant rows/columns, permutations,
    power-of-two diagonal scaling, K = 0;
  * planted mistakes: each plausible slip in the oracle's source (a dropped term, a sign,
    a wrong or transposed index, FP32 products, a bound without absolute values) is
    compiled into a mutant library, and the pins must catch every one of them.
All run on the CPU.
"""
import json
import os
import re
import shutil
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
import tdb_inputs as ti

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 2.0 ** -46


def _exact(A, B):
    """Exact rational product and bound of small float matrices."""
    M, K = A.shape
    N = B.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    D = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            for k in range(K):
                p = Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
                C[i][j] += p
                D[i][j] += abs(p)
    return C, D


def _grid_pair(M, N, K, seed):
    ia = ti.grid_matrix_ints(seed, ti.STREAM_A, M, K).astype(np.int64)
    ib = ti.grid_matrix_ints(seed, ti.STREAM_B, K, N).astype(np.int64)
    A = (ia.astype(np.float64) * 2.0 ** -23).astype(np.float32)
    B = (ib.astype(np.float64) * 2.0 ** -23).astype(np.float32)
    return ia, ib, A, B


# ----------------------------------------------------------------------------- the pin suite
def pin_failures(orc: oracle.OracleLib, square_only: bool = False) -> list:
    """Run a compact set of pins against one oracle library; returns what failed.
    With square_only every input is square (M = N = K, tight leading dimensions), so a
    mutant that transposes an index still reads inside its buffers."""
    fails = []
    rng = np.random.default_rng(7)

    # exact rational brute force
    shapes = [(n, n, n) for n in range(1, 5)] if square_only else \
        [(m, n, k) for m in range(1, 5) for n in range(1, 5) for k in range(1, 5)]
    for (m, n, k) in shapes:
        for kind in ("ints", "floats"):
            if kind == "ints":
                A = rng.integers(-2, 3, (m, k)).astype(np.float32)
                B = rng.integers(-2, 3, (k, n)).astype(np.float32)
            else:
                A = rng.uniform(-1, 1, (m, k)).astype(np.float32)
                B = rng.uniform(-1, 1, (k, n)).astype(np.float32)
            C64, Bnd = orc.gemm_f64(A, B)
            Ce, De = _exact(A, B)
            for i in range(m):
                for j in range(n):
                    tol = (k - 1) * 2.0 ** -53 * float(De[i][j])
                    if abs(Fraction(C64[i, j]) - Ce[i][j]) > Fraction(tol):
                        fails.append(f"brute C {m}x{n}x{k} {kind} ({i},{j})")
                    if abs(Fraction(Bnd[i, j]) - De[i][j]) > Fraction(tol):
                        fails.append(f"brute Bnd {m}x{n}x{k} {kind} ({i},{j})")
            rows = np.arange(m).repeat(n)
            cols = np.tile(np.arange(n), m)
            c, b = orc.gemm_f64_sampled(A, B, rows, cols)
            if not (np.array_equal(c, C64[rows, cols]) and np.array_equal(b, Bnd[rows, cols])):
                fails.append(f"sampled != full {m}x{n}x{k} {kind}")

    # exact integer cross-check on grid inputs
    grid_shapes = [(64, 64, 64)] if square_only else [(64, 64, 64), (37, 53, 29)]
    for (m, n, k) in grid_shapes:
        ia, ib, A, B = _grid_pair(m, n, k, 99)
        S = ia @ ib
        Sa = np.abs(ia) @ np.abs(ib)
        C64, Bnd = orc.gemm_f64(A, B)
        if np.max(np.abs(C64 - S * SCALE)) > 2.0 ** -32:
            fails.append(f"integer C {m}x{n}x{k}")
        if np.max(np.abs(Bnd - Sa * SCALE)) > 2.0 ** -32:
            fails.append(f"integer Bnd {m}x{n}x{k}")
        ri, rj = ti.sample_positions(5, m, n, 200)
        c, b = orc.gemm_f64_sampled(A, B, ri, rj)
        if np.max(np.abs(c - S[ri, rj] * SCALE)) > 2.0 ** -32:
            fails.append(f"integer sampled C {m}x{n}x{k}")
        if np.max(np.abs(b - Sa[ri, rj] * SCALE)) > 2.0 ** -32:
            fails.append(f"integer sampled Bnd {m}x{n}x{k}")

    # closed forms
    n = 24
    B = ti.grid_matrix(3, ti.STREAM_B, n, n)
    C64, _ = orc.gemm_f64(np.eye(n, dtype=np.float32), B)
    if not np.array_equal(C64, B.astype(np.float64)):
        fails.append("identity")
    ones = np.ones((n, n), dtype=np.float32)
    C64, Bnd = orc.gemm_f64(ones, ones)
    if not (np.all(C64 == n) and np.all(Bnd == n)):
        fails.append("all-ones")
    perm = np.random.default_rng(1).permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    C64, _ = orc.gemm_f64(P, B)
    if not np.array_equal(C64, B[perm].astype(np.float64)):
        fails.append("permutation")
    return fails


# ----------------------------------------------------------------------------- tests
def test_oracle_builds_and_loads():
    path = oracle.build()
    assert os.path.exists(path)
    assert oracle.max_threads() >= 1


def test_pin_suite_passes_on_the_oracle():
    assert pin_failures(oracle.default()) == []


def test_worked_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if c.get("K", None) == 0:
            A = np.zeros((len(c["A"]), 0), dtype=np.float32)
            B = np.zeros((0, c["N"]), dtype=np.float32)
        else:
            A = np.array(c["A"], dtype=np.float32)
            B = np.array(c["B"], dtype=np.float32)
        C64, Bnd = oracle.gemm_f64(A, B)
        assert np.array_equal(C64, np.array(c["C"], dtype=np.float64)), c["name"]
        assert np.array_equal(Bnd, np.array(c["Bnd"], dtype=np.float64)), c["name"]


@pytest.mark.parametrize("name", ["square_128", "ragged_127x193x61", "ragged_513x257x129",
                                  "rect_256x1024x128", "rect_1024x128x256"])
def test_integer_exact_on_workloads(name):
    """On the workloads' own grid inputs the FP64 oracle equals the exact product."""
    M, N, K, seed = ti.WORKLOADS[name]
    ia, ib, A, B = _grid_pair(M, N, K, seed)
    A2, B2 = ti.workload_inputs(M, N, K, seed)
    assert np.array_equal(A, A2) and np.array_equal(B, B2)
    C64, Bnd = oracle.gemm_f64(A, B)
    assert np.max(np.abs(C64 - (ia @ ib) * SCALE)) <= 2.0 ** -32
    assert np.max(np.abs(Bnd - (np.abs(ia) @ np.abs(ib)) * SCALE)) <= 2.0 ** -32


def test_integer_exact_square_1024_rows():
    """1024^3: 96 rows of the full oracle against the exact integer product."""
    M, N, K, seed = ti.WORKLOADS["square_1024"]
    ia, ib, A, B = _grid_pair(M, N, K, seed)
    rows = slice(400, 496)
    C64, Bnd = oracle.gemm_f64(A[rows], B)
    assert np.max(np.abs(C64 - (ia[rows] @ ib) * SCALE)) <= 2.0 ** -32
    assert np.max(np.abs(Bnd - (np.abs(ia[rows]) @ np.abs(ib)) * SCALE)) <= 2.0 ** -32


@pytest.mark.parametrize("name", ["square_4096", "square_8192"])
def test_integer_exact_sampled_large(name):
    """The sampled oracle at the large workloads' K, on the workload's own sample positions:
    only the sampled rows of A and columns of B are generated (element index = row-major
    linear index), packed into an n x K and a K x n matrix, and position s is (s, s)."""
    M, N, K, seed = ti.WORKLOADS[name]
    n = 512
    ri, rj = ti.sample_positions(seed, M, N, 4096)
    ri, rj = ri[:n], rj[:n]
    ka = np.arange(K, dtype=np.int64)
    sa = ti.stream_state(seed, ti.STREAM_A)
    sb = ti.stream_state(seed, ti.STREAM_B)
    ia = ((ti.splitmix64(sa, (ri[:, None] * K + ka[None, :]).astype(np.uint64).ravel())
           >> np.uint64(40)).astype(np.int64) - (1 << 23)).reshape(n, K)
    ib = ((ti.splitmix64(sb, (ka[:, None] * N + rj[None, :]).astype(np.uint64).ravel())
           >> np.uint64(40)).astype(np.int64) - (1 << 23)).reshape(K, n)
    A = (ia * 2.0 ** -23).astype(np.float32)
    B = (ib * 2.0 ** -23).astype(np.float32)
    s = np.arange(n)
    c, b = oracle.gemm_f64_sampled(A, B, s, s)
    S = np.einsum("sk,ks->s", ia, ib)
    Sa = np.einsum("sk,ks->s", np.abs(ia), np.abs(ib))
    assert np.max(np.abs(c - S * SCALE)) <= 2.0 ** -32
    assert np.max(np.abs(b - Sa * SCALE)) <= 2.0 ** -32


def test_closed_forms():
    rng = np.random.default_rng(11)
    # K = 1: rank-1 outer product, exact in FP64
    u = ti.grid_matrix(21, 1, 37, 1)
    v = ti.grid_matrix(21, 2, 1, 45)
    C64, Bnd = oracle.gemm_f64(u, v)
    assert np.array_equal(C64, np.outer(u[:, 0].astype(np.float64), v[0].astype(np.float64)))
    assert np.array_equal(Bnd, np.abs(C64))
    # constant rows x constant columns with few significant bits: C = K * u_i * v_j exactly
    for K in (1, 7, 64, 1000):
        u = (rng.integers(-1023, 1024, 19) * 2.0 ** -10).astype(np.float32)
        v = (rng.integers(-1023, 1024, 23) * 2.0 ** -10).astype(np.float32)
        A = np.repeat(u[:, None], K, axis=1)
        B = np.repeat(v[None, :], K, axis=0)
        C64, _ = oracle.gemm_f64(A, B)
        assert np.array_equal(C64, K * np.outer(u.astype(np.float64), v.astype(np.float64)))
    # power-of-two diagonal scaling is exact
    n = 33
    e = rng.integers(-20, 21, n)
    D = np.diag(np.ldexp(1.0, e)).astype(np.float32)
    B = ti.grid_matrix(22, 2, n, 29)
    C64, _ = oracle.gemm_f64(D, B)
    assert np.array_equal(C64, np.ldexp(B.astype(np.float64), e[:, None]))
    # all-ones at the workloads' K values: C = K exactly
    for K in (61, 129, 1024):
        C64, Bnd = oracle.gemm_f64(np.ones((3, K), np.float32), np.ones((K, 5), np.float32))
        assert np.all(C64 == K) and np.all(Bnd == K)
    # K = 0: zeros
    C64, Bnd = oracle.gemm_f64(np.zeros((4, 0), np.float32), np.zeros((0, 6), np.float32))
    assert C64.shape == (4, 6) and not C64.any() and not Bnd.any()


def test_leading_dimensions_and_padding():
    """Views with leading dimension > width: padding (NaN) never reaches the result."""
    M, N, K = 19, 23, 17
    Ab = ti.grid_matrix(31, 1, M, K, ld=K + 5)
    Bb = ti.grid_matrix(31, 2, K, N, ld=N + 3)
    A, B = Ab[:, :K], Bb[:, :N]
    assert A.strides[0] == (K + 5) * 4
    C64, Bnd = oracle.gemm_f64(A, B)
    assert np.all(np.isfinite(C64))
    C2, B2 = oracle.gemm_f64(np.ascontiguousarray(A), np.ascontiguousarray(B))
    assert np.array_equal(C64, C2) and np.array_equal(Bnd, B2)


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.gemm_f64(np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32))
    with pytest.raises(TypeError):
        oracle.gemm_f64(np.zeros((2, 3), np.float64), np.zeros((3, 2), np.float32))
    with pytest.raises(RuntimeError):
        oracle.gemm_f64_sampled(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32),
                                [0, 2], [0, 0])


# ----------------------------------------------------------------------------- tolerance
def test_tolerance_ratio_edges():
    C64 = np.array([1.0, 0.0, -2.0])
    Bnd = np.array([1.0, 0.0, 3.0])
    lim = 1e-5 * Bnd + 1e-6
    assert oracle.tolerance_ratio(C64, C64, Bnd) == 0.0
    r = oracle.tolerance_ratio(C64 + lim, C64, Bnd)
    assert abs(r - 1.0) < 1e-9
    assert oracle.tolerance_ratio(C64 + 1.01 * lim, C64, Bnd) > 1.0
    assert oracle.tolerance_ratio(C64 - 0.5 * lim, C64, Bnd) == pytest.approx(0.5, rel=1e-9)
    assert oracle.tolerance_ratio(np.array([np.nan, 0, 0]), C64, Bnd) == float("inf")
    assert oracle.tolerance_ratio(np.zeros(0), np.zeros(0), np.zeros(0)) == 0.0


def _round_mantissa(X: np.ndarray, bits: int) -> np.ndarray:
    """Round FP32 values to `bits` explicit mantissa bits (nearest, ties to even)."""
    u = X.astype(np.float32).view(np.uint32).astype(np.uint64)
    drop = 23 - bits
    half = np.uint64(1 << (drop - 1))
    lsb = (u >> np.uint64(drop)) & np.uint64(1)
    u = (u + half - np.uint64(1) + lsb) & ~np.uint64((1 << drop) - 1)
    return u.astype(np.uint32).view(np.float32)


def test_tolerance_rejects_10bit_mantissa_products():
    """A TF32/XF32-style shortcut (10-bit mantissa operands) misses the bound already at
    the smallest ragged workload, so passing it requires true FP32 multiplies."""
    M, N, K, seed = ti.WORKLOADS["ragged_127x193x61"]
    A, B = ti.workload_inputs(M, N, K, seed)
    C64, Bnd = oracle.gemm_f64(A, B)
    C10, _ = oracle.gemm_f64(_round_mantissa(A, 10), _round_mantissa(B, 10))
    assert oracle.tolerance_ratio(C10, C64, Bnd) > 1.0


@pytest.mark.parametrize("name", ["ragged_513x257x129", "square_1024"])
def test_tolerance_accepts_fp32_accumulation(name):
    """Straight FP32 summation in k order (the worst order for error growth) passes with
    wide headroom at the workloads' K."""
    M, N, K, seed = ti.WORKLOADS[name]
    A, B = ti.workload_inputs(M, N, K, seed)
    A, = (A[:64],)
    C64, Bnd = oracle.gemm_f64(A, B)
    acc = np.zeros((A.shape[0], N), dtype=np.float32)
    for k in range(K):
        acc += np.outer(A[:, k], B[k]).astype(np.float32)
    r = oracle.tolerance_ratio(acc, C64, Bnd)
    assert r < 0.25, r


# ----------------------------------------------------------------------------- mutants
_MUTANTS = {
    "sign": ("c[j] += p;", "c[j] -= p;"),
    "dropped_last_term": ("c[j] += p;", "if (k + 1 < K) c[j] += p;"),
    "wrong_column_index": ("(double)brow[j];", "(double)brow[N - 1 - j];"),
    "transposed_A": ("(double)A[i * lda + k];", "(double)A[k * lda + i];"),
    "fp32_products": ("const double p = a * (double)brow[j];",
                      "const double p = (float)(a * (double)brow[j]);"),
    "bound_without_abs": ("b[j] += fabs(p);", "b[j] += p;"),
    "sampled_transposed_B": ("(double)B[k * ldb + j];", "(double)B[j * ldb + k];"),
    "sampled_dropped_first": ("c += p;", "c += (k ? p : 0.0);"),
    "sampled_bound_sign": ("b += fabs(p);", "b += p;"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_dir):
    old, new = _MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"anchor for {name} must be unique"
    msrc = os.path.join(mutant_dir, f"{name}.c")
    with open(msrc, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(src=msrc, out=os.path.join(mutant_dir, f"lib{name}.so"))
    fails = pin_failures(oracle.OracleLib(lib), square_only=True)
    assert fails, f"mutant {name} passed every pin"


def test_mutant_anchors_exist():
    src = open(oracle.SRC).read()
    for name, (old, _) in _MUTANTS.items():
        assert re.escape(old) and src.count(old) == 1, name
