"""GPU parity: the HIP library through its C ABI against the FP64 CPU oracle.

Every check is elementwise: |C - C64| <= 1e-5 * Bnd + 1e-6 with C64 = sum_k A B and
Bnd = sum_k |A| |B| from the oracle, on the seeded grid inputs of tdb_inputs.  Full output
up to 4096^3; at 8192^3, 4096 seeded positions (the oracle computes them one by one).
Structural invariants that hold whatever the rounding: single- and double-buffered runs of
one tile configuration are bitwise identical (same MFMA sequence, different schedule),
repeated runs are bitwise identical, C is written and never read, padding is untouched.
"""
import sys

import numpy as np
import pytest

import oracle
import tdb_inputs as ti

torch = pytest.importorskip("torch")
import tiled_double_buffered_amd as tdb  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a CPU-only machine: skip, never fall back
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
NCFG = tdb.gemm_f32_num_configs()
_VID = {"sb": tdb.VARIANT_SB, "db": tdb.VARIANT_DB, "ms": tdb.VARIANT_MS,
        "sb3": tdb.VARIANT_SB3, "ks": tdb.VARIANT_KS}


def _has(cfg, v):
    """Configuration cfg has a kernel for variant v (any configuration: cfg = -1)."""
    return v == "auto" or cfg < 0 or bool(tdb.gemm_f32_config_variants(cfg) & (1 << _VID[v]))


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _run(A, B, variant="auto", cfg=-1, out=None):
    C = tdb.matmul(A, B, out=out, variant=variant, cfg_id=cfg)
    torch.cuda.synchronize()
    return C


def _ratio(C: torch.Tensor, C64, Bnd) -> float:
    return oracle.tolerance_ratio(C.cpu().numpy(), C64, Bnd)


_ORACLE_CACHE = {}


def _workload(name):
    if name not in _ORACLE_CACHE:
        M, N, K, seed = ti.WORKLOADS[name]
        A, B = ti.workload_inputs(M, N, K, seed)
        C64, Bnd = oracle.gemm_f64(A, B)
        _ORACLE_CACHE[name] = (A, B, C64, Bnd)
    return _ORACLE_CACHE[name]


SMALL = ["square_128", "ragged_127x193x61", "ragged_513x257x129", "square_1024",
         "rect_256x1024x128", "rect_1024x128x256"]


@pytest.mark.parametrize("variant", ["auto", "sb", "db", "ms", "sb3", "ks"])
@pytest.mark.parametrize("name", SMALL)
def test_workload_parity(name, variant):
    _say(f"[parity] {name} {variant}")
    A, B, C64, Bnd = _workload(name)
    M, N = C64.shape
    C = torch.full((M, N), float("nan"), device=DEV)   # proves C is not read
    _run(_dev(A), _dev(B), variant, out=C)
    r = _ratio(C, C64, Bnd)
    _say(f"[parity] {name} {variant} ratio={r:.3g}")
    assert r <= 1.0


@pytest.mark.parametrize("cfg", range(NCFG))
def test_every_config_sb_equals_db_and_matches_oracle(cfg):
    """Each tile configuration, on a ragged shape spanning several tiles in M, N and K and
    on aligned ones (one with many K tiles, so the multi-stage ring wraps several times):
    all three variants pass, and agree bit for bit (same MFMA sequence per accumulator)."""
    for (M, N, K, seed) in [(300, 333, 97, 11), (512, 512, 256, 12), (768, 512, 1024, 13)]:
        _say(f"[config] cfg={cfg} {M}x{N}x{K}")
        A, B = ti.workload_inputs(M, N, K, seed)
        C64, Bnd = oracle.gemm_f64(A, B)
        Ad, Bd = _dev(A), _dev(B)
        if not _has(cfg, "db"):  # the 16-row configuration: its K-split kernel only
            Cks = _run(Ad, Bd, "ks", cfg).clone()
            assert _ratio(Cks, C64, Bnd) <= 1.0
            assert torch.equal(_run(Ad, Bd, "ks", cfg), Cks), "K-split is not deterministic"
            assert torch.equal(_run(Ad, Bd, "auto", cfg), Cks), "auto on a K-split-only cfg"
            continue
        Csb = _run(Ad, Bd, "sb", cfg).clone()
        Cdb = _run(Ad, Bd, "db", cfg).clone()
        Csb3 = _run(Ad, Bd, "sb3", cfg).clone()
        assert _ratio(Csb, C64, Bnd) <= 1.0
        assert _ratio(Cdb, C64, Bnd) <= 1.0
        assert torch.equal(Csb, Cdb), "single- and double-buffered results differ"
        assert torch.equal(Csb3, Csb), "split-barrier and single-buffered results differ"
        if _has(cfg, "ms"):
            Cms = _run(Ad, Bd, "ms", cfg).clone()
            assert _ratio(Cms, C64, Bnd) <= 1.0
            assert torch.equal(Cms, Cdb), "multi-stage and double-buffered results differ"
        if _has(cfg, "ks"):  # another summation order: within the bound, deterministic
            Cks = _run(Ad, Bd, "ks", cfg).clone()
            assert _ratio(Cks, C64, Bnd) <= 1.0
            assert torch.equal(_run(Ad, Bd, "ks", cfg), Cks), "K-split is not deterministic"


def _edge_shapes():
    rng = np.random.default_rng(2024)
    dims_mn = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257,
               383, 384, 385]
    dims_k = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100]
    shapes = {(int(rng.choice(dims_mn)), int(rng.choice(dims_mn)), int(rng.choice(dims_k)))
              for _ in range(40)}
    return sorted(shapes)


@pytest.mark.parametrize("cfg", range(NCFG))
def test_edge_residues(cfg):
    """M, N, K around multiples of every tile size, including 1 and 2."""
    for (M, N, K) in _edge_shapes():
        A, B = ti.workload_inputs(M, N, K, 7000 + M + N + K)
        C64, Bnd = oracle.gemm_f64(A, B)
        Ad, Bd = _dev(A), _dev(B)
        for v in [v for v in ("sb", "db", "ms", "sb3", "ks") if _has(cfg, v)]:
            C = torch.full((M, N), float("nan"), device=DEV)
            _run(Ad, Bd, v, cfg, out=C)
            r = _ratio(C, C64, Bnd)
            assert r <= 1.0, (cfg, v, M, N, K, r)


def _dispatched_pairs():
    """(variant name, configuration) of every kernel the dispatcher or the explicit SB, DB
    and MS entry points pick for a workload shape, or for a decode product."""
    names = {tdb.VARIANT_SB: "sb", tdb.VARIANT_DB: "db", tdb.VARIANT_MS: "ms",
             tdb.VARIANT_KS: "ks"}
    pairs = set()
    shapes = [w[:3] for w in ti.WORKLOADS.values()] + [(16, 4096, 4096), (1, 4096, 4096)]
    for (M, N, K) in shapes:
        _, v, c = tdb.gemm_f32_select(M, N, K)
        pairs.add((names[v], c))
        for v in (tdb.VARIANT_SB, tdb.VARIANT_DB, tdb.VARIANT_MS):
            pairs.add((names[v], tdb.gemm_f32_select_cfg(M, N, K, v)))
    return sorted(pairs, key=lambda p: (p[1], p[0]))


@pytest.mark.parametrize("pair", _dispatched_pairs(), ids=lambda p: f"{p[0]}{p[1]}")
def test_residue_sweep(pair):
    """Every residue of M in 1 .. 2 BM, of N in 1 .. 2 BN and of K in 1 .. 2 BK (the other
    two sizes held at ragged values spanning two tiles), C pre-filled with NaN, element by
    element within the bound.  The oracle runs once per M and N sweep on the largest size:
    the first m rows (n columns) of that product are the product of the first m rows of A
    (n columns of B)."""
    v, cfg = pair
    _, info = tdb.gemm_f32_config_info(cfg)
    bm, bn, bk = info["BM"], info["BN"], info["BK"]
    _say(f"[residues] {v} cfg={cfg} {bm}x{bn}x{bk}")
    # M sweep
    N, K = bn + 7, bk + 3
    A, B = ti.workload_inputs(2 * bm, N, K, 7700 + cfg)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    for m in range(1, 2 * bm + 1):
        C = torch.full((m, N), float("nan"), device=DEV)
        _run(Ad[:m], Bd, v, cfg, out=C)
        r = _ratio(C, C64[:m], Bnd[:m])
        assert r <= 1.0, (v, cfg, "M", m, N, K, r)
    # N sweep
    M, K = bm + 5, bk + 3
    A, B = ti.workload_inputs(M, 2 * bn, K, 7800 + cfg)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    for n in range(1, 2 * bn + 1):
        C = torch.full((M, n), float("nan"), device=DEV)
        _run(Ad, Bd[:, :n], v, cfg, out=C)
        r = _ratio(C, C64[:, :n], Bnd[:, :n])
        assert r <= 1.0, (v, cfg, "N", M, n, K, r)
    # K sweep (each K its own sums)
    M, N = bm + 5, bn + 7
    for k in range(1, 2 * bk + 1):
        A, B = ti.workload_inputs(M, N, k, 7900 + 100 * cfg + k)
        C64, Bnd = oracle.gemm_f64(A, B)
        C = torch.full((M, N), float("nan"), device=DEV)
        _run(_dev(A), _dev(B), v, cfg, out=C)
        r = _ratio(C, C64, Bnd)
        assert r <= 1.0, (v, cfg, "K", M, N, k, r)


KS16 = [c for c in range(NCFG) if tdb.gemm_f32_config_variants(c) == 1 << tdb.VARIANT_KS]


def _decode_shapes():
    """Few rows against wide and long operands: every row count 1..17, N and K at and
    around the 16-column tile and the 64-deep K group (the K range splits over 16 waves in
    whole groups, so K from 1 to past 16 groups), and a few layer-sized products."""
    shapes = [(m, 16, 64) for m in range(1, 18)]
    shapes += [(16, n, 100) for n in (1, 2, 15, 17, 31, 33, 255, 257, 1000)]
    shapes += [(7, 48, k) for k in (1, 2, 3, 4, 5, 15, 16, 17, 63, 64, 65, 127, 128, 129,
                                      1023, 1024, 1025, 1087, 2000)]
    shapes += [(1, 4096, 4096), (8, 4096, 4096), (16, 4096, 4096), (16, 11008, 4096),
               (16, 4096, 11008), (33, 512, 3000), (5, 4111, 777)]
    return shapes


@pytest.mark.parametrize("cfg", KS16)
def test_ks16_decode_shapes(cfg):
    """The 16-row K-split kernel: element by element within the bound on every shape, C
    pre-filled with NaN, and the same bits on a second run."""
    for i, (M, N, K) in enumerate(_decode_shapes()):
        _say(f"[ks16] cfg={cfg} {M}x{N}x{K}")
        A, B = ti.workload_inputs(M, N, K, 8100 + i)
        C64, Bnd = oracle.gemm_f64(A, B)
        Ad, Bd = _dev(A), _dev(B)
        C = torch.full((M, N), float("nan"), device=DEV)
        _run(Ad, Bd, "ks", cfg, out=C)
        r = _ratio(C, C64, Bnd)
        assert r <= 1.0, (M, N, K, r)
        assert torch.equal(_run(Ad, Bd, "ks", cfg), C), (M, N, K)


@pytest.mark.parametrize("cfg", KS16)
def test_ks16_matches_the_guarded_loads(cfg):
    """Row strides too large for the 32-bit buffer offsets take the element-wise loads; the
    product is the same bit for bit (same instructions, same order), and within the bound."""
    M, N, K = 9, 70, 300
    A, B = ti.workload_inputs(M, N, K, 8200)
    C64, Bnd = oracle.gemm_f64(A, B)
    fast = _run(_dev(A), _dev(B), "ks", cfg).clone()
    # A rows 2^26 + 5 floats apart: a 16-row block of A spans more than 4 GiB (2.1 GB in all)
    lda = (1 << 26) + 5
    Abig = torch.full(((M - 1) * lda + K,), float("nan"), device=DEV)
    Abig.as_strided((M, K), (lda, 1)).copy_(torch.from_numpy(A))
    Av = Abig.as_strided((M, K), (lda, 1))
    slow = _run(Av, _dev(B), "ks", cfg)
    assert _ratio(slow, C64, Bnd) <= 1.0
    assert torch.equal(slow, fast)
    del Abig, Av


def _random_cases(n=60, seed=31337):
    """Seeded random products: sizes log-uniform in 1..700, leading dimensions padded by
    0..7, base pointers offset by 0 or 1 float, any variant and a configuration that has
    it."""
    rng = np.random.default_rng(seed)
    variants = ["auto", "sb", "db", "ms", "sb3", "ks"]
    cases = []
    for i in range(n):
        M, N, K = (int(np.exp(rng.uniform(0.0, np.log(700.0)))) for _ in range(3))
        v = variants[int(rng.integers(len(variants)))]
        cands = [c for c in range(NCFG) if _has(c, v)]
        cfg = -1 if v == "auto" else cands[int(rng.integers(len(cands)))]
        pads = [int(x) for x in rng.integers(0, 8, 3)]
        offs = [int(x) for x in rng.integers(0, 2, 3)]
        cases.append((i, M, N, K, v, cfg, pads, offs))
    return cases


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: f"r{c[0]}")
def test_random_shapes_strides_and_offsets(case):
    """Elementwise parity on random sizes, strides and alignments, with NaN in every pad
    (it must not leak into C) and C's own pad left untouched."""
    i, M, N, K, v, cfg, (pa, pb, pc), (oa, ob, oc) = case
    lda, ldb, ldc = K + pa, N + pb, N + pc
    _say(f"[random] #{i} {M}x{N}x{K} {v} cfg={cfg} ld=({lda},{ldb},{ldc}) off=({oa},{ob},{oc})")
    Ab = ti.grid_matrix(9300 + i, 1, M, K, ld=lda)
    Bb = ti.grid_matrix(9300 + i, 2, K, N, ld=ldb)
    C64, Bnd = oracle.gemm_f64(Ab[:, :K], Bb[:, :N])
    Ad = torch.full((M * lda + oa,), float("nan"), device=DEV)
    Bd = torch.full((K * ldb + ob,), float("nan"), device=DEV)
    Cd = torch.full((M * ldc + oc,), float("nan"), device=DEV)
    Ad[oa:].view(M, lda).copy_(torch.from_numpy(Ab))
    Bd[ob:].view(K, ldb).copy_(torch.from_numpy(Bb))
    A = Ad[oa:].view(M, lda)[:, :K]
    B = Bd[ob:].view(K, ldb)[:, :N]
    C = Cd[oc:].view(M, ldc)[:, :N]
    _run(A, B, v, cfg, out=C)
    assert _ratio(C, C64, Bnd) <= 1.0, case
    Cfull = Cd[oc:].view(M, ldc).cpu().numpy()
    assert np.all(np.isnan(Cfull[:, N:])), "C padding was written"
    if oc:
        assert torch.isnan(Cd[:oc]).all()


@pytest.mark.parametrize("cfg", [-1] + list(range(NCFG)))
def test_leading_dimensions_padding_and_misalignment(cfg):
    """Row strides larger than the rows, odd strides (rows not 16-byte aligned), base
    pointers offset by 4 bytes; NaN in every pad: it must not leak into C, and C's own pad
    must stay untouched."""
    M, N, K = 150, 140, 70
    cases = [(K + 4, N + 4, N + 12, 0), (K + 1, N + 3, N + 5, 0), (K + 4, N + 4, N + 4, 1)]
    for (lda, ldb, ldc, off) in cases:
        _say(f"[ld] cfg={cfg} lda={lda} ldb={ldb} ldc={ldc} off={off}")
        Ab = ti.grid_matrix(81, 1, M, K, ld=lda)
        Bb = ti.grid_matrix(81, 2, K, N, ld=ldb)
        C64, Bnd = oracle.gemm_f64(Ab[:, :K], Bb[:, :N])
        Ad = torch.full((M * lda + off,), float("nan"), device=DEV)
        Bd = torch.full((K * ldb + off,), float("nan"), device=DEV)
        Cd = torch.full((M * ldc + off,), float("nan"), device=DEV)
        Ad[off:].view(M, lda).copy_(torch.from_numpy(Ab))
        Bd[off:].view(K, ldb).copy_(torch.from_numpy(Bb))
        A = Ad[off:].view(M, lda)[:, :K]
        B = Bd[off:].view(K, ldb)[:, :N]
        C = Cd[off:].view(M, ldc)[:, :N]
        for v in [v for v in ("sb", "db", "ms", "ks") if _has(cfg, v)]:
            _run(A, B, v, cfg, out=C)
            assert _ratio(C, C64, Bnd) <= 1.0, (cfg, v, lda, ldb, ldc, off)
            Cfull = Cd[off:].view(M, ldc).cpu().numpy()
            assert np.all(np.isnan(Cfull[:, N:])), "C padding was written"
        if off:
            assert torch.isnan(Cd[:off]).all()


def test_k_zero_writes_zeros_and_empty_is_noop():
    for v in ("auto", "sb", "db", "ms"):
        C = torch.full((37, 41), float("nan"), device=DEV)
        A = torch.empty((37, 0), device=DEV)
        B = torch.empty((0, 41), device=DEV)
        _run(A, B, v, out=C)
        assert torch.count_nonzero(C).item() == 0 and not torch.isnan(C).any()
    C = torch.full((0, 5), 1.0, device=DEV)
    _run(torch.empty((0, 3), device=DEV), torch.ones((3, 5), device=DEV), out=C)
    C = torch.full((4, 1), 3.0, device=DEV)
    assert tdb.gemm_f32(4, 0, 3, 0, 3, 0, 1, C.data_ptr(), 1, None) == tdb.OK
    torch.cuda.synchronize()
    assert torch.all(C == 3.0)


def test_closed_forms_on_gpu():
    n = 257
    B = ti.grid_matrix(91, 2, n, n)
    I = _dev(np.eye(n, dtype=np.float32))
    for v in ("sb", "db", "ms"):
        C = _run(I, _dev(B), v)
        assert torch.equal(C.cpu(), torch.from_numpy(B)), "identity"
        ones = torch.ones((130, 1000), device=DEV)
        C = _run(ones, torch.ones((1000, 70), device=DEV), v)
        assert torch.all(C == 1000.0), "all-ones"
        u = ti.grid_matrix(92, 1, 300, 1)
        w = ti.grid_matrix(92, 2, 1, 200)
        C = _run(_dev(u), _dev(w), v)
        exact = np.outer(u[:, 0].astype(np.float64), w[0].astype(np.float64))
        assert np.array_equal(C.cpu().numpy(), exact.astype(np.float32)), "rank-1"


def test_deterministic():
    A, B, C64, Bnd = _workload("square_1024")
    Ad, Bd = _dev(A), _dev(B)
    C1 = _run(Ad, Bd).clone()
    for _ in range(3):
        assert torch.equal(_run(Ad, Bd), C1)


def test_non_default_stream():
    A, B, C64, Bnd = _workload("ragged_513x257x129")
    s = torch.cuda.Stream()
    Ad, Bd = _dev(A), _dev(B)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = tdb.matmul(Ad, Bd, stream=s)
    s.synchronize()
    assert _ratio(C, C64, Bnd) <= 1.0


def test_alias_rejected_on_device():
    A = torch.ones((64, 64), device=DEV)
    B = torch.ones((64, 64), device=DEV)
    with pytest.raises(tdb.GemmError) as e:
        tdb.matmul(A, B, out=A)
    assert e.value.code == tdb.ERR_ALIAS
    torch.cuda.synchronize()
    assert torch.all(A == 1.0)


@pytest.mark.slow
def test_square_4096_full():
    _say("[parity] square_4096 oracle (full output) ...")
    A, B, C64, Bnd = _workload("square_4096")
    Ad, Bd = _dev(A), _dev(B)
    Cauto = _run(Ad, Bd, "auto").clone()
    r = _ratio(Cauto, C64, Bnd)
    _say(f"[parity] square_4096 auto ratio={r:.3g}")
    assert r <= 1.0
    ids = {"sb": tdb.VARIANT_SB, "db": tdb.VARIANT_DB, "ms": tdb.VARIANT_MS}
    for v in ("sb", "db", "ms"):
        cfg = tdb.gemm_f32_select_cfg(4096, 4096, 4096, ids[v])
        C = _run(Ad, Bd, v).clone()
        assert _ratio(C, C64, Bnd) <= 1.0, v
        for other_v in ("sb", "db", "ms"):
            if other_v != v:
                other = _run(Ad, Bd, other_v, cfg)
                assert torch.equal(C, other), f"{v} cfg {cfg}: {v} and {other_v} differ"


def test_square_3072_full_on_192_tiles():
    """3072^3 is 16 x 16 tiles of 192 x 192, one per compute unit: the dispatched product
    and both 192-wide configurations in every variant, checked on the full output, with
    the variants bit for bit equal per configuration."""
    M = N = K = 3072
    _say("[parity] 3072^3 oracle (full output) ...")
    A, B = ti.workload_inputs(M, N, K, 3072)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    assert _ratio(_run(Ad, Bd, "auto"), C64, Bnd) <= 1.0
    wide = [c for c in range(NCFG)
            if tdb.gemm_f32_config_info(c)[1]["BM"] == 192 == tdb.gemm_f32_config_info(c)[1]["BN"]]
    assert wide
    for cfg in wide:
        _say(f"[parity] 3072^3 cfg={cfg}")
        Cdb = _run(Ad, Bd, "db", cfg).clone()
        assert _ratio(Cdb, C64, Bnd) <= 1.0, cfg
        for v in ("sb", "ms", "sb3"):
            assert torch.equal(_run(Ad, Bd, v, cfg), Cdb), (cfg, v)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["square_8192", "shard_1024x8192x8192"])
def test_large_workload_sampled(name):
    """8192^3, and the one-GPU share of its eight-way row split (1024 x 8192 x 8192), in the
    launch configuration the benchmark times (dispatcher), checked on the workload's 4096
    seeded output positions, plus the same positions for the SB, DB and MS variants."""
    M, N, K, seed = ti.WORKLOADS[name]
    _say(f"[parity] {name} generating inputs ...")
    A, B = ti.workload_inputs(M, N, K, seed)
    ri, rj = ti.sample_positions(seed, M, N, 4096)
    c64, bnd = oracle.gemm_f64_sampled(A, B, ri, rj)
    Ad, Bd = _dev(A), _dev(B)
    del A, B
    ii, jj = torch.from_numpy(ri).to(DEV), torch.from_numpy(rj).to(DEV)
    for v in ("auto", "sb", "db", "ms"):
        C = _run(Ad, Bd, v)
        got = C[ii, jj].cpu().numpy()
        r = oracle.tolerance_ratio(got, c64, bnd)
        _say(f"[parity] {name} {v} sampled ratio={r:.3g}")
        assert r <= 1.0, v
        assert torch.isfinite(C).all()
        del C


@pytest.mark.parametrize("shape,splits", [((16, 4096, 4096), 4), ((64, 2048, 8192), 8),
                                          ((33, 257, 1000), 3), ((300, 200, 777), 2),
                                          ((128, 128, 4096), 16), ((7, 9, 130), 5)])
def test_splitk_parity(shape, splits):
    """Split-K: each K chunk's partial product in the workspace, a fixed-order sum into C.
    Within the bound; deterministic; the workspace size the library asks for suffices."""
    M, N, K = shape
    _say(f"[splitk] {M}x{N}x{K} splits={splits}")
    A, B = ti.workload_inputs(M, N, K, 8000 + M + K)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    need = tdb.gemm_f32_splitk_workspace(M, N, K, splits)
    ws = torch.full((max(need, 1),), float("nan"), device=DEV)
    C = torch.full((M, N), float("nan"), device=DEV)
    tdb.matmul_splitk(Ad, Bd, splits, out=C, workspace=ws)
    torch.cuda.synchronize()
    r = _ratio(C, C64, Bnd)
    _say(f"[splitk] ratio={r:.3g}")
    assert r <= 1.0
    C2 = tdb.matmul_splitk(Ad, Bd, splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C, C2), "split-K is not deterministic"


@pytest.mark.parametrize("shape,splits", [((1100, 1100, 300), -4), ((1536, 1536, 1536), -8),
                                          ((1000, 1300, 257), -3), ((1536, 1536, 700), 0),
                                          ((300, 200, 777), -2)])
def test_splitk_tail_parity(shape, splits):
    """Tail split (negative split counts, or the automatic choice): the tiles of the full
    rounds of workgroups run whole into C, only the last round's tiles are split into
    packed blocks of the workspace and summed into C.  Within the bound; deterministic;
    the workspace the library asks for suffices (NaN-filled, so a block that is read but
    never written would show).  A product with no full round splits every tile."""
    M, N, K = shape
    _say(f"[splitk-tail] {M}x{N}x{K} splits={splits} "
         f"(chosen {tdb.gemm_f32_splitk_select(M, N, K) if splits == 0 else splits})")
    A, B = ti.workload_inputs(M, N, K, 8100 + M + K)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    need = tdb.gemm_f32_splitk_workspace(M, N, K, splits)
    ws = torch.full((max(need, 1),), float("nan"), device=DEV)
    C = torch.full((M, N), float("nan"), device=DEV)
    tdb.matmul_splitk(Ad, Bd, splits, out=C, workspace=ws)
    torch.cuda.synchronize()
    r = _ratio(C, C64, Bnd)
    _say(f"[splitk-tail] ratio={r:.3g}")
    assert r <= 1.0
    C2 = tdb.matmul_splitk(Ad, Bd, splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C, C2), "tail split is not deterministic"


def _split_cases(n=16, seed=4242):
    """Seeded split-K products.  Half are small (M, N log-uniform in 64..1600, K in
    64..1200) with full, tail and modelled counts; half are large enough for a full round
    of tiles plus a tail (M, N in 1000..2200, K in 64..600) with tail and modelled counts."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        if i % 2 == 0:
            lo, hi, khi, counts = 64.0, 1600.0, 1200.0, [-8, -4, -2, 2, 3, 4, 8, 0]
        else:
            lo, hi, khi, counts = 1000.0, 2200.0, 600.0, [-8, -4, -3, -2, 0]
        M, N = (int(np.exp(rng.uniform(np.log(lo), np.log(hi)))) for _ in range(2))
        K = int(np.exp(rng.uniform(np.log(64.0), np.log(khi))))
        cases.append((i, M, N, K, counts[int(rng.integers(len(counts)))]))
    return cases


@pytest.mark.parametrize("case", _split_cases(), ids=lambda c: f"s{c[0]}")
def test_splitk_random_shapes(case):
    """Every split mode on seeded ragged shapes, C and the workspace NaN-filled."""
    i, M, N, K, splits = case
    _say(f"[splitk-random] {M}x{N}x{K} splits={splits}")
    A, B = ti.workload_inputs(M, N, K, 8200 + i)
    C64, Bnd = oracle.gemm_f64(A, B)
    need = tdb.gemm_f32_splitk_workspace(M, N, K, splits)
    ws = torch.full((max(need, 1),), float("nan"), device=DEV)
    C = torch.full((M, N), float("nan"), device=DEV)
    tdb.matmul_splitk(_dev(A), _dev(B), splits, out=C, workspace=ws)
    torch.cuda.synchronize()
    r = _ratio(C, C64, Bnd)
    assert r <= 1.0, (M, N, K, splits, r)


def test_splitk_one_split_equals_plain_and_errors():
    A, B, C64, Bnd = _workload("square_128")
    Ad, Bd = _dev(A), _dev(B)
    C1 = tdb.matmul_splitk(Ad, Bd, 1)
    C0 = _run(Ad, Bd)
    assert torch.equal(C1, C0)
    # too small a workspace is rejected before anything is launched
    M, N, K = 64, 512, 4096
    Ad = torch.ones((M, K), device=DEV)
    Bd = torch.ones((K, N), device=DEV)
    need = tdb.gemm_f32_splitk_workspace(M, N, K, 4)
    with pytest.raises(tdb.GemmError) as e:
        tdb.matmul_splitk(Ad, Bd, 4, workspace=torch.empty(need - 1, device=DEV))
    assert e.value.code == tdb.ERR_BAD_LD
    C = tdb.matmul_splitk(Ad, Bd, 4)
    torch.cuda.synchronize()
    assert torch.all(C == float(K))


def test_offsets_beyond_2gib():
    """32768 x 32768 x 32: C is 4 GiB, so row offsets pass 2^31 bytes (64-bit addressing in
    the copies and the epilogue).  Checked at 4096 seeded positions plus the last row and
    the last column."""
    M = N = 32768
    K = 32
    _say("[big] 32768x32768x32 generating ...")
    A, B = ti.workload_inputs(M, N, K, 9001)
    Ad, Bd = _dev(A), _dev(B)
    C = torch.empty((M, N), device=DEV)
    ri, rj = ti.sample_positions(9001, M, N, 4096)
    ri = np.concatenate([ri, np.full(64, M - 1), np.arange(M - 64, M)])
    rj = np.concatenate([rj, np.arange(N - 64, N), np.full(64, N - 1)])
    c64, bnd = oracle.gemm_f64_sampled(A, B, ri, rj)
    ii, jj = torch.from_numpy(ri).to(DEV), torch.from_numpy(rj).to(DEV)
    for v in ("auto", "db", "ms"):
        _say(f"[big] {v}")
        _run(Ad, Bd, v, out=C)
        got = C[ii, jj].cpu().numpy()
        assert oracle.tolerance_ratio(got, c64, bnd) <= 1.0, v
    del C


@pytest.mark.parametrize("which", ["A", "B"])
def test_row_stride_beyond_32bit_tile_offsets(which):
    """A row stride so large that the byte offsets inside one tile pass 2^32 (more than
    4 GiB between a tile's first and last row): the 16-byte copies address a tile with a
    32-bit offset from its first element, so such operands must take the element-wise
    path, and the result must still be exact to the bound.  Each case allocates about
    4.2 GiB on the device."""
    M, N, K = 64, 256, 64
    A, B = ti.workload_inputs(M, N, K, 9200)
    C64, Bnd = oracle.gemm_f64(A, B)
    if which == "A":
        ld = (1 << 24) + 4                       # 64 rows x ld x 4 B > 2^32
        big = torch.empty((M - 1) * ld + K, device=DEV)
        Ad = big.as_strided((M, K), (ld, 1))
        Ad.copy_(torch.from_numpy(A))
        Bd = _dev(B)
    else:
        K = 32                                   # one K tile of 32 rows x ld x 4 B > 2^32
        A, B = ti.workload_inputs(M, N, K, 9201)
        C64, Bnd = oracle.gemm_f64(A, B)
        ld = (1 << 25) + 4
        big = torch.empty((K - 1) * ld + N, device=DEV)
        Bd = big.as_strided((K, N), (ld, 1))
        Bd.copy_(torch.from_numpy(B))
        Ad = _dev(A)
    for v, cfg in (("auto", -1), ("sb", 6), ("db", 6), ("ms", 6), ("db", 1)):
        _say(f"[ld32] {which} ld={ld} {v} cfg={cfg}")
        assert _ratio(_run(Ad, Bd, v, cfg), C64, Bnd) <= 1.0, (which, v, cfg)
    del big
    torch.cuda.empty_cache()


def test_large_odd_shapes():
    """Odd sizes large enough for every tile kind at once (interior, right and bottom edges,
    the K tail) with leading dimensions that are not multiples of 4: 1537x2049x1027 in full
    and 4095x4097x4093 on 4096 seeded positions plus its last row and column."""
    M, N, K = 1537, 2049, 1027
    A, B = ti.workload_inputs(M, N, K, 9400)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    for v in ("auto", "sb", "db", "ms"):
        r = _ratio(_run(Ad, Bd, v), C64, Bnd)
        _say(f"[odd] {M}x{N}x{K} {v} ratio={r:.3g}")
        assert r <= 1.0, v
    del Ad, Bd
    M, N, K = 4095, 4097, 4093
    A, B = ti.workload_inputs(M, N, K, 9401)
    ri, rj = ti.sample_positions(9401, M, N, 4096)
    ri = np.concatenate([ri, np.full(64, M - 1), np.arange(M - 64, M)])
    rj = np.concatenate([rj, np.arange(N - 64, N), np.full(64, N - 1)])
    c64, bnd = oracle.gemm_f64_sampled(A, B, ri, rj)
    Ad, Bd = _dev(A), _dev(B)
    ii, jj = torch.from_numpy(ri).to(DEV), torch.from_numpy(rj).to(DEV)
    for v in ("auto", "sb", "db", "ms"):
        C = _run(Ad, Bd, v)
        r = oracle.tolerance_ratio(C[ii, jj].cpu().numpy(), c64, bnd)
        _say(f"[odd] {M}x{N}x{K} {v} sampled ratio={r:.3g}")
        assert r <= 1.0, v


def test_wide_dynamic_range():
    """Rows of A and columns of B scaled by powers of two from 2^-30 to 2^30: every product
    stays a normal FP32 number and the bound is relative, so nothing may lose accuracy."""
    M, N, K = 200, 150, 700
    rng = np.random.default_rng(55)
    A, B = ti.workload_inputs(M, N, K, 9100)
    A = (A * np.ldexp(1.0, rng.integers(-30, 31, (M, 1)))).astype(np.float32)
    B = (B * np.ldexp(1.0, rng.integers(-30, 31, (1, N)))).astype(np.float32)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    for v in ("sb", "db", "ms"):
        assert _ratio(_run(Ad, Bd, v), C64, Bnd) <= 1.0, v


def test_long_k_full_output():
    """K = 16384 (twice the largest workload's K), full output checked."""
    M, N, K = 96, 80, 16384
    A, B = ti.workload_inputs(M, N, K, 9200)
    C64, Bnd = oracle.gemm_f64(A, B)
    Ad, Bd = _dev(A), _dev(B)
    for v in ("auto", "sb", "db", "ms"):
        r = _ratio(_run(Ad, Bd, v), C64, Bnd)
        _say(f"[longk] {v} ratio={r:.3g}")
        assert r <= 1.0, v


def test_raster_order_does_not_change_results(monkeypatch):
    """GEMMF32_RASTER only changes which workgroup computes which tile: bitwise equal."""
    A, B, C64, Bnd = _workload("ragged_513x257x129")
    Ad, Bd = _dev(A), _dev(B)
    M2, N2, K2 = 1100, 900, 300
    A2, B2 = ti.workload_inputs(M2, N2, K2, 9300)
    A2d, B2d = _dev(A2), _dev(B2)
    ref = [_run(Ad, Bd, v).clone() for v in ("db", "ms")]
    ref2 = [_run(A2d, B2d, v, 3).clone() for v in ("sb", "db")]
    for setting in ("1", "3", "16,noxcd", "255"):
        monkeypatch.setenv("GEMMF32_RASTER", setting)
        for r, v in zip(ref, ("db", "ms")):
            assert torch.equal(_run(Ad, Bd, v), r), (setting, v)
        for r, v in zip(ref2, ("sb", "db")):
            assert torch.equal(_run(A2d, B2d, v, 3), r), (setting, v)


def test_peak_probe_measures_the_matrix_pipe():
    """The ceiling probe runs, reports a plausible shader clock and per-wave cycle counts
    of at least one v_mfma_f32_32x32x2_f32 per 64 clocks (256 workgroups: one to three
    waves per SIMD, depending on how the dispatcher places them), and the attained rate
    stays below what 64 clocks per instruction allow at the measured clock."""
    import torch
    blocks, iters = 256, 64
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    rec = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert tdb.gemm_f32_peak_probe(blocks, iters, out.data_ptr(), rec.data_ptr(), s) == tdb.OK
    torch.cuda.synchronize()
    r = rec.view(-1, 2).cpu().numpy().astype(np.float64)
    assert (r > 0).all()
    ghz = r[:, 0].sum() / r[:, 1].sum() * 0.1
    assert 0.5 < ghz < 3.5, ghz
    per_mfma = r[:, 0] / (16 * iters)
    assert per_mfma.min() > 60.0 and per_mfma.max() < 64.0 * 3 * 1.2, per_mfma
    assert torch.isfinite(out).all()
    from tiled_double_buffered_amd import peak
    c = peak.mfma_ceiling(warm_s=0.05, launches=3)
    assert 0.5 * c["at_clock_tflops"] < c["value"] <= 1.02 * c["at_clock_tflops"], c


def test_hip_graph_capture_and_replay():
    """The library's launches can be captured in a HIP graph (they allocate nothing and
    record no memset): dispatched products of three shapes (one on the K-split kernel) and a
    split-K product with its workspace are captured once, then replayed five times with
    eager work and synchronizations between the replays.  Every replay matches the eager
    results bit for bit (same kernels, same order of additions)."""
    cases = [(128, 128, 128, 0), (513, 257, 129, 0), (16, 4096, 4096, 0), (64, 2048, 4096, 4)]
    ins, outs, eager, wss = [], [], [], []
    for i, (M, N, K, splits) in enumerate(cases):
        A, B = ti.workload_inputs(M, N, K, 9500 + i)
        Ad, Bd = _dev(A), _dev(B)
        ws = None
        if splits:
            ws = torch.empty(max(tdb.gemm_f32_splitk_workspace(M, N, K, splits), 1), device=DEV)
            ref = tdb.matmul_splitk(Ad, Bd, splits, workspace=ws)
        else:
            ref = tdb.matmul(Ad, Bd)
        ins.append((Ad, Bd))
        wss.append(ws)
        outs.append(torch.full((M, N), float("nan"), device=DEV))
        eager.append(ref)
    torch.cuda.synchronize()
    _say("[graph] capturing")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for (M, N, K, splits), (Ad, Bd), C, ws in zip(cases, ins, outs, wss):
                if splits:
                    tdb.matmul_splitk(Ad, Bd, splits, out=C, workspace=ws)
                else:
                    tdb.matmul(Ad, Bd, out=C)
    torch.cuda.synchronize()
    for rep in range(5):
        for C in outs:
            C.fill_(float("nan"))
        junk = tdb.matmul(ins[0][0], ins[0][1])  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph] replay {rep}")
        for C, ref in zip(outs, eager):
            assert torch.equal(C, ref), f"replay {rep} differs from the eager result"
        assert torch.equal(junk, eager[0])
