"""The LDS-poison debug build on the GPU.

libgemmf32_lds_poison.so is the library's own source built with GEMMF32_LDS_POISON=1: right
after the barrier that frees an LDS slot (or multi-stage stage), every thread overwrites its
own part of it with NaN, and it does so at the start for every slot.  A kernel whose waves
read a slot after that barrier -- before the barrier that publishes the slot's next tile --
or read a slot never filled, would carry NaN into C.  The case study's argument is that the
one barrier of the double-buffered loop does that double duty, landing tile l+1 and freeing
tile l's buffer ("Case Study: The Double-Buffered GEMM", paragraph after the code figure);
this checks it on every kernel.

Every variant of every tile configuration must give, through the poison build, the same bits
as through the production build, and meet the oracle's bound."""
import sys

import numpy as np
import pytest

import oracle
import tdb_inputs as ti

torch = pytest.importorskip("torch")
import tiled_double_buffered_amd as tdb  # noqa: E402
from tiled_double_buffered_amd import _binding  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
NCFG = tdb.gemm_f32_num_configs()
VARIANTS = {"sb": tdb.VARIANT_SB, "db": tdb.VARIANT_DB, "ms": tdb.VARIANT_MS,
            "sb3": tdb.VARIANT_SB3, "ks": tdb.VARIANT_KS}


@pytest.fixture(scope="module")
def poison_lib():
    lib = _binding.open_library(_binding.LIB_POISON_PATH)
    assert lib.gemm_f32_version().decode().endswith("lds-poison")
    assert not tdb.gemm_f32_version().endswith("lds-poison")
    return lib


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _call(lib, A, B, C, variant, cfg):
    M, K = A.shape
    N = B.shape[1]
    rc = lib.gemm_f32_ex(M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0),
                         C.data_ptr(), C.stride(0), variant, cfg,
                         torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == tdb.OK, tdb.gemm_f32_strerror(rc)
    torch.cuda.synchronize()
    return C


# ragged in M, N and K (a K tail); aligned with many K tiles (the rings wrap many times);
# one K tile (the prologue alone); two K tiles
SHAPES = [(300, 333, 97, 51), (512, 512, 1024, 52), (130, 200, 16, 53), (257, 129, 64, 54)]


@pytest.mark.parametrize("cfg", range(NCFG))
def test_poison_build_matches_production_bit_for_bit(cfg, poison_lib):
    mask = tdb.gemm_f32_config_variants(cfg)
    for (M, N, K, seed) in SHAPES:
        A, B = ti.workload_inputs(M, N, K, seed)
        C64, Bnd = oracle.gemm_f64(A, B)
        Ad = torch.from_numpy(A).to(DEV)
        Bd = torch.from_numpy(B).to(DEV)
        for name, v in VARIANTS.items():
            if not mask & (1 << v):
                continue
            _say(f"[poison] cfg={cfg} {name} {M}x{N}x{K}")
            ref = _call(tdb.load(), Ad, Bd, torch.full((M, N), float("nan"), device=DEV), v,
                        cfg)
            got = _call(poison_lib, Ad, Bd, torch.full((M, N), float("nan"), device=DEV), v,
                        cfg)
            g = got.cpu().numpy()
            assert not np.isnan(g).any(), (cfg, name, M, N, K)
            assert oracle.tolerance_ratio(g, C64, Bnd) <= 1.0, (cfg, name, M, N, K)
            assert torch.equal(got, ref), (cfg, name, M, N, K)
