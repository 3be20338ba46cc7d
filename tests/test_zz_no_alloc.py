"""gemm_f32_splitk_noalloc: the allocation-free split-K entry point, through the C ABI.

Its output must equal that of gemm_f32_splitk with a caller-owned workspace bit for bit
(the same plan, kernels and fixed reduction order), and both must meet the oracle's bound.
Two calls in a row per case, the second smaller, so the second reads a scratch array that
still holds the first call's partials."""
import sys

import numpy as np
import pytest

import oracle
import tdb_inputs as ti

torch = pytest.importorskip("torch")
import tiled_double_buffered_amd as tdb  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _inputs(M, N, K, seed):
    a, b = ti.workload_inputs(M, N, K, seed)
    c64, bnd = oracle.gemm_f64(a, b)
    return torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV), c64, bnd


def _noalloc(A, B, splits, stream):
    M, K = A.shape
    N = B.shape[1]
    C = torch.full((M, N), float("nan"), device=DEV)
    rc = tdb.gemm_f32_splitk_noalloc(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(),
                                     N, splits, stream.cuda_stream)
    assert rc == tdb.OK, tdb.gemm_f32_strerror(rc)
    return C


def _with_workspace(A, B, splits, stream):
    M, K = A.shape
    N = B.shape[1]
    C = torch.full((M, N), float("nan"), device=DEV)
    need = tdb.gemm_f32_splitk_workspace(M, N, K, splits)
    ws = torch.full((max(need, 1),), float("nan"), device=DEV)
    rc = tdb.gemm_f32_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N,
                             splits, ws.data_ptr(), ws.numel(), stream.cuda_stream)
    assert rc == tdb.OK, tdb.gemm_f32_strerror(rc)
    return C


# (first shape, second smaller shape, splits): full splits, tail splits, the modelled
# choice, and a ragged second call
CASES = [
    ((64, 2048, 4096, 8), (16, 512, 1000, 4)),
    ((1100, 1100, 300, -4), (513, 257, 129, -2)),
    ((16, 4096, 4096, 0), (7, 300, 2000, 0)),
    ((256, 256, 8192, 16), (33, 65, 700, 8)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0][:3]}-{c[1][:3]}")
@pytest.mark.parametrize("side_stream", [False, True])
def test_noalloc_equals_workspace_split(case, side_stream):
    stream = torch.cuda.Stream(DEV) if side_stream else torch.cuda.current_stream(DEV)
    for i, (M, N, K, splits) in enumerate(case):
        _say(f"[noalloc] call {i}: {M}x{N}x{K} splits {splits} side_stream {side_stream}")
        A, B, c64, bnd = _inputs(M, N, K, 9100 + 10 * i + M % 7)
        need = tdb.gemm_f32_splitk_workspace(M, N, K, splits)
        assert 0 <= need <= tdb.SCRATCH_FLOATS
        with torch.cuda.stream(stream):
            got = _noalloc(A, B, splits, stream)
            ref = _with_workspace(A, B, splits, stream)
        stream.synchronize()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), \
            f"noalloc differs from the workspace split at {M}x{N}x{K}"
        ratio = oracle.tolerance_ratio(g, c64, bnd)
        assert ratio <= 1.0, ratio


def test_noalloc_unsplit_and_empty_calls():
    """One chunk: the plain dispatched product (nothing touches the scratch); M = 0: a
    no-op; a split larger than the scratch: rejected before any launch."""
    A, B, c64, bnd = _inputs(128, 128, 64, 9201)
    s = torch.cuda.current_stream(DEV)
    C = _noalloc(A, B, 1, s)
    s.synchronize()
    plain = tdb.matmul(A, B)
    torch.cuda.synchronize()
    assert torch.equal(C, plain)
    assert oracle.tolerance_ratio(C.cpu().numpy(), c64, bnd) <= 1.0
    assert tdb.gemm_f32_splitk_noalloc(0, 16, 16, 0, 16, 0, 16, 0, 16, 4,
                                       s.cuda_stream) == tdb.OK
    M = N = K = 4096
    big = tdb.gemm_f32_splitk_workspace(M, N, K, 8)
    assert big > tdb.SCRATCH_FLOATS
    Ab = torch.empty((M, K), device=DEV)
    Bb = torch.empty((K, N), device=DEV)
    Cb = torch.empty((M, N), device=DEV)
    rc = tdb.gemm_f32_splitk_noalloc(M, N, K, Ab.data_ptr(), K, Bb.data_ptr(), N,
                                     Cb.data_ptr(), N, 8, s.cuda_stream)
    assert rc == tdb.ERR_SCRATCH_LIMIT
