"""ctypes binding of libgemmf32.so: the C-ABI entry points under the same names, plus a
tensor-level `matmul` that only marshals arguments (device pointers, leading dimensions,
the current stream) -- every step of the product runs in the library's HIP kernels.

There is no fallback: if the library is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgemmf32.so")
# the LDS-poison debug build of the same source (tests only)
LIB_POISON_PATH = os.path.join(_PKG, "libgemmf32_lds_poison.so")

OK = 0
ERR_NEGATIVE_DIM = -1
ERR_BAD_LD = -2
ERR_NULL_PTR = -3
ERR_MISALIGNED = -4
ERR_ALIAS = -5
ERR_TOO_LARGE = -6
ERR_BAD_CONFIG = -7
ERR_HIP = -8
ERR_SCRATCH_LIMIT = -9
SCRATCH_FLOATS = 8 * 1024 * 1024  # GEMMF32_SCRATCH_FLOATS

VARIANT_AUTO = 0
VARIANT_SB = 1
VARIANT_DB = 2
VARIANT_MS = 3
VARIANT_SB3 = 4
VARIANT_KS = 5
_VARIANTS = {"auto": VARIANT_AUTO, "sb": VARIANT_SB, "db": VARIANT_DB, "ms": VARIANT_MS,
             "sb3": VARIANT_SB3, "ks": VARIANT_KS}

# Every exported symbol and its C signature (kept in step with include/gemmf32.h).
_i64, _int, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_GEMM_ARGS = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
SIGNATURES = {
    "gemm_f32": (_int, _GEMM_ARGS + [_vp]),
    "gemm_f32_sb": (_int, _GEMM_ARGS + [_vp]),
    "gemm_f32_db": (_int, _GEMM_ARGS + [_vp]),
    "gemm_f32_ms": (_int, _GEMM_ARGS + [_vp]),
    "gemm_f32_ex": (_int, _GEMM_ARGS + [_int, _int, _vp]),
    "gemm_f32_splitk": (_int, _GEMM_ARGS + [_int, _vp, _i64, _vp]),
    "gemm_f32_splitk_noalloc": (_int, _GEMM_ARGS + [_int, _vp]),
    "gemm_f32_splitk_workspace": (_i64, [_i64, _i64, _i64, _int]),
    "gemm_f32_splitk_select": (_int, [_i64, _i64, _i64]),
    "gemm_f32_splitk_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_int),
                                    ctypes.POINTER(_int), ctypes.POINTER(_int),
                                    ctypes.POINTER(_i64)]),
    "gemm_f32_select": (_int, [_i64, _i64, _i64, ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "gemm_f32_select_cfg": (_int, [_i64, _i64, _i64, _int]),
    "gemm_f32_num_configs": (_int, []),
    "gemm_f32_config_info": (_int, [_int] + [ctypes.POINTER(_int)] * 6),
    "gemm_f32_config_ms": (_int, [_int, ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "gemm_f32_config_variants": (_int, [_int]),
    "gemm_f32_config_ks": (_int, [_int]),
    "gemm_f32_last_hip_error": (_int, []),
    "gemm_f32_strerror": (ctypes.c_char_p, [_int]),
    "gemm_f32_version": (ctypes.c_char_p, []),
    "gemm_f32_peak_probe": (_int, [_int, _int, _vp, _vp, _vp]),
}

_lib = None


class GemmError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        msg = strerror(code)
        if code == ERR_HIP:
            msg += f" (HIP error {gemm_f32_last_hip_error()})"
        super().__init__(f"{what}: {msg} [{code}]" if what else f"{msg} [{code}]")


def open_library(path: str):
    """A ctypes handle on a build of the library at `path`, every entry point typed.
    Raises if it is not built."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m tiled_double_buffered_amd.build`"
                           " (the GEMM has no fallback path)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path: str = LIB_PATH):
    """Load the library (once).  Raises if it is not built."""
    global _lib
    if _lib is None:
        _lib = open_library(path)
    return _lib


# ----------------------------------------------------------------------------- raw C ABI
def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_sb(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32_sb(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_db(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32_db(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_ms(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return load().gemm_f32_ms(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, variant, cfg_id, stream=None) -> int:
    return load().gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, variant, cfg_id, stream)


def gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace, workspace_floats,
                    stream=None) -> int:
    return load().gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, splits, workspace,
                                  workspace_floats, stream)


def gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, splits, stream=None) -> int:
    return load().gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, splits, stream)


def gemm_f32_splitk_workspace(M, N, K, splits) -> int:
    return load().gemm_f32_splitk_workspace(M, N, K, splits)


def gemm_f32_splitk_select(M, N, K) -> int:
    return load().gemm_f32_splitk_select(M, N, K)


def gemm_f32_splitk_plan(M, N, K, splits=0):
    """Returns (rc, dict): the variant and cfg of a split-K call's GEMM launch, its K chunks
    per split tile (1: no split) and the tiles that run whole over K (split_from)."""
    v, c, ch, sf = _int(0), _int(0), _int(0), _i64(0)
    rc = load().gemm_f32_splitk_plan(M, N, K, splits, ctypes.byref(v), ctypes.byref(c),
                                     ctypes.byref(ch), ctypes.byref(sf))
    return rc, {"variant": v.value, "cfg": c.value, "chunks": ch.value,
                "split_from": sf.value}


def gemm_f32_select(M, N, K):
    """Returns (rc, variant, cfg_id)."""
    v, c = _int(0), _int(0)
    rc = load().gemm_f32_select(M, N, K, ctypes.byref(v), ctypes.byref(c))
    return rc, v.value, c.value


def gemm_f32_select_cfg(M, N, K, variant) -> int:
    return load().gemm_f32_select_cfg(M, N, K, variant)


def gemm_f32_num_configs() -> int:
    return load().gemm_f32_num_configs()


def gemm_f32_config_info(cfg_id):
    """Returns (rc, dict) with BM, BN, BK, threads, lds_bytes_sb, lds_bytes_db."""
    vals = [_int(0) for _ in range(6)]
    rc = load().gemm_f32_config_info(cfg_id, *[ctypes.byref(v) for v in vals])
    keys = ("BM", "BN", "BK", "threads", "lds_bytes_sb", "lds_bytes_db")
    return rc, dict(zip(keys, (v.value for v in vals)))


def gemm_f32_config_variants(cfg_id) -> int:
    """Bit mask of the variants configuration cfg_id has a kernel for (bit v: variant v)."""
    return load().gemm_f32_config_variants(cfg_id)


def gemm_f32_config_ks(cfg_id) -> int:
    """Wave groups of configuration cfg_id's K-split kernel (1: it has none)."""
    return load().gemm_f32_config_ks(cfg_id)


def gemm_f32_config_ms(cfg_id):
    """Returns (rc, dict) with the multi-stage kernel's stages and lds_bytes."""
    st, lds = _int(0), _int(0)
    rc = load().gemm_f32_config_ms(cfg_id, ctypes.byref(st), ctypes.byref(lds))
    return rc, {"stages": st.value, "lds_bytes": lds.value}


def gemm_f32_last_hip_error() -> int:
    return load().gemm_f32_last_hip_error()


def gemm_f32_strerror(code) -> str:
    return load().gemm_f32_strerror(code).decode()


def gemm_f32_version() -> str:
    return load().gemm_f32_version().decode()


def gemm_f32_peak_probe(blocks, iters, out, rec, stream=None) -> int:
    return load().gemm_f32_peak_probe(blocks, iters, out, rec, stream)


strerror = gemm_f32_strerror


# ----------------------------------------------------------------------------- tensors
def _operand(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    if rows > 1 and t.stride(0) < max(cols, 1):
        # an expanded (stride 0) or overlapping view: its rows share storage, and passing
        # the row length as the leading dimension would make the library read or write
        # past the tensor's storage
        raise ValueError(f"{name} has row stride {t.stride(0)} < row length {cols}: "
                         "broadcast or overlapping rows are not supported")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU (the library takes device pointers)")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return t.data_ptr(), ld


def matmul(A, B, out=None, variant: str = "auto", cfg_id: int = -1, stream=None):
    """out = A @ B for row-major float32 GPU tensors through the C ABI.

    A is M x K, B is K x N, out (allocated when None) is M x N; any row stride >= the row
    length is passed as the leading dimension.  The launch goes on `stream` (a
    torch.cuda.Stream; default: the current stream) and is asynchronous."""
    import torch
    if variant not in _VARIANTS:
        raise ValueError(f"variant must be one of {sorted(_VARIANTS)}")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} @ {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    pa, lda = _operand(A, "A")
    pb, ldb = _operand(B, "B")
    pc, ldc = _operand(out, "out")
    s = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    rc = gemm_f32_ex(M, N, K, pa, lda, pb, ldb, pc, ldc, _VARIANTS[variant], cfg_id, s)
    if rc != OK:
        raise GemmError(rc, "gemm_f32")
    return out


def matmul_splitk(A, B, splits=0, out=None, workspace=None, stream=None):
    """out = A @ B through gemm_f32_splitk (`splits`: s > 0 splits every tile into s K
    chunks, -s only the tiles of the last partly filled round of workgroups, 0 the modelled
    choice).  `workspace` is a float32 GPU tensor of at least
    gemm_f32_splitk_workspace(M, N, K, splits) elements; when None, one is allocated here
    with torch (the library itself never allocates)."""
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} @ {tuple(B.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError("out has the wrong shape")
    pa, lda = _operand(A, "A")
    pb, ldb = _operand(B, "B")
    pc, ldc = _operand(out, "out")
    need = gemm_f32_splitk_workspace(M, N, K, splits)
    if need < 0:
        raise GemmError(int(need), "gemm_f32_splitk_workspace")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.float32, device=A.device)
    if workspace.dtype != torch.float32 or not workspace.is_cuda or \
            not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous float32 GPU tensor")
    s = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    rc = gemm_f32_splitk(M, N, K, pa, lda, pb, ldb, pc, ldc, splits, workspace.data_ptr(),
                         workspace.numel(), s)
    if rc != OK:
        raise GemmError(rc, "gemm_f32_splitk")
    return out
