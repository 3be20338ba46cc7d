"""gemmf32 for MI355X: FP32 C = A.B through LDS tiles with single- and double-buffered
K-loops, FP32 matrix-core micro-kernels and a measured per-shape dispatcher.

The compute path is the HIP library `libgemmf32.so` (C ABI in include/gemmf32.h); this
package only loads it and marshals arguments.  Build it with
`python -m tiled_double_buffered_amd.build`.
"""
from ._binding import (  # noqa: F401
    ERR_ALIAS, ERR_BAD_CONFIG, ERR_BAD_LD, ERR_HIP, ERR_MISALIGNED, ERR_NEGATIVE_DIM,
    ERR_NULL_PTR, ERR_SCRATCH_LIMIT, ERR_TOO_LARGE, OK, SCRATCH_FLOATS, SIGNATURES,
    VARIANT_AUTO, VARIANT_DB, VARIANT_KS, VARIANT_MS, VARIANT_SB, VARIANT_SB3, GemmError,
    gemm_f32, gemm_f32_config_info, gemm_f32_config_ks, gemm_f32_config_ms,
    gemm_f32_config_variants, gemm_f32_db, gemm_f32_ex, gemm_f32_last_hip_error, gemm_f32_ms,
    gemm_f32_num_configs, gemm_f32_peak_probe, gemm_f32_sb, gemm_f32_select,
    gemm_f32_select_cfg, gemm_f32_splitk, gemm_f32_splitk_noalloc, gemm_f32_splitk_plan,
    gemm_f32_splitk_select, gemm_f32_splitk_workspace, gemm_f32_strerror, gemm_f32_version,
    load, matmul, matmul_splitk,
)

__version__ = "0.1.0"
