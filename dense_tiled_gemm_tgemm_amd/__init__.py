"""tgemm: dense tiled matrix product for MI355X (gfx950): binary16 in and out
(``mm``), or binary16 / bfloat16 in with binary16, bfloat16 or fp32 out and a
scale / bias / rectifier epilogue (``gemm``).

The compute path is the HIP library ``libtgemm.so`` (C ABI in
include/tgemm.h); this package only marshals arguments to it and raises if
the library has not been built.
"""
from ._binding import (  # noqa: F401
    LIB_PATH,
    TGEMM_B_KxN,
    TGEMM_B_NxK,
    TGEMM_ERR_HIP,
    TGEMM_ERR_INVALID,
    TGEMM_ERR_UNSUPPORTED,
    TGEMM_OK,
    TGEMM_F16,
    TGEMM_BF16,
    TGEMM_F32,
    TGEMM_ACT_NONE,
    TGEMM_ACT_RELU,
    TgemmError,
    last_hip_error,
    gemm,
    load,
    mm,
    status_string,
    tgemm_f16,
    tgemm_f16_config,
    tgemm_gemm,
    tgemm_gemm_config,
    tgemm_plan_f16,
    tgemm_plan_gemm,
    tgemm_tile_of,
    tgemm_tune_gemm,
    tune,
    tuning_clear,
    tuning_entries,
)
