"""tgemm: fp16 dense tiled matrix product for MI355X (gfx950).

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
    TgemmError,
    last_hip_error,
    load,
    mfma_issue_probe,
    mm,
    status_string,
    tgemm_f16,
    tgemm_f16_config,
    tgemm_plan_f16,
    tgemm_tile_of,
)
