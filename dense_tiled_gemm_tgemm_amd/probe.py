"""ctypes binding of libtgemm_probe.so, the measurement aids of
include/tgemm_probe.h (argument marshalling only). Not part of the GEMM: the
benchmark uses the matrix-core ceiling probe to attribute its fraction of
peak, and a test uses the die probe to check the dispatch order the raster
assumes."""
from __future__ import annotations

import ctypes
import os

from ._binding import TGEMM_OK, TgemmError

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_PKG, "libtgemm_probe.so")

_lib = None
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_INT = ctypes.c_int


def load():
    """Load libtgemm_probe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(
            f"{PROBE_LIB_PATH} is missing: build the HIP libraries first "
            "(python -m dense_tiled_gemm_tgemm_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    lib.tgemm_mfma_issue_probe.restype = _INT
    lib.tgemm_mfma_issue_probe.argtypes = [_I64, _INT, _P, _I64, _P, _P, _P]
    lib.tgemm_mfma_stream_probe.restype = _INT
    lib.tgemm_mfma_stream_probe.argtypes = [_INT, _I64, _INT, _P, _I64, _P, _P, _P]
    lib.tgemm_xcd_probe.restype = _INT
    lib.tgemm_xcd_probe.argtypes = [_I64, _P, _P]
    _lib = lib
    return lib


def mfma_issue_probe(workgroups: int, iters: int, data_ptr: int, data_bytes: int, out_ptr: int,
                     clocks_ptr=None, stream=None) -> None:
    """Launch the matrix-core ceiling probe (include/tgemm_probe.h)."""
    rc = int(load().tgemm_mfma_issue_probe(int(workgroups), int(iters), data_ptr, int(data_bytes), out_ptr,
                                           clocks_ptr, stream))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "mfma_issue_probe")


# instruction-stream probe kinds (include/tgemm_probe.h): name -> (code,
# threads per workgroup, flops per workgroup and round)
STREAM_KINDS = {
    "f16_mfma": (0, 256, 1 << 23),
    "f16_reads": (1, 256, 1 << 23),
    "f16_gemm": (2, 256, 1 << 23),
    "f16_gemm_no_barrier": (3, 256, 1 << 23),
    "f16_half_loads": (4, 256, 1 << 23),
    "f16_vgpr_loads": (5, 256, 1 << 23),
    "f16_lds_writes": (6, 256, 1 << 23),
    "f16_32x32": (7, 256, 1 << 23),
    "f16_32x32_gemm": (8, 256, 1 << 23),
    "f16_8w_mfma": (9, 512, 1 << 23),
    "f16_8w_gemm": (10, 512, 1 << 23),
    "f32_gemm": (11, 256, 1 << 22),
}


def mfma_stream_probe(kind: str, workgroups: int, iters: int, data_ptr: int, data_bytes: int, out_ptr: int,
                      clocks_ptr=None, stream=None) -> None:
    """Launch one instruction-stream probe (include/tgemm_probe.h); `kind` is
    a key of STREAM_KINDS, `out` holds workgroups x its threads floats."""
    rc = int(load().tgemm_mfma_stream_probe(STREAM_KINDS[kind][0], int(workgroups), int(iters), data_ptr,
                                            int(data_bytes), out_ptr, clocks_ptr, stream))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "mfma_stream_probe")


def xcd_probe(workgroups: int, out_ptr: int, stream=None) -> None:
    """Launch the die probe (include/tgemm_probe.h): out[w] = die of workgroup w."""
    rc = int(load().tgemm_xcd_probe(int(workgroups), out_ptr, stream))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "xcd_probe")
