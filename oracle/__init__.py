"""CPU oracle for the fp16 tiled matrix product (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product (the HIP library and its
Python binding) never imports, links or calls anything here, and the two share
no code: the oracle decodes binary16 from its IEEE 754 field definition and
sums exact products in fp64 (see ``tgemm_ref.c`` for the passages it follows).

Functions
---------
half_to_double(bits)      exact binary16 -> float64 decode (numpy uint16 in)
ulp16(x)                  binary16 spacing at |x|
gemm(A, B, b_layout)      fp64 reference and sum|a*b| for every output element
gemm_points(A, B, b_layout, I, J)   the same for selected (i, j)
check(got, ref, absum)    the per-element tolerance test
raster                    submodule: the pages' block-id -> tile maps

``A`` is a 2-D numpy float16/uint16 array (M x K, row stride = its first
stride). ``B`` is K x N for ``b_layout="KxN"`` and N x K for ``"NxK"``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import raster  # noqa: F401  (re-exported submodule)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_tgemm.so")
_lib = None

_I64 = ctypes.c_int64
_P = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.ref_half_to_double.restype = ctypes.c_double
    lib.ref_half_to_double.argtypes = [ctypes.c_uint16]
    lib.ref_decode_f16.restype = None
    lib.ref_decode_f16.argtypes = [_I64, _P, _P]
    lib.ref_ulp16.restype = ctypes.c_double
    lib.ref_ulp16.argtypes = [ctypes.c_double]
    lib.ref_num_threads.restype = ctypes.c_int
    lib.ref_num_threads.argtypes = []
    lib.ref_gemm_f16.restype = ctypes.c_int
    lib.ref_gemm_f16.argtypes = [_I64, _I64, _I64, _P, _I64, _P, _I64, ctypes.c_int,
                                 _I64, _P, _P, _P, _P]
    lib.ref_check_f16.restype = _I64
    lib.ref_check_f16.argtypes = [_I64, _P, _P, _P, ctypes.c_double, _P, _P, _I64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits(x: np.ndarray) -> np.ndarray:
    """View a float16/uint16 array as uint16 bit patterns (no copy of data)."""
    if x.dtype == np.float16:
        return x.view(np.uint16)
    if x.dtype == np.uint16:
        return x
    raise TypeError(f"expected float16 or uint16 bits, got {x.dtype}")


def _rows(x: np.ndarray):
    """(rows, cols, row stride in elements) of a 2-D array with unit column stride."""
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    if x.size == 0:
        return x.shape[0], x.shape[1], max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != x.itemsize:
        raise ValueError("columns must be contiguous")
    ld = x.strides[0] // x.itemsize if x.shape[0] > 1 else max(x.shape[1], 1)
    return x.shape[0], x.shape[1], ld


def num_threads() -> int:
    return int(_load().ref_num_threads())


def half_to_double(bits: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(_bits(np.asarray(bits)))
    out = np.empty(src.shape, dtype=np.float64)
    _load().ref_decode_f16(src.size, _ptr(src), _ptr(out))
    return out


def ulp16(x: float) -> float:
    return float(_load().ref_ulp16(float(x)))


_LAYOUTS = {"KxN": 0, "NxK": 1, 0: 0, 1: 1}


def _operands(A, B, b_layout):
    A = _bits(np.asarray(A))
    B = _bits(np.asarray(B))
    lay = _LAYOUTS[b_layout]
    M, K, lda = _rows(A)
    if lay == 0:
        Kb, N, ldb = _rows(B)
    else:
        N, Kb, ldb = _rows(B)
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A has K={K}, B has K={Kb}")
    return A, B, lay, M, N, K, lda, ldb


def gemm_points(A, B, b_layout, I, J):
    """fp64 reference and sum|a*b| at output elements (I[p], J[p])."""
    A, B, lay, M, N, K, lda, ldb = _operands(A, B, b_layout)
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape:
        raise ValueError("I and J differ in shape")
    ref = np.empty(I.size, dtype=np.float64)
    absum = np.empty(I.size, dtype=np.float64)
    rc = _load().ref_gemm_f16(M, N, K, _ptr(A), lda, _ptr(B), ldb, lay,
                              I.size, _ptr(I), _ptr(J), _ptr(ref), _ptr(absum))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return ref, absum


def gemm(A, B, b_layout):
    """fp64 reference and sum|a*b| for the whole M x N output (row-major)."""
    A, B, lay, M, N, K, lda, ldb = _operands(A, B, b_layout)
    ref = np.empty((M, N), dtype=np.float64)
    absum = np.empty((M, N), dtype=np.float64)
    rc = _load().ref_gemm_f16(M, N, K, _ptr(A), lda, _ptr(B), ldb, lay,
                              -1, None, None, _ptr(ref), _ptr(absum))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return ref, absum


def check(got, ref, absum, rel: float = 1e-3, max_report: int = 10) -> dict:
    """Tolerance test: |g - ref| <= rel*absum + ulp16(ref) per element."""
    g = np.ascontiguousarray(_bits(np.asarray(got))).ravel()
    r = np.ascontiguousarray(ref, dtype=np.float64).ravel()
    s = np.ascontiguousarray(absum, dtype=np.float64).ravel()
    if not (g.size == r.size == s.size):
        raise ValueError("got/ref/absum sizes differ")
    worst = np.zeros(1, dtype=np.float64)
    first = np.full(max(max_report, 1), -1, dtype=np.int64)
    nfail = int(_load().ref_check_f16(g.size, _ptr(g), _ptr(r), _ptr(s), float(rel),
                                      _ptr(worst), _ptr(first), max_report))
    return {"n": int(g.size), "nfail": nfail, "worst": float(worst[0]),
            "first_fail": [int(x) for x in first[:min(nfail, max_report)]]}
