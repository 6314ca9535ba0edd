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

Extended operation (other element types, scale / bias / rectifier on store):
bf16_to_double(bits), f32_to_double(bits)   exact decoders (uint16 / uint32 in)
ulp_type(x, c_type)       spacing of binary16 / bfloat16 / binary32 at |x|
gemm_ex(A, B, b_layout, ab_type, alpha, bias, act[, I, J])
                          fp64 reference of act(alpha*sum + bias[j]) and its
                          tolerance magnitude |alpha|*sum|a*b| + |bias[j]|
check_ex(got, c_type, ref, tol_mag)   the tolerance test for any output type

``A`` is a 2-D numpy float16/uint16 array (M x K, row stride = its first
stride). ``B`` is K x N for ``b_layout="KxN"`` and N x K for ``"NxK"``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import raster  # noqa: F401  (re-exported submodule)

_HERE = os.path.dirname(os.path.abspath(__file__))
# TGEMM_ORACLE_LIB: another build of tgemm_ref.c (the sanitizer test tier)
_LIB_PATH = os.environ.get("TGEMM_ORACLE_LIB") or os.path.join(_HERE, "liboracle_tgemm.so")
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
    lib.ref_bf16_to_double.restype = ctypes.c_double
    lib.ref_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.ref_f32_to_double.restype = ctypes.c_double
    lib.ref_f32_to_double.argtypes = [ctypes.c_uint32]
    lib.ref_decode_bf16.restype = None
    lib.ref_decode_bf16.argtypes = [_I64, _P, _P]
    lib.ref_decode_f32.restype = None
    lib.ref_decode_f32.argtypes = [_I64, _P, _P]
    lib.ref_ulp_type.restype = ctypes.c_double
    lib.ref_ulp_type.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.ref_gemm_ex.restype = ctypes.c_int
    lib.ref_gemm_ex.argtypes = [_I64, _I64, _I64, _P, _I64, _P, _I64, ctypes.c_int, ctypes.c_int,
                                ctypes.c_double, _P, ctypes.c_int, _I64, _P, _P, _P, _P]
    lib.ref_check_ex.restype = _I64
    lib.ref_check_ex.argtypes = [_I64, ctypes.c_int, _P, _P, _P, _P, ctypes.c_double, _P, _P, _I64]
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


# ------------------------------------------------- extended operation --

# element type codes: 0 binary16, 1 bfloat16, 2 binary32
_TYPES = {"f16": 0, "bf16": 1, "f32": 2, 0: 0, 1: 1, 2: 2}
_ACTS = {"none": 0, "relu": 1, 0: 0, 1: 1}


def bf16_to_double(bits: np.ndarray) -> np.ndarray:
    src = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    out = np.empty(src.shape, dtype=np.float64)
    _load().ref_decode_bf16(src.size, _ptr(src), _ptr(out))
    return out


def f32_to_double(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits)
    if b.dtype == np.float32:
        b = b.view(np.uint32)
    src = np.ascontiguousarray(b, dtype=np.uint32)
    out = np.empty(src.shape, dtype=np.float64)
    _load().ref_decode_f32(src.size, _ptr(src), _ptr(out))
    return out


def ulp_type(x: float, c_type) -> float:
    return float(_load().ref_ulp_type(float(x), _TYPES[c_type]))


def _u16(x) -> np.ndarray:
    """binary16 or bfloat16 operand as uint16 bit patterns (float16 arrays are viewed)."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    if x.dtype == np.uint16:
        return x
    raise TypeError(f"expected float16 or uint16 bit patterns, got {x.dtype}")


def _operand(x, ab: int) -> np.ndarray:
    """Operand bit patterns of type code ab: uint16 for 0/1, uint32 for 2 (float32 arrays are viewed)."""
    if ab != 2:
        return _u16(x)
    x = np.asarray(x)
    if x.dtype == np.float32:
        return x.view(np.uint32)
    if x.dtype == np.uint32:
        return x
    raise TypeError(f"expected float32 or uint32 bit patterns, got {x.dtype}")


def gemm_ex(A, B, b_layout, ab_type="f16", alpha=1.0, bias=None, act="none", I=None, J=None):
    """fp64 reference of act(alpha * sum_k A[i,k] B[k,j] + bias[j]) and its
    tolerance magnitude |alpha| * sum_k |A[i,k] B[k,j]| + |bias[j]|.

    A, B: bit patterns of ``ab_type`` (uint16 for "f16" / "bf16", float16
    arrays accepted for binary16; float32 or uint32 for "f32"). bias: None or
    N float32 values. I, J: None for the full M x N output (returned as 2-D
    arrays), else the selected elements (1-D)."""
    A = _operand(A, _TYPES[ab_type])
    B = _operand(B, _TYPES[ab_type])
    lay = _LAYOUTS[b_layout]
    M, K, lda = _rows(A)
    if lay == 0:
        Kb, N, ldb = _rows(B)
    else:
        N, Kb, ldb = _rows(B)
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A has K={K}, B has K={Kb}")
    bptr = None
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError(f"bias must hold N={N} values")
        bptr = _ptr(bias)
    if I is None:
        ref = np.empty((M, N), dtype=np.float64)
        tol = np.empty((M, N), dtype=np.float64)
        npts, ip, jp = -1, None, None
    else:
        I = np.ascontiguousarray(I, dtype=np.int64)
        J = np.ascontiguousarray(J, dtype=np.int64)
        if I.shape != J.shape:
            raise ValueError("I and J differ in shape")
        ref = np.empty(I.size, dtype=np.float64)
        tol = np.empty(I.size, dtype=np.float64)
        npts, ip, jp = I.size, _ptr(I), _ptr(J)
    rc = _load().ref_gemm_ex(M, N, K, _ptr(A), lda, _ptr(B), ldb, lay, _TYPES[ab_type], float(alpha), bptr,
                             _ACTS[act], npts, ip, jp, _ptr(ref), _ptr(tol))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return ref, tol


def check_ex(got, c_type, ref, tol_mag, rel: float = 1e-3, max_report: int = 10) -> dict:
    """Tolerance test for outputs of type c_type ("f16", "bf16": uint16 bit
    patterns or float16; "f32": float32 or uint32 bit patterns):
    |g - ref| <= rel * tol_mag + ulp_type(ref) per element."""
    t = _TYPES[c_type]
    g = np.asarray(got)
    if t == 2:
        g = np.ascontiguousarray(g.view(np.uint32) if g.dtype == np.float32 else g, dtype=np.uint32).ravel()
        g16, g32 = None, _ptr(g)
    else:
        g = np.ascontiguousarray(_u16(g)).ravel()
        g16, g32 = _ptr(g), None
    r = np.ascontiguousarray(ref, dtype=np.float64).ravel()
    s = np.ascontiguousarray(tol_mag, dtype=np.float64).ravel()
    if not (g.size == r.size == s.size):
        raise ValueError("got/ref/tol_mag sizes differ")
    worst = np.zeros(1, dtype=np.float64)
    first = np.full(max(max_report, 1), -1, dtype=np.int64)
    nfail = int(_load().ref_check_ex(g.size, t, g16, g32, _ptr(r), _ptr(s), float(rel), _ptr(worst), _ptr(first),
                                     max_report))
    return {"n": int(g.size), "nfail": nfail, "worst": float(worst[0]),
            "first_fail": [int(x) for x in first[:min(nfail, max_report)]]}
