"""ctypes binding of libtgemm.so (argument marshalling only).

Every function here forwards to the C ABI declared in include/tgemm.h; all
arithmetic runs in the HIP kernels. If the library has not been built the
first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtgemm.so")

TGEMM_B_KxN = 0
TGEMM_B_NxK = 1
TGEMM_OK = 0
TGEMM_ERR_INVALID = -1
TGEMM_ERR_UNSUPPORTED = -2
TGEMM_ERR_HIP = -3
TGEMM_F16 = 0
TGEMM_BF16 = 1
TGEMM_F32 = 2
TGEMM_ACT_NONE = 0
TGEMM_ACT_RELU = 1

_LAYOUT = {"KxN": TGEMM_B_KxN, "NxK": TGEMM_B_NxK, TGEMM_B_KxN: TGEMM_B_KxN, TGEMM_B_NxK: TGEMM_B_NxK}
_DTYPE = {"f16": TGEMM_F16, "bf16": TGEMM_BF16, "f32": TGEMM_F32,
          TGEMM_F16: TGEMM_F16, TGEMM_BF16: TGEMM_BF16, TGEMM_F32: TGEMM_F32}
_ACT = {"none": TGEMM_ACT_NONE, "relu": TGEMM_ACT_RELU, TGEMM_ACT_NONE: TGEMM_ACT_NONE,
        TGEMM_ACT_RELU: TGEMM_ACT_RELU}



def _code(table, v):
    """Name -> C enum value; plain integers pass through unchanged (the C side checks them)."""
    return int(v) if isinstance(v, int) else table[v]


_lib = None
_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_INT = ctypes.c_int


class TgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = f"tgemm failed: {status_string(status)} ({status})"
        if status == TGEMM_ERR_HIP:
            msg += f", hipError_t {last_hip_error()}"
        if what:
            msg += f" [{what}]"
        super().__init__(msg)


def load():
    """Load libtgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m dense_tiled_gemm_tgemm_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    gemm_args = [_I64, _I64, _I64, _P, _I64, _P, _I64, _INT, _P, _I64, _P]
    lib.tgemm_f16.restype = _INT
    lib.tgemm_f16.argtypes = gemm_args
    lib.tgemm_f16_config.restype = _INT
    lib.tgemm_f16_config.argtypes = gemm_args + [_INT, _INT, _INT, _INT, _INT, _INT, _INT]
    ex_args = [_I64, _I64, _I64, _INT, _P, _I64, _P, _I64, _INT, _INT, _P, _I64, ctypes.c_float, _P, _INT]
    lib.tgemm_gemm.restype = _INT
    lib.tgemm_gemm.argtypes = ex_args + [_P]
    lib.tgemm_gemm_config.restype = _INT
    lib.tgemm_gemm_config.argtypes = ex_args + [_P, _INT, _INT, _INT, _INT, _INT, _INT, _INT]
    lib.tgemm_plan_gemm.restype = _INT
    lib.tgemm_plan_gemm.argtypes = ex_args + [_INT, _INT, _INT, _INT, _INT, _INT, _INT, _INT, ctypes.POINTER(_I64)]
    lib.tgemm_tune_gemm.restype = _INT
    lib.tgemm_tune_gemm.argtypes = ex_args + [_P, _INT, ctypes.POINTER(_I64)]
    lib.tgemm_tuning_entries.restype = _INT
    lib.tgemm_tuning_entries.argtypes = []
    lib.tgemm_tuning_clear.restype = None
    lib.tgemm_tuning_clear.argtypes = []
    lib.tgemm_status_string.restype = ctypes.c_char_p
    lib.tgemm_status_string.argtypes = [_INT]
    lib.tgemm_last_hip_error.restype = _INT
    lib.tgemm_last_hip_error.argtypes = []
    lib.tgemm_plan_f16.restype = _INT
    lib.tgemm_plan_f16.argtypes = [_I64, _I64, _I64, _P, _I64, _P, _I64, _INT, _P, _I64,
                                   _INT, _INT, _INT, _INT, _INT, _INT, _INT, _INT, ctypes.POINTER(_I64)]
    lib.tgemm_tile_of.restype = _INT
    lib.tgemm_tile_of.argtypes = [_I64, _I64, _INT, _INT, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().tgemm_status_string(int(status)).decode()


def last_hip_error() -> int:
    return int(load().tgemm_last_hip_error())


def tgemm_f16(M, N, K, A, lda, B, ldb, b_layout, C, ldc, stream=None) -> int:
    """Raw C call: pointers are integers (device addresses); returns the status."""
    return int(load().tgemm_f16(M, N, K, A, lda, B, ldb, _LAYOUT[b_layout], C, ldc, stream))


def tgemm_f16_config(M, N, K, A, lda, B, ldb, b_layout, C, ldc, stream=None,
                     force_generic=0, group_m=0, num_xcd=0, k_step=0, stages=0, tile_m=0, producers=0) -> int:
    return int(load().tgemm_f16_config(M, N, K, A, lda, B, ldb, _LAYOUT[b_layout], C, ldc, stream,
                                       int(force_generic), int(group_m), int(num_xcd), int(k_step),
                                       int(stages), int(tile_m), int(producers)))


def tgemm_plan_f16(M, N, K, A, lda, B, ldb, b_layout, C, ldc, force_generic=0, group_m=0, num_xcd=0,
                   k_step=0, stages=0, tile_m=0, producers=0, compute_units=0):
    """Plan query: (status, info dict or None). compute_units=0 asks the current device."""
    info = (_I64 * 10)()
    rc = int(load().tgemm_plan_f16(M, N, K, A, lda, B, ldb, _LAYOUT[b_layout], C, ldc,
                                   int(force_generic), int(group_m), int(num_xcd), int(k_step),
                                   int(stages), int(tile_m), int(producers), int(compute_units), info))
    if rc != TGEMM_OK:
        return rc, None
    keys = ("variant", "bm", "bn", "bk", "workgroups", "group_m", "num_xcd", "threads", "stages",
            "lds_bytes")
    return rc, dict(zip(keys, (int(v) for v in info)))


def tgemm_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha=1.0, bias=None, act="none",
               stream=None) -> int:
    """Raw C call of the typed GEMM with epilogue; returns the status."""
    return int(load().tgemm_gemm(M, N, K, _code(_DTYPE, ab_type), A, lda, B, ldb, _LAYOUT[b_layout], _code(_DTYPE, c_type), C,
                                 ldc, float(alpha), bias, _code(_ACT, act), stream))


def tgemm_gemm_config(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha=1.0, bias=None,
                      act="none", stream=None, force_generic=0, group_m=0, num_xcd=0, k_step=0, stages=0,
                      tile_m=0, producers=0) -> int:
    return int(load().tgemm_gemm_config(M, N, K, _code(_DTYPE, ab_type), A, lda, B, ldb, _LAYOUT[b_layout],
                                        _code(_DTYPE, c_type), C, ldc, float(alpha), bias, _code(_ACT, act), stream,
                                        int(force_generic), int(group_m), int(num_xcd), int(k_step), int(stages),
                                        int(tile_m), int(producers)))


_PLAN_KEYS = ("variant", "bm", "bn", "bk", "workgroups", "group_m", "num_xcd", "threads", "stages", "lds_bytes")


def tgemm_plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha=1.0, bias=None,
                    act="none", force_generic=0, group_m=0, num_xcd=0, k_step=0, stages=0, tile_m=0, producers=0,
                    compute_units=0):
    """Plan query of the typed GEMM: (status, info dict or None). compute_units=0 asks the current device."""
    info = (_I64 * 10)()
    rc = int(load().tgemm_plan_gemm(M, N, K, _code(_DTYPE, ab_type), A, lda, B, ldb, _LAYOUT[b_layout], _code(_DTYPE, c_type),
                                    C, ldc, float(alpha), bias, _code(_ACT, act), int(force_generic), int(group_m),
                                    int(num_xcd), int(k_step), int(stages), int(tile_m), int(producers),
                                    int(compute_units), info))
    if rc != TGEMM_OK:
        return rc, None
    return rc, dict(zip(_PLAN_KEYS, (int(v) for v in info)))


_TUNE_KEYS = ("k_step", "stages", "group_m", "num_xcd", "median_ns", "candidates", "tile_m", "producers")


def tgemm_tune_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha=1.0, bias=None, act="none",
                    stream=None, rounds=5):
    """Raw C call of the runtime tuner: (status, chosen launch dict or None)."""
    info = (_I64 * 8)()
    rc = int(load().tgemm_tune_gemm(M, N, K, _code(_DTYPE, ab_type), A, lda, B, ldb, _LAYOUT[b_layout],
                                    _code(_DTYPE, c_type), C, ldc, float(alpha), bias, _code(_ACT, act), stream,
                                    int(rounds), info))
    if rc != TGEMM_OK:
        return rc, None
    return rc, dict(zip(_TUNE_KEYS, (int(v) for v in info)))


def tuning_entries() -> int:
    return int(load().tgemm_tuning_entries())


def tuning_clear() -> None:
    load().tgemm_tuning_clear()


def tgemm_tile_of(grid_m, grid_n, group_m, num_xcd, wid):
    tm, tn = _I64(), _I64()
    rc = int(load().tgemm_tile_of(grid_m, grid_n, group_m, num_xcd, wid, ctypes.byref(tm), ctypes.byref(tn)))
    if rc != TGEMM_OK:
        raise TgemmError(rc, "tile_of")
    return tm.value, tn.value


# ----------------------------------------------------------- torch tensors --

def _row_major(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    ld = t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)
    return max(ld, 1)


def _check_tensor(t, name):
    import torch
    if t.dtype != torch.float16:
        raise TypeError(f"{name} must be torch.float16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _same_device(A, *others):
    """Every tensor on A's device (the library launches on the current device,
    which the callers set to A's)."""
    for t, name in others:
        if t is not None and t.device != A.device:
            raise ValueError(f"{name} is on {t.device}, A on {A.device}")


def mm(A, B, b_layout: str = "KxN", out=None, stream=None, force_generic: int = 0,
       group_m: int = 0, num_xcd: int = 0, k_step: int = 0, stages: int = 0, tile_m: int = 0,
       producers: int = 0):
    """C = A @ B for fp16 device tensors (fp32 accumulation in the kernel).

    A: (M, K). B: (K, N) when b_layout == "KxN", (N, K) when "NxK".
    out: optional (M, N) fp16 tensor with unit column stride; allocated with
    torch.empty when None. Runs on `stream` (default: torch's current stream).
    """
    import torch
    _check_tensor(A, "A")
    _check_tensor(B, "B")
    lay = _LAYOUT[b_layout]
    M, K = A.shape
    if lay == TGEMM_B_KxN:
        Kb, N = B.shape
    else:
        N, Kb = B.shape
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)} ({b_layout})")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    else:
        _check_tensor(out, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be ({M}, {N})")
    _same_device(A, (B, "B"), (out, "out"))
    lda, ldb, ldc = _row_major(A, "A"), _row_major(B, "B"), _row_major(out, "out")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    with torch.cuda.device(A.device):
        rc = tgemm_f16_config(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, lay, out.data_ptr(), ldc,
                              stream, force_generic, group_m, num_xcd, k_step, stages, tile_m, producers)
    if rc != TGEMM_OK:
        raise TgemmError(rc, f"M={M} N={N} K={K} layout={b_layout}")
    return out


def _torch_code(dtype):
    import torch
    codes = {torch.float16: TGEMM_F16, torch.bfloat16: TGEMM_BF16, torch.float32: TGEMM_F32}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}")
    return codes[dtype]


def tune(A, B, b_layout: str = "KxN", out=None, out_dtype=None, alpha: float = 1.0, bias=None, act: str = "none",
         stream=None, rounds: int = 5):
    """Time every launch choice of this problem on these tensors and record
    the fastest for its shape (later gemm / mm calls with automatic choices
    use it). Returns (C, chosen launch dict). Synchronizes the stream."""
    return gemm(A, B, b_layout, out, out_dtype, alpha, bias, act, stream, _tune_rounds=rounds)


def gemm(A, B, b_layout: str = "KxN", out=None, out_dtype=None, alpha: float = 1.0, bias=None, act: str = "none",
         stream=None, force_generic: int = 0, group_m: int = 0, num_xcd: int = 0, k_step: int = 0,
         stages: int = 0, tile_m: int = 0, producers: int = 0, _tune_rounds: int = 0):
    """C = act(alpha * A @ B + bias) for float16, bfloat16 or float32 device
    tensors (fp32 accumulation and epilogue in the kernel).

    A: (M, K), B: (K, N) for "KxN" or (N, K) for "NxK", both of one dtype
    (float16, bfloat16 or float32). out: optional (M, N) float16 / bfloat16 / float32
    tensor with unit column stride; allocated with torch.empty as `out_dtype`
    (default: A's dtype) when None. bias: None or an (N,) float32 device
    tensor with unit stride. act: "none" or "relu".
    """
    import torch
    for t, name in ((A, "A"), (B, "B")):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    if A.dtype != B.dtype or A.dtype not in (torch.float16, torch.bfloat16, torch.float32):
        raise TypeError(f"A and B must be of one dtype among float16, bfloat16, float32; got {A.dtype} and {B.dtype}")
    lay = _LAYOUT[b_layout]
    M, K = A.shape
    if lay == TGEMM_B_KxN:
        Kb, N = B.shape
    else:
        N, Kb = B.shape
    if Kb != K:
        raise ValueError(f"inner dimensions differ: A is {tuple(A.shape)}, B is {tuple(B.shape)} ({b_layout})")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or A.dtype, device=A.device)
    elif tuple(out.shape) != (M, N) or not out.is_cuda:
        raise ValueError(f"out must be a ({M}, {N}) device tensor")
    bias_ptr = None
    if bias is not None:
        if bias.dtype != torch.float32 or not bias.is_cuda or tuple(bias.shape) != (N,) or (N > 1 and bias.stride(0) != 1):
            raise ValueError(f"bias must be a contiguous ({N},) float32 device tensor")
        bias_ptr = bias.data_ptr()
    _same_device(A, (B, "B"), (out, "out"), (bias, "bias"))
    lda, ldb, ldc = _row_major(A, "A"), _row_major(B, "B"), _row_major(out, "out")
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if _tune_rounds:
        with torch.cuda.device(A.device):
            rc, chosen = tgemm_tune_gemm(M, N, K, _torch_code(A.dtype), A.data_ptr(), lda, B.data_ptr(), ldb, lay,
                                         _torch_code(out.dtype), out.data_ptr(), ldc, alpha, bias_ptr, act, stream,
                                         _tune_rounds)
        if rc != TGEMM_OK:
            raise TgemmError(rc, f"tune M={M} N={N} K={K} layout={b_layout} {A.dtype}->{out.dtype}")
        return out, chosen
    with torch.cuda.device(A.device):
        rc = tgemm_gemm_config(M, N, K, _torch_code(A.dtype), A.data_ptr(), lda, B.data_ptr(), ldb, lay,
                               _torch_code(out.dtype), out.data_ptr(), ldc, alpha, bias_ptr, act, stream,
                               force_generic, group_m, num_xcd, k_step, stages, tile_m, producers)
    if rc != TGEMM_OK:
        raise TgemmError(rc, f"M={M} N={N} K={K} layout={b_layout} {A.dtype}->{out.dtype}")
    return out
