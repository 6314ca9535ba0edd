"""The C-ABI library on the host: it loads, exports what include/tgemm.h
declares, rejects bad arguments before touching the GPU, plans the expected
variant, and rasterizes exactly as the pages' swizzle (no GPU needed)."""
import ctypes
import os
import re

import pytest

import dense_tiled_gemm_tgemm_amd as tg
from oracle import raster

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, well-separated, 256-byte-aligned device addresses (never dereferenced)
PA, PB, PC = 1 << 40, 2 << 40, 3 << 40


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tgemm_\w+)\s*\(", src, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = tg.load()
    names = _declared_functions()
    assert {"tgemm_f16", "tgemm_status_string", "tgemm_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings():
    assert tg.status_string(tg.TGEMM_OK) == "ok"
    assert tg.status_string(tg.TGEMM_ERR_INVALID) == "invalid argument"
    assert tg.status_string(12345) == "unknown status"
    assert tg.last_hip_error() == 0


def _plan(M, N, K, A=PA, lda=None, B=PB, ldb=None, lay="KxN", C=PC, ldc=None, **kw):
    lda = K if lda is None else lda
    ldb = (N if lay == "KxN" else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return tg.tgemm_plan_f16(M, N, K, A, lda, B, ldb, lay, C, ldc, **kw)


@pytest.mark.parametrize("args", [
    dict(M=-1, N=4, K=4),
    dict(M=4, N=-1, K=4),
    dict(M=4, N=4, K=-1),
    dict(M=1 << 31, N=4, K=4),
    dict(M=4, N=4, K=8, lda=7),
    dict(M=4, N=9, K=8, ldb=8),                  # KxN needs ldb >= N
    dict(M=4, N=9, K=8, lay="NxK", ldb=7),       # NxK needs ldb >= K
    dict(M=4, N=9, K=8, ldc=8),
    dict(M=4, N=4, K=4, A=0),
    dict(M=4, N=4, K=4, B=0),
    dict(M=4, N=4, K=4, C=0),
    dict(M=4, N=4, K=4, A=PA + 1),               # odd byte address
    dict(M=4, N=4, K=4, C=PC + 3),
    dict(M=4, N=4, K=4, C=PA + 8),               # C overlaps A
    dict(M=4, N=4, K=4, C=PB),                   # C overlaps B
    dict(M=4, N=4, K=4, force_generic=2),
    dict(M=4, N=4, K=4, group_m=-1),
    dict(M=4, N=4, K=4, group_m=1025),
    dict(M=4, N=4, K=4, num_xcd=65),
    dict(M=4, N=4, K=4, k_step=16),
    dict(M=4, N=4, K=4, stages=1),
    dict(M=4, N=4, K=4, stages=6),
    dict(M=4, N=4, K=4, k_step=64, stages=3),
    dict(M=4, N=4, K=64, k_step=64),             # 64-deep steps need K > 64
])
def test_invalid_arguments_rejected(args):
    rc, info = _plan(**args)
    assert rc == tg.TGEMM_ERR_INVALID and info is None
    # the launching entry point returns the same code without touching the GPU
    a = dict(args)
    kw = {k: a.pop(k) for k in ("force_generic", "group_m", "num_xcd", "k_step", "stages") if k in a}
    M, N, K = a["M"], a["N"], a["K"]
    lay = a.get("lay", "KxN")
    lda = a.get("lda", K)
    ldb = a.get("ldb", N if lay == "KxN" else K)
    ldc = a.get("ldc", N)
    rc2 = tg.tgemm_f16_config(M, N, K, a.get("A", PA), lda, a.get("B", PB), ldb, lay,
                              a.get("C", PC), ldc, None, **kw)
    assert rc2 == tg.TGEMM_ERR_INVALID


def test_bad_layout_rejected():
    lib = tg.load()
    assert lib.tgemm_f16(4, 4, 4, PA, 4, PB, 4, 2, PC, 4, None) == tg.TGEMM_ERR_INVALID
    info = (ctypes.c_int64 * 10)()
    assert lib.tgemm_plan_f16(4, 4, 4, PA, 4, PB, 4, -1, PC, 4, 0, 0, 0, 0, 0, info) == tg.TGEMM_ERR_INVALID


def test_empty_outputs_are_noops_without_gpu():
    # M == 0 or N == 0: success, nothing launched (these calls run on a GPU-less host)
    assert tg.tgemm_f16(0, 5, 7, PA, 7, PB, 5, "KxN", PC, 5) == tg.TGEMM_OK
    assert tg.tgemm_f16(5, 0, 7, PA, 7, PB, 1, "KxN", PC, 1) == tg.TGEMM_OK
    assert tg.tgemm_f16(0, 0, 0, 0, 1, 0, 1, "NxK", 0, 1) == tg.TGEMM_OK
    rc, info = _plan(0, 5, 7)
    assert rc == tg.TGEMM_OK and info["workgroups"] == 0


def test_plan_variants_and_grid():
    V, C8, NXK, DMA = 1, 2, 4, 8
    rc, info = _plan(8192, 8192, 8192, lay="NxK")
    assert rc == 0
    assert info["variant"] == V | C8 | NXK | DMA
    assert info["workgroups"] == 32 * 32 and info["group_m"] == 8 and info["num_xcd"] == 8
    assert (info["bm"], info["bn"], info["threads"]) == (256, 256, 256)
    assert (info["bk"], info["stages"], info["lds_bytes"]) == (64, 2, 128 * 1024)
    rc, info = _plan(8192, 8192, 8192, lay="NxK", k_step=32)
    assert (info["bk"], info["stages"], info["lds_bytes"]) == (32, 4, 128 * 1024)
    rc, info = _plan(8192, 8192, 8192, lay="NxK", stages=3)
    assert (info["bk"], info["stages"], info["lds_bytes"]) == (32, 3, 96 * 1024)
    rc, info = _plan(8192, 8192, 8192, lay="NxK", k_step=32, stages=5)
    assert (info["bk"], info["stages"], info["lds_bytes"]) == (32, 5, 160 * 1024)
    # ragged, odd strides (2-byte aligned rows): still streamed into LDS; element-wise C stores
    rc, info = _plan(3001, 5003, 4099)
    assert rc == 0 and info["variant"] == DMA and info["workgroups"] == 12 * 20
    # forced register-staged path with element-wise loads
    rc, info = _plan(256, 256, 256, force_generic=1)
    assert info["variant"] == C8
    rc, info = _plan(512, 512, 512, lay="NxK", force_generic=1)
    assert info["variant"] == C8 | NXK
    # base not 16-byte aligned: no 128-bit flag, still direct-to-LDS; C 8-byte aligned keeps 64-bit stores
    rc, info = _plan(256, 256, 256, A=PA + 8)
    assert info["variant"] == C8 | DMA
    rc, info = _plan(256, 256, 256, C=PC + 2)
    assert info["variant"] == V | DMA
    rc, info = _plan(4096, 4096, 4096)
    assert info["variant"] == V | C8 | DMA and (info["bk"], info["stages"]) == (64, 2)
    rc, info = _plan(4096, 4096, 4096, k_step=64)
    assert rc == 0 and (info["bk"], info["stages"], info["lds_bytes"]) == (64, 2, 128 * 1024)
    rc, info = _plan(4096, 4096, 4099, lda=4104)
    assert info["variant"] == V | C8 | DMA    # K % 8 != 0 is fine: the straddling chunk is cleared
    # strides past the 32-bit panel-offset limit: register-staged path
    rc, info = _plan(512, 512, 512, lay="NxK", lda=4_000_008)
    assert info["variant"] == V | C8 | NXK
    rc, info = _plan(512, 512, 512, ldb=(1 << 30) // (512 + 64))
    assert not info["variant"] & DMA
    rc, info = _plan(512, 512, 512, ldb=((1 << 30) - 512) // (512 + 64) - 1)
    assert info["variant"] & DMA
    # K <= 64 streams 32-deep steps; K == 0 (zeros only) takes the register-staged kernel
    rc, info = _plan(512, 512, 64, lay="NxK")
    assert info["variant"] & DMA and (info["bk"], info["stages"]) == (32, 4)
    rc, info = _plan(512, 512, 0, lay="NxK", lda=1, ldb=1)
    assert rc == 0 and not info["variant"] & DMA
    # group_m larger than the tile rows is clamped (same map)
    rc, info = _plan(512, 4096, 64, group_m=100)
    assert info["group_m"] == 2


def test_raster_matches_page1_swizzle_without_die_remap():
    for gm in range(1, 14):
        for gn in range(1, 14):
            for G in (1, 2, 3, 8):
                Gc = min(G, gm)
                for w in range(gm * gn):
                    assert tg.tgemm_tile_of(gm, gn, Gc, 1, w) == raster.swizzle_2d_from_bid(gm, gn, 1, 1, G, w)


@pytest.mark.parametrize("gm,gn", [(1, 1), (3, 5), (12, 20), (32, 32), (32, 48), (16, 16), (7, 9)])
def test_raster_with_die_remap_is_page_swizzle_of_remapped_id(gm, gn):
    W = gm * gn
    seen = set()
    for w in range(W):
        got = tg.tgemm_tile_of(gm, gn, min(8, gm), 8, w)
        want = raster.swizzle_2d_from_bid(gm, gn, 1, 1, 8, raster.xcd_remap(w, W, 8))
        assert got == want
        seen.add(got)
    assert len(seen) == W


def test_tile_of_rejects_out_of_grid():
    with pytest.raises(tg.TgemmError):
        tg.tgemm_tile_of(4, 4, 2, 8, 16)
    with pytest.raises(tg.TgemmError):
        tg.tgemm_tile_of(0, 4, 2, 8, 0)


def test_header_declares_layout_and_status_values():
    src = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    assert "TGEMM_B_KxN = 0" in src and "TGEMM_B_NxK = 1" in src
    for name, val in (("TGEMM_OK", 0), ("TGEMM_ERR_INVALID", -1), ("TGEMM_ERR_UNSUPPORTED", -2),
                      ("TGEMM_ERR_HIP", -3)):
        assert re.search(rf"{name}\s*=\s*{val}\b", src)
        assert getattr(tg, name) == val


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    from dense_tiled_gemm_tgemm_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "libtgemm.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.load()
