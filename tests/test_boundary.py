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


def _declared_functions(header="tgemm.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tgemm_\w+)\s*\(", src, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = tg.load()
    names = _declared_functions()
    assert {"tgemm_f16", "tgemm_status_string", "tgemm_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_measurement_library_is_separate():
    """The probes live in libtgemm_probe.so (include/tgemm_probe.h), which
    exports what its header declares; the GEMM library exports none of them."""
    from dense_tiled_gemm_tgemm_amd import probe
    plib = probe.load()
    names = _declared_functions("tgemm_probe.h")
    assert set(names) == {"tgemm_mfma_issue_probe", "tgemm_mfma_stream_probe", "tgemm_xcd_probe"}
    lib = tg.load()
    for n in names:
        assert ctypes.cast(getattr(plib, n), ctypes.c_void_p).value
        assert not hasattr(lib, n), n
    # bad sizes are refused before any launch
    assert plib.tgemm_mfma_issue_probe(0, 4, PA, 1 << 20, PC, None, None) == tg.TGEMM_ERR_INVALID
    assert plib.tgemm_xcd_probe(0, PC, None) == tg.TGEMM_ERR_INVALID
    # unknown stream kinds, and the sizes the ceiling probe refuses, too
    for kind in (-1, 12):
        assert plib.tgemm_mfma_stream_probe(kind, 8, 4, PA, 1 << 20, PC, None, None) == tg.TGEMM_ERR_INVALID
    assert plib.tgemm_mfma_stream_probe(0, 0, 4, PA, 1 << 20, PC, None, None) == tg.TGEMM_ERR_INVALID
    assert plib.tgemm_mfma_stream_probe(0, 8, 4, PA, (1 << 20) + 2, PC, None, None) == tg.TGEMM_ERR_INVALID


def test_stream_probe_kinds_match_the_header():
    """The binding's kind table holds exactly the kinds include/tgemm_probe.h
    enumerates, with the same codes."""
    from dense_tiled_gemm_tgemm_amd import probe
    src = open(os.path.join(ROOT, "include", "tgemm_probe.h")).read()
    enum = {m.group(1).lower(): int(m.group(2)) for m in re.finditer(r"TGEMM_STREAM_(\w+) = (\d+)", src)}
    assert enum == {k: v[0] for k, v in probe.STREAM_KINDS.items()}
    assert all(v[1] == (512 if "8w" in k else 256) for k, v in probe.STREAM_KINDS.items())


def test_status_strings():
    assert tg.status_string(tg.TGEMM_OK) == "ok"
    assert tg.status_string(tg.TGEMM_ERR_INVALID) == "invalid argument"
    assert tg.status_string(12345) == "unknown status"
    assert tg.last_hip_error() == 0


def _plan(M, N, K, A=PA, lda=None, B=PB, ldb=None, lay="KxN", C=PC, ldc=None, **kw):
    lda = K if lda is None else lda
    ldb = (N if lay == "KxN" else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    kw.setdefault("compute_units", 256)          # MI355X; no device query on this host
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
    dict(M=4, N=16, K=64, k_step=64),            # 64-deep steps need K > 64
    dict(M=4, N=4, K=4, tile_m=96),
    dict(M=4, N=4, K=4, tile_m=32),
    dict(M=4, N=4, K=4, producers=2),
    dict(M=4, N=4, K=4, producers=4, tile_m=64),  # producer/consumer workgroups have 128-row tiles
    dict(M=4, N=4, K=4, producers=4, tile_m=256),
    dict(M=300, N=300, K=300, tile_m=128, k_step=64),  # the smaller tiles take 32-deep steps
    dict(M=300, N=300, K=300, tile_m=128, stages=4),   # two workgroups per unit: at most 80 KiB of ring
])
def test_invalid_arguments_rejected(args):
    rc, info = _plan(**args)
    assert rc == tg.TGEMM_ERR_INVALID and info is None
    # the launching entry point returns the same code without touching the GPU
    a = dict(args)
    kw = {k: a.pop(k) for k in ("force_generic", "group_m", "num_xcd", "k_step", "stages", "tile_m", "producers")
          if k in a}
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
    assert lib.tgemm_plan_f16(4, 4, 4, PA, 4, PB, 4, -1, PC, 4, 0, 0, 0, 0, 0, 0, 0, 256, info) == \
        tg.TGEMM_ERR_INVALID


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
    # 1024 tiles on 256 compute units: one persistent workgroup per unit
    assert info["workgroups"] == 256 and info["group_m"] == 4 and info["num_xcd"] == 8
    rc, info = _plan(8192, 8192, 8192, lay="NxK", compute_units=304)
    assert info["workgroups"] == 304
    rc, info = _plan(8192, 8192, 8192, lay="NxK", compute_units=1536)
    assert info["workgroups"] == 1024                  # fewer tiles than units: one workgroup per tile
    # 32-deep steps are not persistent: one workgroup per tile
    rc, info = _plan(8192, 8192, 8192, lay="NxK", k_step=32)
    assert info["workgroups"] == 1024
    rc, info = _plan(8192, 8192, 8192, lay="NxK")
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
    # strides past the 32-bit panel-offset limit: register-staged path (128-bit loads when aligned)
    rc, info = _plan(512, 512, 512, lay="NxK", lda=4_000_008)
    assert info["variant"] == V | C8 | NXK
    rc, info = _plan(512, 512, 512, lay="NxK", ldb=4_000_008)
    assert info["variant"] == V | C8 | NXK
    rc, info = _plan(512, 512, 512, ldb=4_000_008)
    assert info["variant"] == V | C8
    rc, info = _plan(512, 512, 512, lay="NxK", ldb=4_000_000)
    assert info["variant"] == V | C8 | NXK | DMA
    # B stored K x N is rebased at every K step: its limit is the row stride alone,
    # whatever K is (a vocabulary-sized projection, 2.5 GB of B, streams into LDS)
    rc, info = _plan(8192, 152064, 8192)
    assert info["variant"] == V | C8 | DMA and (info["bk"], info["workgroups"]) == (64, 256)
    rc, info = _plan(512, 512, 1000, ldb=1_100_000)
    assert info["variant"] & DMA
    rc, info = _plan(512, 512, 512, ldb=4_000_000)
    assert info["variant"] & DMA
    # K <= 64 streams 32-deep steps; K == 0 (zeros only) takes the register-staged kernel
    rc, info = _plan(512, 512, 64, lay="NxK", tile_m=256)
    assert info["variant"] & DMA and (info["bk"], info["stages"]) == (32, 4)
    rc, info = _plan(512, 512, 0, lay="NxK", lda=1, ldb=1)
    assert rc == 0 and not info["variant"] & DMA
    # group_m larger than the tile rows is clamped (same map)
    rc, info = _plan(512, 4096, 64, group_m=100)
    assert info["group_m"] == 2


def test_tile_choices_plan():
    """Smaller tiles (128 or 64 rows x 256 columns, two workgroups per compute
    unit, 32-deep steps, 3 stages by default) and producer/consumer workgroups
    (512 threads, 128-row tiles): grid, threads and LDS bytes follow."""
    DMA = 8
    rc, info = _plan(4096, 4096, 4096, tile_m=128)
    assert rc == 0 and info["variant"] & DMA
    assert (info["bm"], info["bn"], info["bk"], info["stages"]) == (128, 256, 32, 3)
    assert (info["workgroups"], info["threads"], info["lds_bytes"]) == (32 * 16, 256, 3 * 384 * 32 * 2)
    rc, info = _plan(4096, 4096, 4096, tile_m=128, stages=2)
    assert (info["stages"], info["lds_bytes"]) == (2, 2 * 384 * 32 * 2)
    rc, info = _plan(256, 256, 256, tile_m=64)
    assert (info["bm"], info["workgroups"], info["lds_bytes"]) == (64, 4, 3 * 320 * 32 * 2)
    rc, info = _plan(3001, 5003, 4099, tile_m=128)                 # ragged: 24 x 20 tiles
    assert (info["bm"], info["workgroups"]) == (128, 24 * 20)
    rc, info = _plan(8192, 8192, 8192, lay="NxK", producers=4)
    assert rc == 0 and (info["bm"], info["threads"], info["bk"], info["stages"]) == (128, 512, 32, 3)
    assert info["workgroups"] == 64 * 32
    rc, info = _plan(8192, 8192, 8192, lay="NxK", producers=4, stages=5)
    assert (info["stages"], info["lds_bytes"]) == (5, 5 * 384 * 32 * 2)
    assert _plan(8192, 8192, 8192, lay="NxK", producers=4, stages=4)[0] == tg.TGEMM_ERR_UNSUPPORTED
    # only the direct-to-LDS path has the smaller tiles
    assert _plan(512, 512, 512, tile_m=128, force_generic=1)[0] == tg.TGEMM_ERR_UNSUPPORTED
    assert _plan(512, 512, 512, lay="NxK", lda=4_000_008, tile_m=128)[0] == tg.TGEMM_ERR_UNSUPPORTED
    assert _plan(512, 512, 512, tile_m=256, force_generic=1)[0] == tg.TGEMM_OK
    # every 16-bit type combination has the default depth of the smaller tiles;
    # producer/consumer workgroups only the plain binary16 product
    for ab, ct, kw in (("bf16", "bf16", {}), ("f16", "f32", {}), ("f16", "f16", dict(alpha=2.0))):
        for tm in (128, 64):
            assert _plan_ex(1024, 1024, 1024, ab=ab, ct=ct, tile_m=tm, **kw)[0] == tg.TGEMM_OK
        assert _plan_ex(1024, 1024, 1024, ab=ab, ct=ct, tile_m=128, stages=2, **kw)[0] == tg.TGEMM_ERR_UNSUPPORTED
        assert _plan_ex(1024, 1024, 1024, ab=ab, ct=ct, producers=4, **kw)[0] == tg.TGEMM_ERR_UNSUPPORTED
    # binary32 operands: the smaller tiles on the direct-to-LDS kernel (3 stages),
    # not on the general kernel
    for lay in ("NxK", "KxN"):
        for tm in (128, 64):
            rc, info = _plan_ex(1024, 1024, 1024, ab="f32", ct="f32", lay=lay, tile_m=tm)
            assert rc == 0 and (info["bm"], info["bk"], info["stages"]) == (tm, 16, 3)
        assert _plan_ex(1024, 1024, 1024, ab="f32", ct="f32", lay=lay, tile_m=128, stages=2)[0] == \
            tg.TGEMM_ERR_UNSUPPORTED
    assert _plan_ex(1024, 1022, 1024, ab="f32", ct="f32", tile_m=128, force_generic=1)[0] == \
        tg.TGEMM_ERR_UNSUPPORTED


def test_small_grids_take_smaller_tiles():
    """Automatic launches whose grid of 256-row tiles fills at most a quarter of
    the compute units take 64-row tiles (four times the workgroups), at most
    half 128-row tiles; explicit choices, the register-staged path and larger
    grids keep 256 rows."""
    rc, info = _plan(256, 256, 256)
    assert rc == 0 and (info["bm"], info["workgroups"], info["bk"], info["stages"]) == (64, 4, 32, 3)
    rc, info = _plan(2048, 2048, 2048, lay="NxK")                  # 64 tiles of 256 rows: a quarter of 256
    assert (info["bm"], info["workgroups"]) == (64, 256)
    rc, info = _plan(2304, 2048, 2048)                             # 72 tiles
    assert (info["bm"], info["workgroups"], info["stages"]) == (128, 144, 3)
    rc, info = _plan(4096, 2048, 2048)                             # 128 tiles: half of 256
    assert (info["bm"], info["workgroups"]) == (128, 256)
    rc, info = _plan(4352, 2048, 2048)                             # 136 tiles
    assert (info["bm"], info["workgroups"]) == (256, 136)
    rc, info = _plan(2048, 2048, 2048, compute_units=255)
    assert info["bm"] == 128
    rc, info = _plan(2048, 2048, 2048, compute_units=127)
    assert info["bm"] == 256
    rc, info = _plan(256, 256, 256, tile_m=256)
    assert (info["bm"], info["workgroups"]) == (256, 1)
    rc, info = _plan(256, 256, 256, force_generic=1)
    assert info["bm"] == 256
    for ab, ct in (("bf16", "f32"), ("f16", "bf16")):
        assert _plan_ex(256, 256, 256, ab=ab, ct=ct, alpha=0.5)[1]["bm"] == 64
    assert _plan_ex(256, 256, 256, ab="f32", ct="f32")[1]["bm"] == 64
    assert _plan_ex(256, 254, 256, ab="f32", ct="f32", force_generic=1)[1]["bm"] == 256   # general kernel


@pytest.mark.parametrize("M,N,cu,bm", [
    (256, 256, 256, 64), (4096, 2048, 256, 64),          # a tile, half a round
    (2560, 4096, 256, 64), (3072, 4096, 256, 64),        # 160 and 192 tiles on 256 units
    (3584, 4096, 256, 256), (4096, 4096, 256, 256),      # 224 (7/8) and 256 tiles
    (5120, 4096, 256, 64), (6144, 4096, 256, 64),        # 320 and 384: rounds 5/8 and 3/4 full
    (8192, 8192, 256, 256), (8192, 12288, 256, 256),     # 1024 and 1536: whole rounds
    (4096, 4096, 255, 64), (3584, 4096, 224, 256),       # the fill is counted on the device's units
])
def test_binary32_tile_rows_follow_round_fill(M, N, cu, bm):
    """Binary32 operands (either B layout): 64-row tiles unless 256-row tiles
    fill at least 7/8 of their rounds over the compute units; explicit tile
    rows are left alone."""
    for lay in ("NxK", "KxN"):
        rc, info = _plan_ex(M, N, 2048, ab="f32", ct="f32", lay=lay, compute_units=cu)
        assert rc == 0 and info["bm"] == bm
        assert info["stages"] == (2 if bm == 256 else 3)
        rc, info = _plan_ex(M, N, 2048, ab="f32", ct="f32", lay=lay, compute_units=cu, tile_m=256)
        assert rc == 0 and info["bm"] == 256


def test_default_die_count_follows_the_compute_units():
    """The die-aware renumbering spreads over compute units / 32 dies (gfx950:
    32 compute units per die), 1 to 8: a whole MI355X has 8, a partitioned
    one 4, 2 or 1. An explicit num_xcd is kept."""
    for cu, x in ((256, 8), (128, 4), (64, 2), (32, 1), (16, 1), (304, 8)):
        rc, info = _plan(8192, 8192, 8192, lay="NxK", compute_units=cu)
        assert rc == 0 and info["num_xcd"] == x, (cu, info)
    rc, info = _plan(8192, 8192, 8192, lay="NxK", compute_units=64, num_xcd=8)
    assert info["num_xcd"] == 8


def test_kxn_one_round_rule_follows_the_compute_unit_count():
    """Automatic launches with B stored K x N, K > 64 not a multiple of 64 and at
    most one tile per compute unit take 32-deep steps (default ring depth); more
    tiles than units, K a multiple of 64, or B stored N x K keep the persistent
    64-deep ring. The count is an argument of the query, so the rule is checked
    here without a device."""
    rc, info = _plan(3001, 5003, 4099)                              # 240 tiles
    assert rc == 0 and (info["bk"], info["stages"], info["workgroups"]) == (32, 4, 240)
    rc, info = _plan(3001, 5003, 4099, compute_units=240)
    assert (info["bk"], info["stages"], info["workgroups"]) == (32, 4, 240)
    rc, info = _plan(3001, 5003, 4099, compute_units=239)            # one tile more than units
    assert (info["bk"], info["stages"], info["workgroups"]) == (64, 2, 239)
    rc, info = _plan(3001, 5003, 4096)                              # K a multiple of 64
    assert (info["bk"], info["stages"], info["workgroups"]) == (64, 2, 240)
    rc, info = _plan(3001, 5003, 4099, lay="NxK")                   # B stored N x K
    assert (info["bk"], info["stages"]) == (64, 2)
    rc, info = _plan(3001, 5003, 4099, k_step=64)                   # an explicit choice wins
    assert (info["bk"], info["stages"]) == (64, 2)
    for ab in ("f16", "bf16"):
        rc, info = _plan_ex(3001, 5003, 4099, ab=ab, ct="f32", alpha=0.5)
        assert rc == 0 and (info["bk"], info["stages"]) == (32, 4)


def test_plan_query_device_count_needs_a_device():
    """compute_units = 0 asks the current device; on a host without one the
    query reports a HIP error once the arguments have passed (argument errors
    and empty outputs need no device). Negative counts are invalid."""
    rc, _ = _plan(300, 300, 300, compute_units=0)
    assert rc in (tg.TGEMM_OK, tg.TGEMM_ERR_HIP)
    import torch
    if not torch.cuda.is_available():
        assert rc == tg.TGEMM_ERR_HIP
    rc, info = _plan(0, 300, 300, compute_units=0)
    assert rc == tg.TGEMM_OK and info["workgroups"] == 0
    rc, _ = _plan(300, 300, 300, lda=5, compute_units=0)
    assert rc == tg.TGEMM_ERR_INVALID
    rc, _ = _plan(300, 300, 300, compute_units=-1)
    assert rc == tg.TGEMM_ERR_INVALID


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


# ------------------------------------------------ typed GEMM with epilogue --

def _plan_ex(M, N, K, ab="f16", ct="f16", A=PA, lda=None, B=PB, ldb=None, lay="KxN", C=PC, ldc=None,
             alpha=1.0, bias=None, act="none", **kw):
    lda = K if lda is None else lda
    ldb = (N if lay == "KxN" else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    kw.setdefault("compute_units", 256)          # MI355X; no device query on this host
    return tg.tgemm_plan_gemm(M, N, K, ab, A, lda, B, ldb, lay, ct, C, ldc, alpha, bias, act, **kw)


PBIAS = 4 << 40


@pytest.mark.parametrize("args", [
    dict(M=4, N=4, K=4, ab=3),
    dict(M=4, N=4, K=4, ab=-1),
    dict(M=4, N=4, K=4, ab="f32", A=PA + 2),          # binary32 operands must be 4-byte aligned
    dict(M=4, N=4, K=4, ab="f32", B=PB + 6),
    dict(M=4, N=4, K=4, ab="f32", C=PA + 40),         # A spans 4-byte elements: C overlaps it
    dict(M=4, N=4, K=4, ct=3),
    dict(M=4, N=4, K=4, act=2),
    dict(M=4, N=4, K=4, ct="f32", C=PC + 2),          # fp32 C must be 4-byte aligned
    dict(M=4, N=4, K=4, bias=PBIAS + 2),              # bias must be 4-byte aligned
    dict(M=4, N=4, K=4, bias=PC + 4),                 # bias overlaps C
    dict(M=4, N=4, K=4, ct="f32", C=PA + 16),         # fp32 C spans 4-byte elements: overlaps A
    dict(M=4, N=9, K=8, ct="f32", ldc=8),
])
def test_typed_invalid_arguments_rejected(args):
    rc, info = _plan_ex(**args)
    assert rc == tg.TGEMM_ERR_INVALID and info is None
    # the launching entry point returns the same code without touching the GPU
    a = dict(args)
    M, N, K = a.pop("M"), a.pop("N"), a.pop("K")
    rc2 = tg.tgemm_gemm(M, N, K, a.get("ab", "f16"), a.get("A", PA), K, a.get("B", PB), N, "KxN",
                        a.get("ct", "f16"), a.get("C", PC), a.get("ldc", N), 1.0, a.get("bias"),
                        a.get("act", "none"))
    assert rc2 == tg.TGEMM_ERR_INVALID


def test_fp32_output_overlap_uses_four_byte_elements():
    # 4 x 4 fp32 C ends 64 bytes after its base; A 40 bytes after C's base overlaps only as fp32
    assert _plan_ex(4, 4, 4, ct="f16", C=PA - 40)[0] == tg.TGEMM_OK
    assert _plan_ex(4, 4, 4, ct="f32", C=PA - 40)[0] == tg.TGEMM_ERR_INVALID


def test_typed_plans_match_f16_plans():
    for ab in ("f16", "bf16"):
        for ct in ("f16", "bf16", "f32"):
            for kw in (dict(), dict(alpha=0.5), dict(bias=PBIAS), dict(act="relu")):
                rc, info = _plan_ex(8192, 8192, 8192, ab=ab, ct=ct, lay="NxK", **kw)
                rc0, info0 = _plan(8192, 8192, 8192, lay="NxK")
                assert rc == rc0 == 0 and info == info0, (ab, ct, kw)
                rc, info = _plan_ex(512, 512, 64, ab=ab, ct=ct, tile_m=256, **kw)
                assert rc == 0 and (info["bk"], info["stages"]) == (32, 4)
                rc, info = _plan_ex(300, 200, 100, ab=ab, ct=ct, force_generic=1, **kw)
                assert rc == 0 and not info["variant"] & 8


def test_typed_ring_depths_other_than_default_are_unsupported():
    # every depth for the plain binary16 product
    for st in (2, 3, 4, 5):
        assert _plan_ex(1024, 1024, 1024, stages=st)[0] == tg.TGEMM_OK
    # the default depth of each K step for every other combination
    for ab, ct, kw in (("bf16", "bf16", {}), ("f16", "f32", {}), ("f16", "f16", dict(alpha=2.0))):
        assert _plan_ex(1024, 1024, 1024, ab=ab, ct=ct, k_step=32, stages=4, **kw)[0] == tg.TGEMM_OK
        assert _plan_ex(1024, 1024, 1024, ab=ab, ct=ct, k_step=64, **kw)[0] == tg.TGEMM_OK
        for st in (2, 3, 5):
            assert _plan_ex(1024, 1024, 1024, ab=ab, ct=ct, k_step=32, stages=st, **kw)[0] == \
                tg.TGEMM_ERR_UNSUPPORTED
            # the launching entry point refuses the same way, before any GPU call
            lib = tg.load()
            rc = lib.tgemm_gemm_config(1024, 1024, 1024, tg._binding._DTYPE[ab], PA, 1024, PB, 1024, 0,
                                       tg._binding._DTYPE[ct], PC, 1024, kw.get("alpha", 1.0), None, 0, None,
                                       0, 0, 0, 32, st, 0, 0)
            assert rc == tg.TGEMM_ERR_UNSUPPORTED


def test_fp32_output_store_width_flags():
    V, CV, DMA = 1, 2, 8
    # fp32 C: 16-byte-aligned rows (base and 4 * ldc) give 128-bit stores
    rc, info = _plan_ex(256, 256, 256, ct="f32")
    assert info["variant"] == V | CV | DMA
    rc, info = _plan_ex(256, 254, 256, ct="f32", ldb=256, ldc=254)
    assert info["variant"] == V | DMA
    rc, info = _plan_ex(256, 256, 256, ct="f32", C=PC + 8)
    assert info["variant"] == V | DMA


def test_typed_empty_outputs_are_noops_without_gpu():
    lib = tg.load()
    assert lib.tgemm_gemm(0, 5, 7, 1, PA, 7, PB, 5, 0, 2, PC, 5, 1.0, None, 0, None) == tg.TGEMM_OK
    assert lib.tgemm_gemm(5, 0, 7, 1, PA, 7, PB, 1, 0, 2, PC, 1, 2.0, PBIAS, 1, None) == tg.TGEMM_OK


def test_header_declares_type_and_activation_values():
    src = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    for name, val in (("TGEMM_F16", 0), ("TGEMM_BF16", 1), ("TGEMM_F32", 2), ("TGEMM_ACT_NONE", 0),
                      ("TGEMM_ACT_RELU", 1)):
        assert re.search(rf"{name}\s*=\s*{val}\b", src)
        assert getattr(tg, name) == val


# ------------------------------------------------------------ runtime tuning --

def test_tuning_rejects_bad_arguments_without_gpu():
    lib = tg.load()
    assert tg.tuning_entries() == 0
    # argument errors of tgemm_gemm, and rounds outside 1..100: nothing runs
    assert tg.tgemm_tune_gemm(4, 4, 4, "f16", PA, 3, PB, 4, "KxN", "f16", PC, 4)[0] == tg.TGEMM_ERR_INVALID
    assert tg.tgemm_tune_gemm(4, 4, 4, "f16", PA, 4, PB, 4, "KxN", "f32", PC + 2, 4)[0] == tg.TGEMM_ERR_INVALID
    assert tg.tgemm_tune_gemm(4, 4, 4, "f16", PA, 4, PB, 4, "KxN", "f16", PC, 4, rounds=0)[0] == \
        tg.TGEMM_ERR_INVALID
    assert tg.tgemm_tune_gemm(4, 4, 4, "f16", PA, 4, PB, 4, "KxN", "f16", PC, 4, rounds=101)[0] == \
        tg.TGEMM_ERR_INVALID
    # empty output: nothing to tune, nothing recorded
    rc, info = tg.tgemm_tune_gemm(0, 4, 4, "bf16", PA, 4, PB, 4, "KxN", "f32", PC, 4)
    assert rc == tg.TGEMM_OK and all(v == 0 for v in info.values())
    assert tg.tuning_entries() == 0
    tg.tuning_clear()
    assert tg.tuning_entries() == 0
    assert lib.tgemm_tune_gemm(0, 4, 4, 0, PA, 4, PB, 4, 0, 0, PC, 4, 1.0, None, 0, None, 5, None) == tg.TGEMM_OK


def test_fp32_operand_plans():
    V, CV, NXK, PIPE = 1, 2, 4, 8
    # binary32 operands with B stored N x K: the direct-to-LDS kernel on the
    # operands' bytes, 256 x 256 tiles, 16-deep steps, 2 stages of
    # 2 x 256 x 16 floats, one tile per workgroup
    rc, info = _plan_ex(8192, 8192, 8192, ab="f32", ct="f32", lay="NxK")
    assert rc == 0 and info["variant"] == V | CV | NXK | PIPE
    assert (info["bm"], info["bn"]) == (256, 256)
    assert (info["bk"], info["stages"], info["lds_bytes"], info["workgroups"]) == (16, 2, 64 * 1024, 1024)
    # the K step choice does not apply; rings of 2 or 3 stages are built
    rc2, info2 = _plan_ex(8192, 8192, 8192, ab="f32", ct="f32", lay="NxK", k_step=32)
    assert rc2 == 0 and info2 == info
    rc3, info3 = _plan_ex(8192, 8192, 8192, ab="f32", ct="f32", lay="NxK", stages=3)
    assert rc3 == 0 and (info3["stages"], info3["lds_bytes"]) == (3, 96 * 1024)
    assert _plan_ex(8192, 8192, 8192, ab="f32", ct="f32", lay="NxK", stages=5)[0] == tg.TGEMM_ERR_UNSUPPORTED
    assert _plan_ex(8192, 8192, 8192, ab="f32", ct="f32", lay="NxK", producers=4)[0] == tg.TGEMM_ERR_UNSUPPORTED
    # any K, and row strides of at least 4 floats (8 16-bit units)
    rc, info = _plan_ex(300, 200, 101, ab="f32", ct="f16", lay="NxK")
    assert rc == 0 and info["variant"] == CV | NXK | PIPE
    rc, info = _plan_ex(300, 200, 4, ab="f32", ct="f32", lay="NxK")
    assert rc == 0 and info["variant"] & PIPE
    rc, info = _plan_ex(300, 200, 3, ab="f32", ct="f32", lay="NxK")
    assert rc == 0 and not info["variant"] & PIPE
    rc, info = _plan_ex(300, 202, 100, ab="f32", ct="f16", lay="NxK", ldc=208)
    assert rc == 0 and info["variant"] == V | CV | NXK | PIPE
    # B stored K x N: the same kernel (any K, any N)
    rc, info = _plan_ex(8192, 8192, 8192, ab="f32", ct="f32")
    assert rc == 0 and info["variant"] == V | CV | PIPE
    assert (info["bm"], info["bn"]) == (256, 256)
    assert (info["bk"], info["stages"], info["lds_bytes"], info["workgroups"]) == (16, 2, 64 * 1024, 1024)
    rc, info = _plan_ex(300, 200, 101, ab="f32", ct="f16", lda=101)
    assert rc == 0 and info["variant"] == CV | PIPE
    rc3, info3 = _plan_ex(8192, 8192, 8192, ab="f32", ct="f32", stages=4)
    assert rc3 == 0 and (info3["stages"], info3["lds_bytes"]) == (4, 128 * 1024)
    rc, info = _plan_ex(300, 202, 100, ab="f32", ct="f16", lda=100, ldb=202, ldc=208)
    assert rc == 0 and info["variant"] == CV | PIPE
    # row strides under 4 floats, or forced: the general kernel
    rc, info = _plan_ex(300, 3, 100, ab="f32", ct="f16", lda=100, ldb=3, ldc=8)
    assert rc == 0 and info["variant"] == CV
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="f16", lda=100, ldb=200, force_generic=1)
    assert rc == 0 and info["variant"] == CV
    assert (info["bn"], info["lds_bytes"], info["workgroups"]) == (256, 64 * 1024, 2)
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="f16", lay="NxK", force_generic=1)
    assert rc == 0 and info["variant"] == CV | NXK
    # 4-byte-aligned bases are fine (buffer loads)
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="bf16", A=PA + 4)
    assert rc == 0 and info["variant"] == CV | PIPE
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="bf16", lay="NxK", A=PA + 4)
    assert rc == 0 and info["variant"] == CV | NXK | PIPE
    # strides past the 32-bit offset limits: the general kernel
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="f32", lay="NxK", lda=2_000_004)
    assert rc == 0 and not info["variant"] & PIPE
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="f32", lay="NxK", ldb=2_000_004)
    assert rc == 0 and not info["variant"] & PIPE
    rc, info = _plan_ex(300, 200, 100, ab="f32", ct="f32", ldb=2_000_004)
    assert rc == 0 and not info["variant"] & PIPE
    # B stored K x N is rebased at every step: a wide B stays on the direct-to-LDS kernel
    rc, info = _plan_ex(300, 200, 8192, ab="f32", ct="f32", ldb=2_000_000)
    assert rc == 0 and info["variant"] & PIPE


@pytest.mark.parametrize("lay,M,N,K,lda,ldb,dma", [
    ("KxN", 64, 3, 100, 100, 3, False),      # B rows of 3 elements
    ("KxN", 64, 7, 100, 100, 7, False),
    ("KxN", 64, 8, 100, 100, 8, True),
    ("KxN", 64, 3, 100, 100, 8, True),       # padded rows: a stride of 8 is enough
    ("NxK", 64, 300, 5, 5, 5, False),        # A and B rows of 5 elements
    ("NxK", 64, 300, 5, 8, 8, True),
    ("KxN", 64, 300, 7, 7, 300, False),
])
def test_narrow_operands_take_register_staged_path(lay, M, N, K, lda, ldb, dma):
    """The direct-to-LDS path needs row strides of at least 8 elements: then a
    16-byte access runs past the end of an operand only in its last row, which
    the kernel reloads element by element. Narrower operands (K or N below 8
    with tight strides) go to the register-staged kernel, which masks every
    element load."""
    rc, info = _plan(M, N, K, lda=lda, ldb=ldb, lay=lay)
    assert rc == 0
    assert bool(info["variant"] & 8) == dma, info
