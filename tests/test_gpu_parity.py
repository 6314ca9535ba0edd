"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case draws seeded inputs, runs tgemm on cuda:0, and compares element by
element with the oracle: bit-exact where the answer is exactly representable
(integer-valued products, identities, all-ones), otherwise within
|g - ref| <= 1e-3 * sum_k |a*b| + ulp16(ref).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import dense_tiled_gemm_tgemm_amd as tg  # noqa: E402
from dense_tiled_gemm_tgemm_amd import inputs, probe  # noqa: E402

DEV = "cuda:0"
NAN16 = 0x7E01          # a quiet-NaN binary16 pattern used as a sentinel


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    yield
    torch.cuda.synchronize()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _run(A, B, lay, **kw):
    C = tg.mm(_dev(A), _dev(B), lay, **kw)
    return _host(C)


def _full_check(oracle_mod, A, B, lay, got, what):
    ref, ab = oracle_mod.gemm(A, B, lay)
    res = oracle_mod.check(got, ref, ab)
    assert res["nfail"] == 0, f"{what}: {res}"
    return res


SMALL = [(1, 1, 1), (1, 300, 7), (31, 17, 65), (64, 64, 64), (255, 257, 63), (256, 256, 64),
         (257, 255, 129), (300, 520, 200), (513, 300, 8), (96, 1100, 1000), (512, 512, 512)]


@pytest.mark.parametrize("mode", ["auto", "tile256", "generic"])
@pytest.mark.parametrize("lay", ["KxN", "NxK"])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes_full_parity(oracle_mod, M, N, K, lay, mode):
    """The automatic launch (at these sizes mostly 64-row tiles), the 256-row
    direct-to-LDS tile and the register-staged kernel, each in full parity."""
    print(f"case small M={M} N={N} K={K} {lay} {mode}", flush=True)
    seed = (M * 7 + N * 13 + K * 17) % 100003
    A = inputs.random_f16((M, K), seed)
    B = inputs.random_f16((K, N) if lay == "KxN" else (N, K), seed + 1)
    kw = {"auto": {}, "tile256": dict(tile_m=256), "generic": dict(force_generic=1)}[mode]
    got = _run(A, B, lay, **kw)
    _full_check(oracle_mod, A, B, lay, got, f"{M}x{N}x{K} {lay} {mode}")


@pytest.mark.parametrize("lay,offset,M,N,K,pad", [
    ("KxN", 0, 300, 270, 130, (13, 9, 11)),
    ("KxN", 1, 300, 270, 130, (13, 9, 11)),
    ("NxK", 0, 300, 270, 130, (13, 9, 11)),
    ("NxK", 1, 300, 270, 130, (13, 9, 11)),
    # 16-byte-aligned strides: the direct-to-LDS path, with edge tiles and a K tail
    ("NxK", 0, 700, 600, 264, (8, 16, 8)),
    ("NxK", 8, 520, 777, 72, (24, 8, 4)),
    ("KxN", 0, 700, 600, 264, (8, 16, 8)),
])
def test_strided_offset_operands_and_guard_band(oracle_mod, lay, offset, M, N, K, pad):
    """Operands inside larger buffers (ld > row length, optional element offset
    that may leave them only 2-byte aligned); C inside a NaN-filled buffer with a
    column guard band and a guard row: every element outside M x N stays intact."""
    print(f"case strided {lay} offset={offset} {M}x{N}x{K} pad={pad}", flush=True)
    lda, ldb, ldc = K + pad[0], (N if lay == "KxN" else K) + pad[1], N + pad[2]
    rows_b = K if lay == "KxN" else N
    Abuf = inputs.random_f16((M * lda + offset,), 71)
    Bbuf = inputs.random_f16((rows_b * ldb + offset,), 72)
    A = np.lib.stride_tricks.as_strided(Abuf[offset:], (M, K), (2 * lda, 2))
    B = np.lib.stride_tricks.as_strided(Bbuf[offset:], (rows_b, K if lay == "NxK" else N), (2 * ldb, 2))
    Ad, Bd = _dev(Abuf), _dev(Bbuf)
    for tile_m in (0, 256):                          # automatic (small grid: 64-row tiles) and 256-row tiles
        Cd = torch.full(((M + 1) * ldc + 5,), NAN16, dtype=torch.int32).to(torch.int16).view(torch.float16).to(DEV)
        rc = tg.tgemm_f16_config(M, N, K, Ad.data_ptr() + 2 * offset, lda, Bd.data_ptr() + 2 * offset, ldb, lay,
                                 Cd.data_ptr() + 2 * offset, ldc, torch.cuda.current_stream().cuda_stream,
                                 tile_m=tile_m)
        assert rc == tg.TGEMM_OK
        Cbits = _host(Cd).view(np.uint16)
        inside = np.zeros(Cbits.shape, dtype=bool)
        idx = offset + (np.arange(M)[:, None] * ldc + np.arange(N)[None, :])
        inside[idx.ravel()] = True
        assert np.all(Cbits[~inside] == NAN16), f"write outside M x N (tile_m {tile_m})"
        got = Cbits[idx]
        _full_check(oracle_mod, np.ascontiguousarray(A), np.ascontiguousarray(B), lay, got, f"strided {tile_m}")
    # inputs were not modified
    assert np.array_equal(_host(Ad).view(np.uint16), Abuf.view(np.uint16))
    assert np.array_equal(_host(Bd).view(np.uint16), Bbuf.view(np.uint16))


@pytest.mark.parametrize("K", [1, 64, 65, 4096, 4099, 8192])
def test_all_ones_closed_form(K):
    """All-ones operands: every C element is binary16(K) (4099 -> 4100)."""
    print(f"case ones K={K}", flush=True)
    M, N = 300, 260
    for lay in ("KxN", "NxK"):
        A = torch.ones((M, K), dtype=torch.float16, device=DEV)
        B = torch.ones((K, N) if lay == "KxN" else (N, K), dtype=torch.float16, device=DEV)
        C = tg.mm(A, B, lay)
        want = float(np.float16(K))
        assert bool((C == want).all()), f"K={K} {lay}: values {torch.unique(C)[:5]}"


@pytest.mark.parametrize("lay", ["KxN", "NxK"])
def test_identity_closed_form(lay):
    """B = I gives C = A bit for bit; A = I gives C = B."""
    print(f"case identity {lay}", flush=True)
    M, K = 517, 384
    A = _dev(inputs.random_f16((M, K), 81))
    I = torch.eye(K, dtype=torch.float16, device=DEV)
    C = tg.mm(A, I, lay)
    assert torch.equal(C.view(torch.int16), A.view(torch.int16))
    Bk = _dev(inputs.random_f16((K, 333), 82))
    C2 = tg.mm(I, Bk if lay == "KxN" else Bk.t().contiguous(), lay)
    assert torch.equal(C2.view(torch.int16), Bk.view(torch.int16))


def _ternary_case(oracle_mod, M, N, K, lay, seed, npts=None):
    A = inputs.ternary_f16((M, K), seed)
    B = inputs.ternary_f16((K, N) if lay == "KxN" else (N, K), seed + 1)
    C = tg.mm(_dev(A), _dev(B), lay)
    got = _host(C)
    if npts is None:
        ref, _ = oracle_mod.gemm(A, B, lay)
        sel = got
    else:
        I, J = inputs.sample_points(M, N, npts, seed + 2)
        ref, _ = oracle_mod.gemm_points(A, B, lay, I, J)
        sel = got[I, J]
    assert np.abs(ref).max() <= 2048, "ternary sums must stay exactly representable"
    # every partial sum is an integer below 2^24: the result is exact in any order
    assert np.array_equal(sel.astype(np.float64), ref), f"ternary {M}x{N}x{K} {lay} not bit-exact"
    g = got.astype(np.float64)
    assert np.all(g == np.round(g)) and np.abs(g).max() <= K


@pytest.mark.parametrize("name", ["sq256", "sq4096", "ragged", "sq8192_nt", "qkv_proj"])
def test_ternary_bit_exact_at_workload_shapes(oracle_mod, name):
    w = inputs.WORKLOADS[name]
    print(f"case ternary {name}", flush=True)
    full = w.M * w.N * w.K <= 2 ** 37
    _ternary_case(oracle_mod, w.M, w.N, w.K, w.b_layout, 100 + w.seed, None if full else 8192)


@pytest.mark.parametrize("name", ["sq256", "sq4096", "ragged", "sq8192_nt", "qkv_proj"])
def test_workload_parity(oracle_mod, name):
    """The five workloads, launched exactly as the benchmark launches them."""
    w = inputs.WORKLOADS[name]
    print(f"case workload {name}", flush=True)
    A, B = inputs.make_inputs(w)
    Ad, Bd = _dev(A), _dev(B)
    C = torch.empty((w.M, w.N), dtype=torch.float16, device=DEV)
    rc = tg.tgemm_f16(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), B.shape[1], w.b_layout,
                      C.data_ptr(), w.N, torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TGEMM_OK
    got = _host(C)
    assert np.isfinite(got.astype(np.float32)).all()
    if w.M * w.N * w.K <= 2 ** 37:
        ref, ab = oracle_mod.gemm(A, B, w.b_layout)
        res = oracle_mod.check(got, ref, ab)
    else:
        I, J = inputs.sample_points(w.M, w.N, 8192, w.seed + 1000)
        ref, ab = oracle_mod.gemm_points(A, B, w.b_layout, I, J)
        res = oracle_mod.check(got[I, J], ref, ab)
    print(f"  {name}: {res['n']} checked, {res['nfail']} fail, worst {res['worst']:.4f}", flush=True)
    assert res["nfail"] == 0, res


def test_deterministic_and_inputs_unchanged():
    print("case determinism", flush=True)
    w = inputs.WORKLOADS["ragged"]
    A, B = inputs.make_inputs(w)
    Ad, Bd = _dev(A), _dev(B)
    C1 = tg.mm(Ad, Bd, w.b_layout)
    C2 = tg.mm(Ad, Bd, w.b_layout)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    assert np.array_equal(_host(Ad).view(np.uint16), A.view(np.uint16))
    assert np.array_equal(_host(Bd).view(np.uint16), B.view(np.uint16))


@pytest.mark.parametrize("group_m,num_xcd", [(1, 1), (3, 1), (8, 8), (64, 5), (2, 8)])
def test_raster_choice_does_not_change_result(group_m, num_xcd):
    print(f"case raster g={group_m} x={num_xcd}", flush=True)
    A = _dev(inputs.random_f16((1300, 700), 91))
    B = _dev(inputs.random_f16((1500, 700), 92))
    base = tg.mm(A, B, "NxK")
    other = tg.mm(A, B, "NxK", group_m=group_m, num_xcd=num_xcd)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), other.view(torch.int16))


def test_degenerate_shapes():
    print("case degenerate", flush=True)
    # K == 0 writes zeros
    A = torch.empty((300, 0), dtype=torch.float16, device=DEV)
    B = torch.empty((0, 270), dtype=torch.float16, device=DEV)
    C = torch.full((300, 270), 7.0, dtype=torch.float16, device=DEV)
    tg.mm(A, B, "KxN", out=C)
    torch.cuda.synchronize()
    assert bool((C == 0).all())
    # M == 0 / N == 0 leave C untouched
    C = torch.full((4, 4), 3.0, dtype=torch.float16, device=DEV)
    A4 = torch.ones((4, 4), dtype=torch.float16, device=DEV)
    B4 = torch.ones((4, 4), dtype=torch.float16, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    # M == 0: A may be NULL (no elements), B still holds K x N elements
    assert tg.tgemm_f16(0, 4, 4, 0, 4, B4.data_ptr(), 4, "KxN", C.data_ptr(), 4, st) == 0
    # N == 0: B and C hold no elements
    assert tg.tgemm_f16(4, 0, 4, A4.data_ptr(), 4, 0, 1, "KxN", 0, 1, st) == 0
    assert tg.tgemm_f16(4, 0, 4, A4.data_ptr(), 4, B4.data_ptr(), 1, "KxN", C.data_ptr(), 4, st) == 0
    torch.cuda.synchronize()
    assert bool((C == 3.0).all())


def test_runs_on_a_side_stream(oracle_mod):
    print("case side stream", flush=True)
    A = inputs.random_f16((400, 300), 95)
    B = inputs.random_f16((300, 500), 96)
    Ad, Bd = _dev(A), _dev(B)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = tg.mm(Ad, Bd, "KxN")
    s.synchronize()
    _full_check(oracle_mod, A, B, "KxN", C.cpu().numpy(), "side stream")


# (K step, ring depth, tile rows, producer waves)
PIPES = [(64, 2, 0, 0), (32, 2, 0, 0), (32, 3, 0, 0), (32, 4, 0, 0), (32, 5, 0, 0),
         (32, 3, 128, 0), (32, 2, 128, 0), (32, 3, 64, 0), (32, 3, 128, 4), (32, 5, 128, 4)]


@pytest.mark.parametrize("lay", ["NxK", "KxN"])
@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (700, 600, 264), (1000, 1300, 8), (256, 256, 4096 + 32),
                                   (3001, 1030, 1000)])
def test_pipeline_choices_are_bit_identical(oracle_mod, M, N, K, lay):
    """Every direct-to-LDS pipeline (K step x ring depth x tile rows x
    producer/consumer workgroups) and the register-staged path produce the same
    bits: each output's 32-deep K slices are summed in the same order. Odd step
    counts (K = 8, 264, 4128 at K step 32) cover the leading all-zero step that
    makes a 32-deep ring's step count even; M = 3001 leaves partial 128- and
    64-row tiles."""
    print(f"case pipelines {M}x{N}x{K} {lay}", flush=True)
    A = inputs.random_f16((M, K), M + K)
    B = inputs.random_f16((N, K) if lay == "NxK" else (K, N), N + K)
    Ad, Bd = _dev(A), _dev(B)
    base = tg.mm(Ad, Bd, lay, force_generic=1)
    got = _host(base)
    _full_check(oracle_mod, A, B, lay, got, f"pipelines {M}x{N}x{K} {lay}")
    for ks, st, tm, pr in PIPES:
        kw = dict(k_step=ks, stages=st, tile_m=tm, producers=pr)
        if ks == 64 and K <= 64:                     # 64-deep steps need two steps or more
            with pytest.raises(tg.TgemmError, match="invalid"):
                tg.mm(Ad, Bd, lay, **kw)
            continue
        C = tg.mm(Ad, Bd, lay, **kw)
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), base.view(torch.int16)), kw


@pytest.mark.parametrize("lay", ["NxK", "KxN"])
@pytest.mark.parametrize("M,N,K", [(4300, 4300, 1000), (4608, 3840, 200), (4352, 4096, 128)])
def test_persistent_grid_matches_register_staged(oracle_mod, M, N, K, lay):
    """More output tiles (270 .. 289) than compute units: the direct-to-LDS kernel
    runs one workgroup per compute unit, each walking one or two tiles with the
    next tile's first K steps streamed in while the current one finishes. Edge
    tiles, partial last K steps (K % 64 = 40, 8) and the shortest persistent K
    (two steps) included. Bit-identical to the register-staged kernel (one
    workgroup per tile), also under another raster, and within tolerance of the
    oracle on sampled outputs."""
    print(f"case persistent {M}x{N}x{K} {lay}", flush=True)
    A = inputs.random_f16((M, K), M + 7 * K)
    B = inputs.random_f16((N, K) if lay == "NxK" else (K, N), N + 5 * K)
    Ad, Bd = _dev(A), _dev(B)
    base = tg.mm(Ad, Bd, lay, force_generic=1)
    C = tg.mm(Ad, Bd, lay)
    C2 = tg.mm(Ad, Bd, lay, group_m=3, num_xcd=1)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), base.view(torch.int16))
    assert torch.equal(C2.view(torch.int16), base.view(torch.int16))
    got = _host(C)
    I, J = inputs.sample_points(M, N, 4096, M + N + K)
    ref, ab = oracle_mod.gemm_points(A, B, lay, I, J)
    res = oracle_mod.check(got[I, J], ref, ab)
    assert res["nfail"] == 0, res


@pytest.mark.parametrize("lay", ["NxK", "KxN"])
@pytest.mark.parametrize("M,N,K", [(8192, 8192, 1024), (8000, 8192, 640)])
def test_persistent_tile_changes_bit_identical(oracle_mod, M, N, K, lay):
    """About four tiles per workgroup, so most workgroups change tiles three
    times (the next tile's first steps load while the current tile's C is
    stored), with whole tiles only and with edge tiles (M = 8000). Every output
    bit-identical to the register-staged kernel; sampled outputs within
    tolerance of the oracle."""
    print(f"case persistent tile changes {M}x{N}x{K} {lay}", flush=True)
    A = inputs.random_f16((M, K), 3 * M + K)
    B = inputs.random_f16((N, K) if lay == "NxK" else (K, N), 5 * N + K)
    Ad, Bd = _dev(A), _dev(B)
    base = tg.mm(Ad, Bd, lay, force_generic=1)
    C = tg.mm(Ad, Bd, lay)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), base.view(torch.int16))
    got = _host(C)
    I, J = inputs.sample_points(M, N, 2048, M + N + K + 1)
    ref, ab = oracle_mod.gemm_points(A, B, lay, I, J)
    res = oracle_mod.check(got[I, J], ref, ab)
    assert res["nfail"] == 0, res


def _nan_padded(rows, cols, ld, seed, offset):
    """A rows x cols matrix at `offset` elements into a buffer with row stride ld,
    every element outside the matrix (row padding and trailing space) a NaN."""
    buf = np.full(offset + rows * ld + 64, np.float16(np.nan), dtype=np.float16)
    view = np.lib.stride_tricks.as_strided(buf[offset:], (rows, cols), (2 * ld, 2))
    view[...] = inputs.random_f16((rows, cols), seed)
    return buf, np.ascontiguousarray(view)


@pytest.mark.parametrize("mode", ["auto", "tile256", "generic"])
@pytest.mark.parametrize("lay", ["NxK", "KxN"])
@pytest.mark.parametrize("K", [5, 37, 261, 264, 512 + 24, 1000])
def test_nan_beyond_k_and_edges_never_leaks(oracle_mod, lay, K, mode):
    """Padding past K, past N (row stride slack) and after the last element is NaN;
    odd strides and an odd element offset leave the rows only 2-byte aligned. Every
    output must still match the oracle, so no padded element reaches the sums."""
    print(f"case nan-padding {lay} K={K} {mode}", flush=True)
    M, N, off = 300, 270, 3
    lda = K + 5
    Abuf, A = _nan_padded(M, K, lda, K, off)
    if lay == "NxK":
        ldb = K + 3
        Bbuf, B = _nan_padded(N, K, ldb, K + 1, off)
    else:
        ldb = N + 7
        Bbuf, B = _nan_padded(K, N, ldb, K + 1, off)
    Ad, Bd = _dev(Abuf), _dev(Bbuf)
    C = torch.empty((M, N), dtype=torch.float16, device=DEV)
    rc = tg.tgemm_f16_config(M, N, K, Ad.data_ptr() + 2 * off, lda, Bd.data_ptr() + 2 * off, ldb, lay,
                             C.data_ptr(), N, torch.cuda.current_stream().cuda_stream, int(mode == "generic"),
                             tile_m=256 if mode == "tile256" else 0)
    assert rc == tg.TGEMM_OK
    got = _host(C)
    assert np.isfinite(got.astype(np.float32)).all(), "a padded NaN reached an output"
    _full_check(oracle_mod, A, B, lay, got, f"nan padding {lay} K={K} {mode}")


@pytest.mark.parametrize("lay,M,N,K,ldb", [
    ("KxN", 64, 3, 100, 3), ("KxN", 100, 7, 300, 7), ("KxN", 129, 1, 77, 1), ("KxN", 64, 3, 100, 8),
    ("NxK", 70, 5, 130, 130), ("NxK", 64, 300, 5, 5), ("KxN", 64, 300, 5, 300), ("NxK", 64, 300, 5, 8),
])
def test_narrow_operands(oracle_mod, lay, M, N, K, ldb):
    """Operands with rows narrower than 8 elements (K or N below 8, tight
    strides) and the same shapes with strides of 8: full parity with the
    oracle. In a K x N B of 3-element rows a 16-byte access at row k runs past
    the end of B for the last rows, not only the last one."""
    print(f"case narrow {lay} {M}x{N}x{K} ldb={ldb}", flush=True)
    lda = K if K >= 8 or ldb < 8 else 8
    A = inputs.random_f16((M, K), M + N + K)
    B = inputs.random_f16((K, N) if lay == "KxN" else (N, K), 3 * (M + N + K))
    rows, cols = B.shape
    Abuf = np.zeros((M, lda), dtype=np.float16)
    Abuf[:, :K] = A
    Bbuf = np.zeros((rows, ldb), dtype=np.float16)
    Bbuf[:, :cols] = B
    Ad, Bd = _dev(Abuf), _dev(Bbuf)
    for tile_m in (0, 256):                          # automatic (small grid: 64-row tiles) and 256-row tiles
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        rc = tg.tgemm_f16_config(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, lay, C.data_ptr(), N,
                                 torch.cuda.current_stream().cuda_stream, 0, tile_m=tile_m)
        assert rc == tg.TGEMM_OK
        _full_check(oracle_mod, A, B, lay, _host(C), f"narrow {lay} {M}x{N}x{K} ldb={ldb} tile_m={tile_m}")


@pytest.mark.parametrize("lay", ["NxK", "KxN"])
def test_inf_in_neighbouring_row_stays_local(lay):
    """Compact operands (ld = row length): an Inf in one row of B must not turn the
    neighbouring output column into NaN (elements past K belong to the next row)."""
    print(f"case inf neighbour {lay}", flush=True)
    M, N, K = 300, 270, 264 + 4
    A = inputs.random_f16((M, K), 7)
    B = inputs.random_f16((N, K) if lay == "NxK" else (K, N), 8)
    if lay == "NxK":
        B[6, 0] = np.float16(np.inf)          # B[:, 6] holds the Inf; k = K of row 5 would be this element
    else:
        B[0, 6] = np.float16(np.inf)
    C = _run(A, B, lay)
    cols = np.isfinite(C.astype(np.float32)).all(axis=0)
    assert not cols[6] and cols[5] and cols[7] and cols[:6].all() and cols[7:].all()


def test_mfma_issue_probe_runs():
    """The matrix-core ceiling probe (measurement aid) launches on binary16 data and
    produces finite sums; bad sizes are rejected before any launch."""
    print("case mfma ceiling probe", flush=True)
    data = _dev(inputs.random_f16((1 << 19,), 7) * np.float16(0.1))     # 1 MiB
    out = torch.empty(8 * 256, dtype=torch.float32, device=DEV)
    clk = torch.zeros(16, dtype=torch.int64, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    probe.mfma_issue_probe(8, 4, data.data_ptr(), 1 << 20, out.data_ptr(), clk.data_ptr(), st)
    probe.mfma_issue_probe(8, 4, data.data_ptr(), 1 << 20, out.data_ptr(), None, st)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    # shader cycles and 100 MHz ticks per workgroup: a clock between 0.5 and 3 GHz
    c = clk.cpu().numpy().reshape(8, 2).astype(np.float64)
    assert (c > 0).all()
    ghz = c[:, 0] / c[:, 1] / 10.0
    assert ((ghz > 0.5) & (ghz < 3.0)).all(), ghz
    for wg, nb in ((0, 1 << 20), (8, (1 << 20) + 2), (8, 1 << 19)):
        with pytest.raises(tg.TgemmError):
            probe.mfma_issue_probe(wg, 4, data.data_ptr(), nb, out.data_ptr(), None, st)


@pytest.mark.parametrize("kind", list(probe.STREAM_KINDS))
def test_mfma_stream_probe_runs(kind):
    """Each instruction-stream probe (measurement aid) launches on binary16 data,
    produces finite sums in every thread's slot and records a plausible clock."""
    print(f"case stream probe {kind}", flush=True)
    _, threads, _ = probe.STREAM_KINDS[kind]
    data = _dev(inputs.random_f16((1 << 19,), 8) * np.float16(0.1))     # 1 MiB
    out = torch.full((8 * threads,), float("nan"), dtype=torch.float32, device=DEV)
    clk = torch.zeros(16, dtype=torch.int64, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    probe.mfma_stream_probe(kind, 8, 4, data.data_ptr(), 1 << 20, out.data_ptr(), clk.data_ptr(), st)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    c = clk.cpu().numpy().reshape(8, 2).astype(np.float64)
    assert (c > 0).all()
    ghz = c[:, 0] / c[:, 1] / 10.0
    assert ((ghz > 0.5) & (ghz < 3.0)).all(), ghz


def test_xcd_probe_dispatch_order():
    """The die probe (measurement aid for the die-aware raster): over launches of
    8192 workgroups every recorded die number lies in [0, 8) and workgroup w ran
    on die (w + c) mod 8, c fixed within a launch (the round-robin starts where
    the previous launch stopped). So the workgroups that share a die are those
    with equal w mod 8, which is what the raster's renumbering assumes."""
    print("case xcd probe", flush=True)
    n = 8192
    st = torch.cuda.current_stream().cuda_stream
    out = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    for launch in range(3):
        probe.xcd_probe(n - launch, out.data_ptr(), st)     # 8192, 8191, 8190 workgroups
        torch.cuda.synchronize()
        got = out.cpu().numpy()[: n - launch]
        c = (got - np.arange(n - launch)) % 8
        print(f"  launch {launch}: per die {np.bincount(np.clip(got, 0, 15), minlength=8).tolist()}, "
              f"offsets {sorted(set(c.tolist()))}", flush=True)
        assert got.min() >= 0 and got.max() < 8
        assert (c == c[0]).all()
    with pytest.raises(tg.TgemmError):
        probe.xcd_probe(0, out.data_ptr(), st)


def _signed(bits, rng):
    return bits | (rng.integers(0, 2, size=bits.shape).astype(np.uint16) << 15)


@pytest.mark.parametrize("generic", [0, 1])
@pytest.mark.parametrize("lay", ["NxK", "KxN"])
def test_binary16_subnormals_kept(lay, generic):
    """Subnormal binary16 values pass through unchanged. As operands: random
    subnormals times the identity give C = A bit for bit, so the matrix
    instructions do not flush subnormal inputs. As results: the smallest normals
    (even significands) times 1/2 are exact subnormals, so the fp32 -> binary16
    store does not flush them either."""
    print(f"case subnormals {lay} generic={generic}", flush=True)
    M = N = K = 256
    rng = np.random.default_rng(11)
    A1 = _signed(rng.integers(1, 0x400, size=(M, K)).astype(np.uint16), rng).view(np.float16)
    eye = np.eye(K, dtype=np.float16)                        # symmetric: either layout
    C1 = _run(A1, eye, lay, force_generic=generic)
    lost = int(np.sum(C1.view(np.uint16) != A1.view(np.uint16)))
    assert lost == 0, f"{lost} of {M * K} subnormal operands changed"
    A2 = _signed((0x400 | (2 * rng.integers(0, 0x200, size=(M, K)))).astype(np.uint16), rng).view(np.float16)
    C2 = _run(A2, (0.5 * eye).astype(np.float16), lay, force_generic=generic)
    want = (A2.astype(np.float64) / 2).astype(np.float16)
    assert (np.abs(want.astype(np.float64)) < 2.0 ** -14).all() and (want != 0).all()
    lost = int(np.sum(C2.view(np.uint16) != want.view(np.uint16)))
    assert lost == 0, f"{lost} of {M * K} subnormal results changed"


def test_bfloat16_subnormal_operands_kept():
    """The same for bfloat16 operands (exponent field 0, significand 1..127),
    bfloat16 C: A times the identity gives A bit for bit."""
    print("case bf16 subnormals", flush=True)
    M = N = K = 256
    rng = np.random.default_rng(12)
    A = _signed(rng.integers(1, 0x80, size=(M, K)).astype(np.uint16), rng)
    eye = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    Ad = torch.from_numpy(A.view(np.int16)).to(DEV).view(torch.bfloat16)
    Bd = torch.from_numpy(eye.view(np.int16)).to(DEV).view(torch.bfloat16)
    for generic in (0, 1):
        C = tg.gemm(Ad, Bd, "KxN", out_dtype=torch.bfloat16, force_generic=generic)
        got = C.view(torch.int16).cpu().numpy().view(np.uint16)
        lost = int(np.sum(got != A))
        assert lost == 0, f"generic={generic}: {lost} of {M * K} subnormal operands changed"
