"""GPU parity at row strides past the direct-to-LDS limits, and for B stored
K x N wider than 2^31 bytes per 64 k rows' worth of offsets.

* Row strides above 4,000,000 elements (16-byte aligned) take the
  register-staged kernel with 128-bit operand loads: full oracle parity for
  both B layouts, plain and with the epilogue, with M, N edges and a K tail,
  every element outside the operands a NaN; bit-identical to the same kernel
  with element loads.
* B stored K x N is rebased at every K step, so a B of several GiB (a
  vocabulary-sized projection, or a padded stride) streams straight into LDS:
  the plan says so, and the result is bit-identical to the register-staged
  kernel and within tolerance of the oracle.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import dense_tiled_gemm_tgemm_amd as tg  # noqa: E402
from dense_tiled_gemm_tgemm_amd import inputs  # noqa: E402

DEV = "cuda:0"
V, DMA = 1, 8
WIDE = 4_000_008            # elements: past the direct-to-LDS stride limit, 16-byte rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    yield
    torch.cuda.synchronize()


def _st():
    return torch.cuda.current_stream().cuda_stream


def _padded(x16, ld, dt=torch.float16):
    """The rows of x16 (numpy uint16/float16, rows x cols) placed at row stride ld
    in a device buffer whose every other element is a NaN."""
    rows, cols = x16.shape
    buf = torch.full((rows * ld + 64,), float("nan"), dtype=dt, device=DEV)
    src = torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).to(DEV).view(dt)
    buf.as_strided((rows, cols), (ld, 1)).copy_(src)
    return buf


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("wide", ["A", "B"])
@pytest.mark.parametrize("lay", ["KxN", "NxK"])
def test_register_staged_128bit_loads_full_parity(oracle_mod, lay, wide):
    """lda or ldb = 4,000,008: 128-bit loads through registers. M = 37 and
    N = 300 leave partial tiles, K = 200 a partial 64-deep step."""
    M, N, K = 37, 300, 200
    print(f"case wide stride {wide} {lay} {M}x{N}x{K}", flush=True)
    A = inputs.random_f16((M, K), 501)
    B = inputs.random_f16((K, N) if lay == "KxN" else (N, K), 502)
    lda = WIDE if wide == "A" else K
    ldb = WIDE if wide == "B" else (304 if lay == "KxN" else K)
    Ad, Bd = _padded(A, lda), _padded(B, ldb)
    C = torch.empty((M, N), dtype=torch.float16, device=DEV)
    rc, plan = tg.tgemm_plan_f16(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, lay, C.data_ptr(), N)
    assert rc == tg.TGEMM_OK and plan["variant"] & V and not plan["variant"] & DMA, plan
    assert tg.tgemm_f16(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, lay, C.data_ptr(), N, _st()) == tg.TGEMM_OK
    got = _bits(C)
    ref, absum = oracle_mod.gemm(A, B, lay)
    res = oracle_mod.check(got, ref, absum)
    assert res["nfail"] == 0, res
    # the same kernel with element loads gives the same bits
    C2 = torch.empty_like(C)
    assert tg.tgemm_f16_config(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, lay, C2.data_ptr(), N, _st(),
                               1) == tg.TGEMM_OK
    assert np.array_equal(_bits(C2), got)


@pytest.mark.parametrize("lay", ["KxN", "NxK"])
@pytest.mark.parametrize("ab,ct", [("f16", "f32"), ("bf16", "bf16")])
def test_register_staged_128bit_loads_with_epilogue(oracle_mod, lay, ab, ct):
    """The same kernel with alpha, a per-column bias and the rectifier, binary16
    or bfloat16 operands, fp32 or bfloat16 C, lda = 4,000,008."""
    M, N, K = 37, 300, 200
    print(f"case wide stride epilogue {ab}->{ct} {lay}", flush=True)
    gen = inputs.random_f16 if ab == "f16" else inputs.random_bf16
    dt = torch.float16 if ab == "f16" else torch.bfloat16
    A = gen((M, K), 511)
    B = gen((K, N) if lay == "KxN" else (N, K), 512)
    bias = inputs.random_bias(N, 513)
    lda, ldb = WIDE, (304 if lay == "KxN" else K)
    Ad, Bd = _padded(A, lda, dt), _padded(B, ldb, dt)
    bd = torch.from_numpy(bias).to(DEV)
    cdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[ct]
    C = torch.empty((M, N), dtype=cdt, device=DEV)
    rc, plan = tg.tgemm_plan_gemm(M, N, K, ab, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, lay, ct, C.data_ptr(), N,
                                  0.5, bd.data_ptr(), "relu")
    assert rc == tg.TGEMM_OK and plan["variant"] & V and not plan["variant"] & DMA, plan
    assert tg.tgemm_gemm(M, N, K, ab, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, lay, ct, C.data_ptr(), N, 0.5,
                         bd.data_ptr(), "relu", _st()) == tg.TGEMM_OK
    torch.cuda.synchronize()
    got = C.cpu().numpy() if ct == "f32" else C.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, tol = oracle_mod.gemm_ex(A, B, lay, ab, 0.5, bias, "relu")
    res = oracle_mod.check_ex(got, ct, ref, tol)
    assert res["nfail"] == 0, res


def test_padded_kxn_stride_streams_into_lds(oracle_mod):
    """B stored K x N with a padded stride whose K-step offsets from the first
    k row exceed 2^31 bytes ((K + 64) * ldb * 2 > 2^31): still the direct-to-LDS
    kernel (each K step has its own resource), K = 1000 with a partial last
    step, rows past K and the padding NaN. Bit-identical to the register-staged
    kernel; full parity with the oracle."""
    M, N, K, ldb = 300, 700, 1000, 1_100_000
    print(f"case padded K x N stride {M}x{N}x{K} ldb={ldb}", flush=True)
    assert (K + 64) * ldb * 2 > 2 ** 31
    A = inputs.random_f16((M, K), 521)
    B = inputs.random_f16((K, N), 522)
    Ad, Bd = _padded(A, K), _padded(B, ldb)
    C = torch.empty((M, N), dtype=torch.float16, device=DEV)
    rc, plan = tg.tgemm_plan_f16(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), ldb, "KxN", C.data_ptr(), N)
    assert rc == tg.TGEMM_OK and plan["variant"] & DMA, plan
    for ks, st in ((0, 0), (64, 2), (32, 3)):
        Cx = torch.empty_like(C)
        assert tg.tgemm_f16_config(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), ldb, "KxN", Cx.data_ptr(), N, _st(),
                                   0, 0, 0, ks, st) == tg.TGEMM_OK
        if ks == 0:
            C = Cx
        else:
            assert np.array_equal(_bits(Cx), _bits(C)), (ks, st)
    got = _bits(C)
    Cg = torch.empty_like(C)
    assert tg.tgemm_f16_config(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), ldb, "KxN", Cg.data_ptr(), N, _st(),
                               1) == tg.TGEMM_OK
    assert np.array_equal(_bits(Cg), got)
    ref, absum = oracle_mod.gemm(A, B, "KxN")
    res = oracle_mod.check(got, ref, absum)
    assert res["nfail"] == 0, res


def test_vocabulary_projection_kxn_streams_into_lds(oracle_mod):
    """A vocabulary-sized projection with B stored K x N: 300 x 152064 x 8192,
    2.5 GB of B, 1188 tiles on the persistent direct-to-LDS kernel.
    Bit-identical to the register-staged kernel; every output of a row and
    column subset (all tail rows, the last tile's columns, seeded others)
    within tolerance of the oracle, which needs only those rows of A and
    columns of B."""
    M, N, K = 300, 152064, 8192
    print(f"case vocabulary projection K x N {M}x{N}x{K}", flush=True)
    A = inputs.random_f16((M, K), 531)
    B = np.empty((K, N), dtype=np.float16)
    step = 8192
    for c0 in range(0, N, step):
        c1 = min(N, c0 + step)
        B[:, c0:c1] = inputs.random_f16((K, c1 - c0), 532 + c0 // step)
    Ad = torch.from_numpy(A.view(np.int16)).to(DEV).view(torch.float16)
    Bd = torch.from_numpy(B.view(np.int16)).to(DEV).view(torch.float16)
    C = torch.empty((M, N), dtype=torch.float16, device=DEV)
    rc, plan = tg.tgemm_plan_f16(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, "KxN", C.data_ptr(), N)
    assert rc == tg.TGEMM_OK and plan["variant"] & DMA and plan["bk"] == 64, plan
    assert tg.tgemm_f16(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, "KxN", C.data_ptr(), N, _st()) == tg.TGEMM_OK
    got = _bits(C)
    Cg = torch.empty_like(C)
    assert tg.tgemm_f16_config(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N, "KxN", Cg.data_ptr(), N, _st(),
                               1) == tg.TGEMM_OK
    assert np.array_equal(_bits(Cg), got)
    rng = np.random.default_rng(533)
    rows = np.unique(np.concatenate([np.arange(256, M), rng.choice(256, 24, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(N - 256, N), rng.choice(N - 256, 256, replace=False)]))
    ref, absum = oracle_mod.gemm(np.ascontiguousarray(A[rows]), np.ascontiguousarray(B[:, cols]), "KxN")
    res = oracle_mod.check(np.ascontiguousarray(got[np.ix_(rows, cols)]), ref, absum)
    assert res["nfail"] == 0, res


def test_binary32_operands_padded_kxn_stride(oracle_mod):
    """Binary32 operands, B stored K x N with a stride whose K-step offsets
    from the first k row exceed 2^31 bytes: the pipelined buffer-load kernel
    (each 16-deep step has its own B resource), rows past K and the padding
    NaN. Bit-identical to the general register-staged kernel; full parity
    with the oracle, plain and with the epilogue into fp32."""
    M, N, K, ldb = 300, 520, 1000, 600_000
    print(f"case binary32 padded K x N stride {M}x{N}x{K} ldb={ldb}", flush=True)
    assert (K + 64) * ldb * 4 > 2 ** 31
    A = inputs.random_f32((M, K), 541)
    B = inputs.random_f32((K, N), 542)
    Ad = torch.from_numpy(A).to(DEV)
    Bd = torch.full((K * ldb + 64,), float("nan"), dtype=torch.float32, device=DEV)
    Bd.as_strided((K, N), (ldb, 1)).copy_(torch.from_numpy(B).to(DEV))
    bias = inputs.random_bias(N, 543)
    bd = torch.from_numpy(bias).to(DEV)
    for alpha, bptr, act in ((1.0, None, "none"), (0.5, bd.data_ptr(), "relu")):
        C = torch.empty((M, N), dtype=torch.float32, device=DEV)
        rc, plan = tg.tgemm_plan_gemm(M, N, K, "f32", Ad.data_ptr(), K, Bd.data_ptr(), ldb, "KxN", "f32",
                                      C.data_ptr(), N, alpha, bptr, act)
        assert rc == tg.TGEMM_OK and plan["variant"] & DMA, plan
        assert tg.tgemm_gemm(M, N, K, "f32", Ad.data_ptr(), K, Bd.data_ptr(), ldb, "KxN", "f32", C.data_ptr(), N,
                             alpha, bptr, act, _st()) == tg.TGEMM_OK
        Cg = torch.empty_like(C)
        assert tg.tgemm_gemm_config(M, N, K, "f32", Ad.data_ptr(), K, Bd.data_ptr(), ldb, "KxN", "f32",
                                    Cg.data_ptr(), N, alpha, bptr, act, _st(), 1) == tg.TGEMM_OK
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), Cg.cpu().numpy().view(np.uint32))
        ref, tol = oracle_mod.gemm_ex(A, B, "KxN", "f32", alpha, bias if bptr else None, act)
        res = oracle_mod.check_ex(got, "f32", ref, tol)
        assert res["nfail"] == 0, res
