"""GPU parity of the typed GEMM (binary16 / bfloat16 inputs; binary16,
bfloat16 or fp32 output; scale, bias and rectifier on store) through the C
ABI, against the extended CPU oracle:

  |g - ref| <= 1e-3 * (|alpha| * sum_k |a*b| + |bias[j]|) + ulp_out(ref)

element by element, and bit-exact where the answer is exactly representable
(integer sums stored in fp32) or where two outputs of the library must agree
(one accumulation rounded to two output types; every pipeline and raster).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import dense_tiled_gemm_tgemm_amd as tg  # noqa: E402
from dense_tiled_gemm_tgemm_amd import inputs  # noqa: E402

DEV = "cuda:0"
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
COMBOS = [(ab, ct) for ab in ("f16", "bf16") for ct in ("f16", "bf16", "f32")]
EPI = {"plain": dict(alpha=1.0, bias=False, act="none"),
       "epi": dict(alpha=-0.625, bias=True, act="relu")}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.load()
    yield
    torch.cuda.synchronize()


def _bits(shape, seed, ab, dist=("uniform", -1.0, 1.0)):
    """Seeded operand as uint16 bit patterns of its type."""
    if ab == "f16":
        return inputs.random_f16(shape, seed, dist).view(np.uint16)
    return inputs.random_bf16(shape, seed, dist)


def _dev(bits, ab):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)
    return t.view(TORCH_DT[ab])


def _out_np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _bias(N, seed, on):
    if not on:
        return None, None
    b = inputs.random_bias(N, seed, scale=2.0)
    return b, torch.from_numpy(b).to(DEV)


def _check(oracle_mod, A, B, lay, ab, ct, got, alpha, bias_np, act, what, I=None, J=None):
    ref, tol = oracle_mod.gemm_ex(A, B, lay, ab, alpha, bias_np, act, I=I, J=J)
    sel = got if I is None else got[I, J]
    res = oracle_mod.check_ex(sel, ct, ref, tol)
    assert res["nfail"] == 0, f"{what}: {res}"
    return res


SMALL = [(1, 1, 1), (31, 17, 65), (255, 257, 63), (300, 520, 200), (513, 300, 8), (512, 512, 512)]


@pytest.mark.parametrize("epi", ["plain", "epi"])
@pytest.mark.parametrize("lay", ["KxN", "NxK"])
@pytest.mark.parametrize("ab,ct", COMBOS)
@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes_full_parity(oracle_mod, M, N, K, ab, ct, lay, epi):
    print(f"case typed {M}x{N}x{K} {ab}->{ct} {lay} {epi}", flush=True)
    seed = (M * 7 + N * 13 + K * 17) % 100003
    A = _bits((M, K), seed, ab)
    B = _bits((K, N) if lay == "KxN" else (N, K), seed + 1, ab)
    e = EPI[epi]
    b_np, b_dev = _bias(N, seed + 2, e["bias"])
    Ad, Bd = _dev(A, ab), _dev(B, ab)
    C = tg.gemm(Ad, Bd, lay, out_dtype=TORCH_DT[ct], alpha=e["alpha"], bias=b_dev, act=e["act"])
    _check(oracle_mod, A, B, lay, ab, ct, _out_np(C), e["alpha"], b_np, e["act"], f"{M}x{N}x{K} {ab}->{ct} {lay}")
    # 256-row tiles (the automatic launch takes smaller ones on these grids): the same bits
    C256 = tg.gemm(Ad, Bd, lay, out_dtype=TORCH_DT[ct], alpha=e["alpha"], bias=b_dev, act=e["act"], tile_m=256)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C256.view(torch.int16))


@pytest.mark.parametrize("lay", ["KxN", "NxK"])
@pytest.mark.parametrize("ab,ct", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("M,N,K", [(300, 520, 200), (257, 255, 129)])
def test_register_staged_path_full_parity(oracle_mod, M, N, K, ab, ct, lay):
    print(f"case typed generic {M}x{N}x{K} {ab}->{ct} {lay}", flush=True)
    A = _bits((M, K), M + 3 * K, ab)
    B = _bits((K, N) if lay == "KxN" else (N, K), N + 5 * K, ab)
    b_np, b_dev = _bias(N, 11, True)
    Ad, Bd = _dev(A, ab), _dev(B, ab)
    C = tg.gemm(Ad, Bd, lay, out_dtype=TORCH_DT[ct], alpha=0.5, bias=b_dev, act="relu", force_generic=1)
    _check(oracle_mod, A, B, lay, ab, ct, _out_np(C), 0.5, b_np, "relu", "generic")
    C2 = tg.gemm(Ad, Bd, lay, out_dtype=TORCH_DT[ct], alpha=0.5, bias=b_dev, act="relu")
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16) if ct != "f32" else C, C2.view(torch.int16) if ct != "f32" else C2)


def test_plain_f16_equals_tgemm_f16_bitwise():
    """The typed entry point without epilogue is the binary16 product, bit for bit."""
    print("case typed plain = f16", flush=True)
    A = _dev(_bits((700, 300), 1, "f16"), "f16")
    B = _dev(_bits((600, 300), 2, "f16"), "f16")
    C1 = tg.mm(A, B, "NxK")
    C2 = tg.gemm(A, B, "NxK")
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("lay,M,N,K", [("NxK", 700, 600, 264), ("KxN", 1300, 1000, 4099), ("NxK", 520, 777, 72)])
def test_one_accumulation_rounded_to_each_output_type(ab, lay, M, N, K):
    """The fp32 output holds the accumulator itself; the binary16 and bfloat16
    outputs are that value rounded to nearest even (torch's CPU conversions),
    bit for bit. The same holds with the epilogue applied."""
    print(f"case typed rounding {ab} {lay} {M}x{N}x{K}", flush=True)
    A = _dev(_bits((M, K), M + K, ab), ab)
    B = _dev(_bits((N, K) if lay == "NxK" else (K, N), N + K, ab), ab)
    _, b_dev = _bias(N, 5, True)
    for kw in (dict(), dict(alpha=-1.75, bias=b_dev, act="relu")):
        c32 = tg.gemm(A, B, lay, out_dtype=torch.float32, **kw)
        c16 = tg.gemm(A, B, lay, out_dtype=torch.float16, **kw)
        cbf = tg.gemm(A, B, lay, out_dtype=torch.bfloat16, **kw)
        torch.cuda.synchronize()
        h32 = c32.cpu()
        assert torch.equal(h32.to(torch.float16).view(torch.int16), c16.cpu().view(torch.int16))
        assert torch.equal(h32.to(torch.bfloat16).view(torch.int16), cbf.cpu().view(torch.int16))


@pytest.mark.parametrize("ab", ["f16", "bf16"])
def test_epilogue_is_one_fused_multiply_add_then_rectifier(ab):
    """fp32 output with the epilogue equals rn32(alpha * s + b) clipped at zero,
    s the plain fp32 output (the fused multiply-add rounds once: computed here
    in fp64 from the exact product alpha * s, within one fp32 ulp)."""
    print(f"case typed epilogue closed form {ab}", flush=True)
    M, N, K = 640, 900, 333
    A = _dev(_bits((M, K), 21, ab), ab)
    B = _dev(_bits((K, N), 22, ab), ab)
    b_np, b_dev = _bias(N, 23, True)
    s = _out_np(tg.gemm(A, B, "KxN", out_dtype=torch.float32)).astype(np.float64)
    alpha = np.float32(0.3)
    got = _out_np(tg.gemm(A, B, "KxN", out_dtype=torch.float32, alpha=float(alpha), bias=b_dev,
                          act="relu")).astype(np.float64)
    want = np.maximum((float(alpha) * s + b_np.astype(np.float64)).astype(np.float32), 0).astype(np.float64)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp)
    assert (got == 0).sum() > 0 and (got > 0).sum() > 0
    # scale only, no bias: the product alpha * s rounded once
    got2 = _out_np(tg.gemm(A, B, "KxN", out_dtype=torch.float32, alpha=-2.0)).astype(np.float64)
    assert np.array_equal(got2, -2.0 * s)


@pytest.mark.parametrize("name", ["sq256", "sq4096", "ragged", "sq8192_nt", "qkv_proj"])
def test_bf16_ternary_bit_exact_fp32_output(oracle_mod, name):
    """Entries in {-1, 0, 1} are exact in bfloat16 and every partial sum is an
    integer below 2^24: the fp32 output is exact at the workload shapes."""
    w = inputs.WORKLOADS[name]
    print(f"case typed ternary {name}", flush=True)
    A = inputs.to_bf16_bits(inputs.ternary_f16((w.M, w.K), 200 + w.seed).astype(np.float64))
    B = inputs.to_bf16_bits(inputs.ternary_f16(w.b_shape, 201 + w.seed).astype(np.float64))
    C = tg.gemm(_dev(A, "bf16"), _dev(B, "bf16"), w.b_layout, out_dtype=torch.float32)
    got = _out_np(C)
    I, J = inputs.sample_points(w.M, w.N, 8192, 202 + w.seed)
    ref, _ = oracle_mod.gemm_ex(A, B, w.b_layout, "bf16", I=I, J=J)
    assert np.array_equal(got[I, J].astype(np.float64), ref)
    g = got.astype(np.float64)
    assert np.all(g == np.round(g)) and np.abs(g).max() <= w.K


@pytest.mark.parametrize("ct", ["bf16", "f32"])
@pytest.mark.parametrize("name", ["sq4096", "ragged", "sq8192_nt", "qkv_proj"])
def test_bf16_workload_parity(oracle_mod, name, ct):
    """The workloads with bfloat16 operands drawn from the same seeded values,
    launched as the benchmark launches them (raw C call on torch's stream)."""
    w = inputs.WORKLOADS[name]
    print(f"case typed workload {name} bf16->{ct}", flush=True)
    A, B = inputs.make_inputs(w, "bf16")
    Ad, Bd = _dev(A, "bf16"), _dev(B, "bf16")
    C = torch.empty((w.M, w.N), dtype=TORCH_DT[ct], device=DEV)
    rc = tg.tgemm_gemm(w.M, w.N, w.K, "bf16", Ad.data_ptr(), w.K, Bd.data_ptr(), B.shape[1], w.b_layout, ct,
                       C.data_ptr(), w.N, 1.0, None, "none", torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TGEMM_OK
    got = _out_np(C)
    I, J = inputs.sample_points(w.M, w.N, 8192, w.seed + 3000)
    res = _check(oracle_mod, A, B, w.b_layout, "bf16", ct, got, 1.0, None, "none", name, I, J)
    print(f"  {name}: {res['n']} checked, worst {res['worst']:.4f}", flush=True)


@pytest.mark.parametrize("ab,ct", [("f16", "f32"), ("f16", "f16"), ("bf16", "bf16")])
def test_epilogue_workload_parity(oracle_mod, ab, ct):
    """Scale, bias and rectifier on the projection workload (fused QKV width)."""
    w = inputs.WORKLOADS["qkv_proj"]
    print(f"case typed epilogue workload {ab}->{ct}", flush=True)
    A, B = inputs.make_inputs(w, ab)
    if ab == "f16":
        A, B = A.view(np.uint16), B.view(np.uint16)
    b_np, b_dev = _bias(w.N, 31, True)
    C = tg.gemm(_dev(A, ab), _dev(B, ab), w.b_layout, out_dtype=TORCH_DT[ct], alpha=0.125, bias=b_dev,
                act="relu")
    got = _out_np(C)
    I, J = inputs.sample_points(w.M, w.N, 8192, 32)
    _check(oracle_mod, A, B, w.b_layout, ab, ct, got, 0.125, b_np, "relu", "qkv epilogue", I, J)


@pytest.mark.parametrize("ab,ct", COMBOS)
@pytest.mark.parametrize("lay", ["NxK", "KxN"])
def test_persistent_grid_and_pipelines_agree(oracle_mod, ab, ct, lay):
    """More tiles than compute units (the persistent kernel), with the
    epilogue: bit-identical to the register-staged kernel, to 32-deep steps,
    to the 128- and 64-row tiles (two workgroups per compute unit) and under
    another raster; sampled outputs within tolerance."""
    M, N, K = 4300, 4300, 1000
    print(f"case typed persistent {ab}->{ct} {lay}", flush=True)
    A = _bits((M, K), 41, ab)
    B = _bits((N, K) if lay == "NxK" else (K, N), 42, ab)
    b_np, b_dev = _bias(N, 43, True)
    Ad, Bd = _dev(A, ab), _dev(B, ab)
    kw = dict(out_dtype=TORCH_DT[ct], alpha=-0.75, bias=b_dev, act="relu")
    outs = [tg.gemm(Ad, Bd, lay, **kw), tg.gemm(Ad, Bd, lay, force_generic=1, **kw),
            tg.gemm(Ad, Bd, lay, k_step=32, **kw), tg.gemm(Ad, Bd, lay, group_m=3, num_xcd=1, **kw),
            tg.gemm(Ad, Bd, lay, tile_m=128, **kw), tg.gemm(Ad, Bd, lay, tile_m=64, **kw)]
    torch.cuda.synchronize()
    base = outs[0] if ct == "f32" else outs[0].view(torch.int16)
    for o in outs[1:]:
        assert torch.equal(base, o if ct == "f32" else o.view(torch.int16))
    I, J = inputs.sample_points(M, N, 4096, 44)
    _check(oracle_mod, A, B, lay, ab, ct, _out_np(outs[0]), -0.75, b_np, "relu", "persistent", I, J)


@pytest.mark.parametrize("ab,ct", [c for c in COMBOS if c[1] != "f32"])
@pytest.mark.parametrize("lay", ["NxK", "KxN"])
def test_tile_changes_with_epilogue_bit_identical(oracle_mod, ab, ct, lay):
    """16-bit C with α, bias and the rectifier, four tiles per workgroup of the
    persistent kernel (the bias loads sit between the next tile's first loads
    and this tile's C stores): bit-identical to the register-staged kernel; sampled
    outputs within tolerance."""
    M, N, K = 8192, 8192, 640
    print(f"case typed tile changes {ab}->{ct} {lay}", flush=True)
    A = _bits((M, K), 51, ab)
    B = _bits((N, K) if lay == "NxK" else (K, N), 52, ab)
    b_np, b_dev = _bias(N, 53, True)
    Ad, Bd = _dev(A, ab), _dev(B, ab)
    kw = dict(out_dtype=TORCH_DT[ct], alpha=1.25, bias=b_dev, act="relu")
    C = tg.gemm(Ad, Bd, lay, **kw)
    base = tg.gemm(Ad, Bd, lay, force_generic=1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), base.view(torch.int16))
    I, J = inputs.sample_points(M, N, 2048, 54)
    _check(oracle_mod, A, B, lay, ab, ct, _out_np(C), 1.25, b_np, "relu", "tile changes", I, J)


@pytest.mark.parametrize("ab,ct", COMBOS)
@pytest.mark.parametrize("lay", ["NxK", "KxN"])
def test_odd_step_count_32_deep_ring_agrees(oracle_mod, ab, ct, lay):
    """K = 1040: 33 steps of 32 (an odd count, so the ring runs one leading
    all-zero step) with a partial last step (K mod 32 = 16). The 32-deep ring,
    the default 64-deep pipeline, the 128- and 64-row tiles and the
    register-staged kernel give the same bits, with the epilogue; every
    output within tolerance of the oracle."""
    M, N, K = 520, 777, 1040
    print(f"case typed odd steps {ab}->{ct} {lay}", flush=True)
    A = _bits((M, K), 61, ab)
    B = _bits((N, K) if lay == "NxK" else (K, N), 62, ab)
    b_np, b_dev = _bias(N, 63, True)
    Ad, Bd = _dev(A, ab), _dev(B, ab)
    kw = dict(out_dtype=TORCH_DT[ct], alpha=1.25, bias=b_dev, act="relu")
    outs = [tg.gemm(Ad, Bd, lay, k_step=32, **kw), tg.gemm(Ad, Bd, lay, **kw),
            tg.gemm(Ad, Bd, lay, force_generic=1, **kw), tg.gemm(Ad, Bd, lay, tile_m=128, **kw),
            tg.gemm(Ad, Bd, lay, tile_m=64, **kw)]
    torch.cuda.synchronize()
    base = outs[0] if ct == "f32" else outs[0].view(torch.int16)
    for o in outs[1:]:
        assert torch.equal(base, o if ct == "f32" else o.view(torch.int16))
    _check(oracle_mod, A, B, lay, ab, ct, _out_np(outs[0]), 1.25, b_np, "relu", "odd steps")


@pytest.mark.parametrize("ct", ["f16", "bf16", "f32"])
def test_k_zero_stores_rectified_bias(ct):
    print(f"case typed K=0 {ct}", flush=True)
    A = torch.empty((300, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, 270), dtype=torch.bfloat16, device=DEV)
    b_np, b_dev = _bias(270, 51, True)
    C = torch.full((300, 270), 7.0, dtype=TORCH_DT[ct], device=DEV)
    tg.gemm(A, B, "KxN", out=C, alpha=2.0, bias=b_dev, act="relu")
    want = torch.from_numpy(np.maximum(b_np, 0)).to(TORCH_DT[ct])
    assert torch.equal(C.cpu(), want.expand(300, 270))


@pytest.mark.parametrize("ct,offset,pad", [
    ("f32", 0, 2),      # rows 16-byte aligned
    ("f32", 2, 6),      # rows 8-byte aligned: 16-byte stores at 8-byte alignment
    ("f32", 1, 3),      # rows 4-byte aligned
    ("bf16", 0, 2),     # rows 16-byte aligned
    ("f16", 4, 2),      # rows 8-byte aligned
    ("bf16", 1, 3),     # rows 2-byte aligned: 16-byte stores at 2-byte alignment
])
def test_output_alignment_paths_and_guard_band(oracle_mod, ct, offset, pad):
    """C inside a larger NaN-filled buffer (row stride N + pad, start `offset`
    elements in): 16-byte stores at every row alignment, element stores at the
    right edge, edge tiles, with the automatic launch (64-row tiles here) and
    with 256-row tiles; nothing outside the M x N window changes."""
    M, N, K = 300, 270, 130
    print(f"case typed guard {ct} offset={offset} pad={pad}", flush=True)
    A = _bits((M, K), 61, "bf16")
    B = _bits((K, N), 62, "bf16")
    b_np, b_dev = _bias(N, 63, True)
    ldc = N + pad
    total = offset + M * ldc + 64
    if ct == "f32":
        buf = torch.full((total,), float("nan"), dtype=torch.float32, device=DEV)
    else:
        buf = torch.full((total,), 0x7FC1 if ct == "bf16" else 0x7E01, dtype=torch.int16, device=DEV)
        buf = buf.view(TORCH_DT[ct])
    Ad, Bd = _dev(A, "bf16"), _dev(B, "bf16")
    fresh = buf.clone()
    for tile_m in (0, 256):
        buf = fresh.clone()
        rc = tg.tgemm_gemm_config(M, N, K, "bf16", Ad.data_ptr(), K, Bd.data_ptr(), N, "KxN", ct,
                                  buf.data_ptr() + offset * buf.element_size(), ldc, 1.5, b_dev.data_ptr(), "none",
                                  torch.cuda.current_stream().cuda_stream, tile_m=tile_m)
        assert rc == tg.TGEMM_OK
        host = _out_np(buf)
        win = host[offset:offset + M * ldc].reshape(M, ldc)
        _check(oracle_mod, A, B, "KxN", "bf16", ct, np.ascontiguousarray(win[:, :N]), 1.5, b_np, "none",
               f"guard {tile_m}")
        outside = np.concatenate([host[:offset], win[:, N:].ravel(), host[offset + M * ldc:]])
        if ct == "f32":
            assert np.isnan(outside).all()
        else:
            assert (outside == (0x7FC1 if ct == "bf16" else 0x7E01)).all()


def test_bias_nan_and_inf_propagate(oracle_mod):
    """A NaN bias makes its column NaN (the rectifier keeps NaN); an infinite
    bias its column infinite (or zero after the rectifier for -inf)."""
    print("case typed bias specials", flush=True)
    M, N, K = 64, 40, 32
    A = _bits((M, K), 71, "f16")
    B = _bits((K, N), 72, "f16")
    b = inputs.random_bias(N, 73)
    b[3], b[10], b[20] = np.nan, np.inf, -np.inf
    for act in ("none", "relu"):
        C = tg.gemm(_dev(A, "f16"), _dev(B, "f16"), "KxN", out_dtype=torch.float32, bias=torch.from_numpy(b).to(DEV),
                    act=act)
        got = _out_np(C)
        assert np.isnan(got[:, 3]).all()
        assert (got[:, 10] == np.inf).all()
        assert (got[:, 20] == (-np.inf if act == "none" else 0)).all()
        keep = [j for j in range(N) if j not in (3, 10, 20)]
        ref, tol = oracle_mod.gemm_ex(A, B, "KxN", "f16", 1.0, b, act)
        res = oracle_mod.check_ex(np.ascontiguousarray(got[:, keep]), "f32", np.ascontiguousarray(ref[:, keep]),
                                  np.ascontiguousarray(tol[:, keep]))
        assert res["nfail"] == 0, res


def test_binary16_output_overflow_is_infinity(oracle_mod):
    """Sums past binary16's range are stored as infinities of their sign."""
    print("case typed overflow", flush=True)
    K = 64
    A = np.full((32, K), 60.0, dtype=np.float16).view(np.uint16)
    B = np.full((K, 48), 30.0, dtype=np.float16)
    B[:, 1::2] *= -1
    B = B.view(np.uint16)
    C = tg.gemm(_dev(A, "f16"), _dev(B, "f16"), "KxN")        # sums are +-115200
    got = _out_np(C)
    ref, tol = oracle_mod.gemm_ex(A, B, "KxN", "f16")
    assert oracle_mod.check_ex(got, "f16", ref, tol)["nfail"] == 0
    f = got.view(np.float16)
    assert np.isposinf(f[:, 0::2]).all() and np.isneginf(f[:, 1::2]).all()


# ------------------------------------------------------------ binary32 operands --

def _f32(shape, seed, dist=("uniform", -1.0, 1.0)):
    return inputs.random_f32(shape, seed, dist)


def _d32(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.mark.parametrize("epi", ["plain", "epi"])
@pytest.mark.parametrize("lay", ["KxN", "NxK"])
@pytest.mark.parametrize("ct", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("M,N,K", SMALL + [(257, 255, 129)])
def test_f32_operands_small_shapes_full_parity(oracle_mod, M, N, K, ct, lay, epi):
    print(f"case f32-in {M}x{N}x{K} ->{ct} {lay} {epi}", flush=True)
    seed = (M * 11 + N * 5 + K * 3) % 100003
    A = _f32((M, K), seed)
    B = _f32((K, N) if lay == "KxN" else (N, K), seed + 1)
    e = EPI[epi]
    b_np, b_dev = _bias(N, seed + 2, e["bias"])
    Ad, Bd = _d32(A), _d32(B)
    C = tg.gemm(Ad, Bd, lay, out_dtype=TORCH_DT[ct], alpha=e["alpha"], bias=b_dev, act=e["act"])
    _check(oracle_mod, A, B, lay, "f32", ct, _out_np(C), e["alpha"], b_np, e["act"], f"f32 {M}x{N}x{K} {lay}")
    # element-wise operand loads (force_generic) give the same bits
    C2 = tg.gemm(Ad, Bd, lay, out_dtype=TORCH_DT[ct], alpha=e["alpha"], bias=b_dev, act=e["act"], force_generic=1)
    torch.cuda.synchronize()
    if ct == "f32":
        assert torch.equal(C, C2)
    else:
        assert torch.equal(C.view(torch.int16), C2.view(torch.int16))


@pytest.mark.parametrize("lay,offset,pad,N,K", [
    ("KxN", 1, 3, 270, 133), ("NxK", 1, 5, 270, 133), ("NxK", 0, 3, 270, 133), ("KxN", 2, 2, 270, 133),
    # K (and N for B stored K x N) multiples of 4: the pipelined kernel (buffer loads)
    ("KxN", 1, 3, 272, 132), ("NxK", 1, 5, 270, 132), ("NxK", 0, 4, 270, 132), ("KxN", 2, 2, 272, 4100),
])
def test_f32_operands_strided_and_offset(oracle_mod, lay, offset, pad, N, K):
    """Operands inside larger NaN-filled buffers: row strides of K + pad
    (N + pad) floats, bases `offset` floats in (only 4-byte aligned when offset
    is odd): NaN past K, past N or after the last row must never reach C."""
    M = 300
    print(f"case f32-in strided {lay} offset={offset} pad={pad} N={N} K={K}", flush=True)
    A = _f32((M, K), 91)
    B = _f32((K, N) if lay == "KxN" else (N, K), 92)
    bufA = np.full(offset + M * (K + pad), np.nan, dtype=np.float32)
    va = bufA[offset:offset + M * (K + pad)].reshape(M, K + pad)
    va[:, :K] = A
    rows_b, cols_b = B.shape
    bufB = np.full(offset + rows_b * (cols_b + pad), np.nan, dtype=np.float32)
    vb = bufB[offset:offset + rows_b * (cols_b + pad)].reshape(rows_b, cols_b + pad)
    vb[:, :cols_b] = B
    dA, dB = _d32(bufA), _d32(bufB)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    rc = tg.tgemm_gemm(M, N, K, "f32", dA.data_ptr() + 4 * offset, K + pad, dB.data_ptr() + 4 * offset,
                       cols_b + pad, lay, "f32", C.data_ptr(), N, 1.0, None, "none",
                       torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TGEMM_OK
    _check(oracle_mod, A, B, lay, "f32", "f32", _out_np(C), 1.0, None, "none", "f32 strided")


@pytest.mark.parametrize("M,N,K", [(300, 260, 133), (257, 512, 29), (64, 4, 5), (33, 300, 16), (1000, 1028, 1000),
                                   (520, 768, 4096), (300, 259, 133), (64, 5, 5), (33, 301, 16), (129, 1023, 64),
                                   (70, 6, 4)])
def test_f32_operands_kxn_direct_to_lds(oracle_mod, M, N, K):
    """Binary32 operands with B stored K x N take the direct-to-LDS kernel:
    full parity with the oracle (partial tiles in both directions, K tails,
    N not a multiple of 4 so that B's last row ends inside a 16-byte chunk,
    narrow B), and the same bits from every tile shape and ring depth and
    from the general kernel."""
    print(f"case f32-in KxN direct-to-LDS {M}x{N}x{K}", flush=True)
    seed = (M * 7 + N * 3 + K) % 1009
    A = _f32((M, K), seed)
    B = _f32((K, N), seed + 1)
    Ad, Bd = _d32(A), _d32(B)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    rc, info = tg.tgemm_plan_gemm(M, N, K, "f32", Ad.data_ptr(), K, Bd.data_ptr(), N, "KxN", "f32", C.data_ptr(), N)
    assert rc == 0 and info["variant"] & 8 and info["bn"] == 256, info
    C = tg.gemm(Ad, Bd, "KxN", out_dtype=torch.float32)
    _check(oracle_mod, A, B, "KxN", "f32", "f32", _out_np(C), 1.0, None, "none", f"f32 KxN {M}x{N}x{K}")
    for kw in (dict(tile_m=256), dict(tile_m=128), dict(tile_m=64), dict(tile_m=256, stages=3),
               dict(tile_m=256, stages=4), dict(force_generic=1)):
        C2 = tg.gemm(Ad, Bd, "KxN", out_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        assert torch.equal(C, C2), kw


@pytest.mark.parametrize("name", ["sq256", "sq4096", "ragged", "sq8192_nt", "qkv_proj"])
def test_f32_operands_ternary_bit_exact(oracle_mod, name):
    """Entries in {-1, 0, 1}: every product and partial sum is an integer below
    2^24, so the fp32 output is exact at the workload shapes."""
    w = inputs.WORKLOADS[name]
    print(f"case f32-in ternary {name}", flush=True)
    A = inputs.ternary_f16((w.M, w.K), 300 + w.seed).astype(np.float32)
    B = inputs.ternary_f16(w.b_shape, 301 + w.seed).astype(np.float32)
    C = tg.gemm(_d32(A), _d32(B), w.b_layout, out_dtype=torch.float32)
    got = _out_np(C)
    I, J = inputs.sample_points(w.M, w.N, 8192, 302 + w.seed)
    ref, _ = oracle_mod.gemm_ex(A, B, w.b_layout, "f32", I=I, J=J)
    assert np.array_equal(got[I, J].astype(np.float64), ref)
    g = got.astype(np.float64)
    assert np.all(g == np.round(g)) and np.abs(g).max() <= w.K


@pytest.mark.parametrize("name", ["sq4096", "ragged", "sq8192_nt", "qkv_proj"])
def test_f32_operands_workload_parity(oracle_mod, name):
    w = inputs.WORKLOADS[name]
    print(f"case f32-in workload {name}", flush=True)
    A, B = inputs.make_inputs(w, "f32")
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    Ad, Bd = _d32(A), _d32(B)
    rc = tg.tgemm_gemm(w.M, w.N, w.K, "f32", Ad.data_ptr(), w.K, Bd.data_ptr(), B.shape[1], w.b_layout, "f32",
                       C.data_ptr(), w.N, 1.0, None, "none", torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TGEMM_OK
    got = _out_np(C)
    I, J = inputs.sample_points(w.M, w.N, 8192, w.seed + 4000)
    res = _check(oracle_mod, A, B, w.b_layout, "f32", "f32", got, 1.0, None, "none", name, I, J)
    print(f"  {name}: {res['n']} checked, worst {res['worst']:.4f}", flush=True)


def test_f32_operands_one_accumulation_rounded_to_each_output_type():
    print("case f32-in rounding", flush=True)
    M, N, K = 700, 600, 264
    A, B = _d32(_f32((M, K), 93)), _d32(_f32((N, K), 94))
    _, b_dev = _bias(N, 95, True)
    for kw in (dict(), dict(alpha=-1.75, bias=b_dev, act="relu")):
        c32 = tg.gemm(A, B, "NxK", out_dtype=torch.float32, **kw)
        c16 = tg.gemm(A, B, "NxK", out_dtype=torch.float16, **kw)
        cbf = tg.gemm(A, B, "NxK", out_dtype=torch.bfloat16, **kw)
        torch.cuda.synchronize()
        h32 = c32.cpu()
        assert torch.equal(h32.to(torch.float16).view(torch.int16), c16.cpu().view(torch.int16))
        assert torch.equal(h32.to(torch.bfloat16).view(torch.int16), cbf.cpu().view(torch.int16))


def test_f32_operands_k_zero_and_raster():
    print("case f32-in K=0 and raster", flush=True)
    A = torch.empty((300, 0), dtype=torch.float32, device=DEV)
    B = torch.empty((0, 270), dtype=torch.float32, device=DEV)
    C = torch.full((300, 270), 7.0, dtype=torch.float32, device=DEV)
    tg.gemm(A, B, "KxN", out=C)
    torch.cuda.synchronize()
    assert bool((C == 0).all())
    A = _d32(_f32((1300, 700), 96))
    B = _d32(_f32((1500, 700), 97))
    base = tg.gemm(A, B, "NxK", out_dtype=torch.float32)
    other = tg.gemm(A, B, "NxK", out_dtype=torch.float32, group_m=3, num_xcd=1)
    torch.cuda.synchronize()
    assert torch.equal(base, other)


@pytest.mark.parametrize("ct,ldc", [("f16", 17_000_000), ("f32", 4_400_000), ("f16", 8_000_000)])
def test_c_row_stride_beyond_buffer_offsets(oracle_mod, ct, ldc):
    """16-byte C stores use 32-bit offsets within a wave's 128 rows; a C whose
    row stride puts those offsets past 2^31 takes the 8-byte stores instead
    (ldc 17e6 for binary16, 4.4e6 for fp32), one just below keeps them
    (8e6). Two rows only, so the allocation stays small."""
    M, N, K = 2, 300, 96
    print(f"case typed large ldc {ct} {ldc}", flush=True)
    A = _bits((M, K), 81, "bf16")
    B = _bits((K, N), 82, "bf16")
    total = (M - 1) * ldc + N
    C = torch.full((total,), float("nan"), dtype=TORCH_DT[ct], device=DEV)
    Ad, Bd = _dev(A, "bf16"), _dev(B, "bf16")          # kept alive until the launch has run
    rc = tg.tgemm_gemm(M, N, K, "bf16", Ad.data_ptr(), K, Bd.data_ptr(), N, "KxN", ct,
                       C.data_ptr(), ldc, 1.0, None, "none", torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TGEMM_OK
    torch.cuda.synchronize()
    rows = torch.stack([C[0:N], C[ldc:ldc + N]])
    got = _out_np(rows.contiguous())
    _check(oracle_mod, A, B, "KxN", "bf16", ct, got, 1.0, None, "none", f"ldc {ldc}")
    gap = C[N:ldc]                                      # the padding between the two rows is untouched
    assert bool(torch.isnan(gap.float()).all())


def test_graph_capture_replays_match_eager():
    """One launch per call, no allocation, no synchronization: the typed entry
    point can be captured in a HIP graph. Each replay (with new operands copied
    into the captured buffers, and eager work between replays) equals the eager
    result bit for bit."""
    print("case typed graph capture", flush=True)
    M, N, K = 1000, 900, 700
    A = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    bias = torch.from_numpy(inputs.random_bias(N, 90)).to(DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    A.copy_(_dev(_bits((M, K), 91, "bf16"), "bf16"))
    B.copy_(_dev(_bits((N, K), 92, "bf16"), "bf16"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm-up outside the graph
        tg.gemm(A, B, "NxK", out=C, alpha=0.5, bias=bias, act="relu")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tg.gemm(A, B, "NxK", out=C, alpha=0.5, bias=bias, act="relu")
    for rep in range(4):
        A.copy_(_dev(_bits((M, K), 100 + rep, "bf16"), "bf16"))
        B.copy_(_dev(_bits((N, K), 200 + rep, "bf16"), "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = C.clone()
        eager = tg.gemm(A, B, "NxK", out_dtype=torch.float32, alpha=0.5, bias=bias, act="relu")
        torch.cuda.synchronize()
        assert torch.equal(got, eager), rep


def test_concurrent_streams():
    """Two products in flight on two streams, each equal to its lone result."""
    print("case typed two streams", flush=True)
    A1, B1 = _dev(_bits((2048, 1024), 301, "f16"), "f16"), _dev(_bits((3072, 1024), 302, "f16"), "f16")
    A2, B2 = _dev(_bits((1536, 2048), 303, "bf16"), "bf16"), _dev(_bits((2048, 2560), 304, "bf16"), "bf16")
    ref1 = tg.gemm(A1, B1, "NxK")
    ref2 = tg.gemm(A2, B2, "KxN", out_dtype=torch.float32)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            c1 = tg.gemm(A1, B1, "NxK")
        with torch.cuda.stream(s2):
            c2 = tg.gemm(A2, B2, "KxN", out_dtype=torch.float32)
        outs.append((c1, c2))
    torch.cuda.synchronize()
    for c1, c2 in outs:
        assert torch.equal(c1.view(torch.int16), ref1.view(torch.int16))
        assert torch.equal(c2, ref2)


@pytest.mark.parametrize("ct", ["f16", "f32"])
@pytest.mark.parametrize("lay", ["NxK", "KxN"])
def test_c_placement_selects_store_policy_same_bits(oracle_mod, lay, ct):
    """The 16-byte C stores are streamed where C's base and row pitch are
    multiples of 128 bytes and use the default policy elsewhere: the same
    product stored at 128-byte-aligned rows, at 16-byte-aligned rows, at
    2-byte-aligned rows and at a base 64 bytes past a 128-byte boundary gives
    the same bits, matches the oracle, and leaves the NaN guard around C
    intact. The 256-row-tile launch and the automatic one both run."""
    M, N, K = 520, 1000, 200
    print(f"case store policy {lay} {ct}", flush=True)
    A = _bits((M, K), 91, "f16")
    B = _bits((K, N) if lay == "KxN" else (N, K), 92, "f16")
    Ad, Bd = _dev(A, "f16"), _dev(B, "f16")
    esz = 4 if ct == "f32" else 2
    ref, tol = oracle_mod.gemm_ex(A, B, lay, "f16")
    outs = []
    for ldc, off_bytes in ((1024, 0), (1000, 0), (1001, 0), (1024, 64)):
        for tile_m in (0, 256):
            n_el = (M + 1) * ldc + 64
            if ct == "f32":
                buf = torch.full((n_el,), float("nan"), dtype=torch.float32, device=DEV)
            else:
                buf = torch.full((n_el,), 0x7E01, dtype=torch.int32).to(torch.int16).to(DEV)
            off = off_bytes // esz
            rc = tg.tgemm_gemm_config(M, N, K, "f16", Ad.data_ptr(), K, Bd.data_ptr(), B.shape[1], lay, ct,
                                      buf.data_ptr() + off_bytes, ldc, 1.0, None, "none",
                                      torch.cuda.current_stream().cuda_stream, tile_m=tile_m)
            assert rc == tg.TGEMM_OK, (ldc, off_bytes, tile_m)
            host = _out_np(buf)
            idx = off + (np.arange(M)[:, None] * ldc + np.arange(N)[None, :])
            inside = np.zeros(host.shape, dtype=bool)
            inside[idx.ravel()] = True
            if ct == "f32":
                assert np.isnan(host[~inside]).all(), (ldc, off_bytes, tile_m)
            else:
                assert (host[~inside] == 0x7E01).all(), (ldc, off_bytes, tile_m)
            got = np.ascontiguousarray(host[idx])
            res = oracle_mod.check_ex(got, ct, ref, tol)
            assert res["nfail"] == 0, (ldc, off_bytes, tile_m, res)
            outs.append(got.view(np.uint32 if ct == "f32" else np.uint16))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
