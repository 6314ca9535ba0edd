"""GPU tests of runtime tuning: the tuner records a launch choice per problem
key, later automatic calls use it (visible in the plan query), and the result
is the same bits as without tuning and within the oracle's tolerance."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import dense_tiled_gemm_tgemm_amd as tg  # noqa: E402
from dense_tiled_gemm_tgemm_amd import inputs  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _clean_table():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.tuning_clear()
    yield
    torch.cuda.synchronize()
    tg.tuning_clear()


def _dev16(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(dt)


def _plan(A, B, C, lay, ab, ct, **kw):
    M, K = A.shape
    N = C.shape[1]
    return tg.tgemm_plan_gemm(M, N, K, ab, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0), lay, ct,
                              C.data_ptr(), C.stride(0), **kw)


def test_tuned_choice_is_recorded_used_and_changes_no_bits():
    print("case tuning f16 NxK", flush=True)
    M, N, K = 2304, 5120, 1000          # 180 tiles of 256 rows: more than half the compute units
    A = _dev16(inputs.random_f16((M, K), 1).view(np.uint16), torch.float16)
    B = _dev16(inputs.random_f16((N, K), 2).view(np.uint16), torch.float16)
    base = tg.mm(A, B, "NxK")
    C = torch.empty_like(base)
    rc0, plan0 = _plan(A, B, C, "NxK", "f16", "f16")
    assert rc0 == 0 and (plan0["bk"], plan0["stages"], plan0["group_m"]) == (64, 2, 4)
    C, chosen = tg.tune(A, B, "NxK", out=C, rounds=3)
    torch.cuda.synchronize()
    print(f"  chosen {chosen}", flush=True)
    assert torch.equal(C.view(torch.int16), base.view(torch.int16))
    assert tg.tuning_entries() == 1
    assert chosen["candidates"] == 30 and chosen["median_ns"] > 0     # 10 pipelines x 3 group heights
    assert (chosen["k_step"], chosen["stages"]) in {(64, 2), (32, 2), (32, 3), (32, 4), (32, 5)}
    # raster groups 4, 8 and 16 tile rows, each capped at the tile rows of M
    # (9 of 256 rows, 18 of 128, 36 of 64)
    assert chosen["group_m"] in (4, 8, 9, 16) and chosen["num_xcd"] == 8
    rc, plan = _plan(A, B, C, "NxK", "f16", "f16")
    assert (plan["bk"], plan["stages"], plan["group_m"], plan["num_xcd"], plan["bm"]) == \
        (chosen["k_step"], chosen["stages"], chosen["group_m"], chosen["num_xcd"], chosen["tile_m"])
    # another key (other types) is not affected
    C32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    rc, plan32 = _plan(A, B, C32, "NxK", "f16", "f32")
    assert (plan32["bk"], plan32["stages"], plan32["group_m"]) == (64, 2, 4)
    # the tuned automatic call gives the same bits
    again = tg.mm(A, B, "NxK")
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), base.view(torch.int16))
    tg.tuning_clear()
    rc, plan = _plan(A, B, C, "NxK", "f16", "f16")
    assert plan == plan0


def test_tuning_with_epilogue_and_bf16(oracle_mod):
    print("case tuning bf16 -> f32 epilogue", flush=True)
    M, N, K = 2600, 1300, 4099          # 11 tile rows: group heights 4, 8 and 11
    A = inputs.random_bf16((M, K), 3)
    B = inputs.random_bf16((K, N), 4)
    bias = inputs.random_bias(N, 5)
    Ad, Bd = _dev16(A, torch.bfloat16), _dev16(B, torch.bfloat16)
    bd = torch.from_numpy(bias).to(DEV)
    base = tg.gemm(Ad, Bd, "KxN", out_dtype=torch.float32, alpha=0.25, bias=bd, act="relu")
    C, chosen = tg.tune(Ad, Bd, "KxN", out_dtype=torch.float32, alpha=0.25, bias=bd, act="relu", rounds=3)
    torch.cuda.synchronize()
    print(f"  chosen {chosen}", flush=True)
    # bfloat16 -> fp32 with an epilogue builds the default ring depth of each K
    # step and of the 128- and 64-row tiles: 4 pipelines x 3 group heights
    assert chosen["candidates"] == 12
    assert (chosen["k_step"], chosen["stages"], chosen["tile_m"]) in {(64, 2, 256), (32, 4, 256), (32, 3, 128),
                                                                      (32, 3, 64)}
    assert chosen["producers"] == 0
    assert torch.equal(C, base)
    got = tg.gemm(Ad, Bd, "KxN", out_dtype=torch.float32, alpha=0.25, bias=bd, act="relu").cpu().numpy()
    I, J = inputs.sample_points(M, N, 4096, 6)
    ref, tol = oracle_mod.gemm_ex(A, B, "KxN", "bf16", 0.25, bias, "relu", I=I, J=J)
    res = oracle_mod.check_ex(got[I, J], "f32", ref, tol)
    assert res["nfail"] == 0, res
    assert np.array_equal(got, base.cpu().numpy())


@pytest.mark.parametrize("lay,K,tiles_m,ab,want", [
    ("KxN", 1000, 4, "f16", (32, 4)),     # B K x N, K % 64 != 0, one round: 32-deep default ring
    ("KxN", 1000, 4, "bf16", (32, 4)),
    ("KxN", 1024, 4, "f16", (64, 2)),     # K a multiple of 64
    ("NxK", 1000, 4, "f16", (64, 2)),     # B stored N x K
    ("KxN", 1000, 40, "f16", (64, 2)),    # more tiles than compute units: persistent 64-deep
])
def test_automatic_pipeline_choice(lay, K, tiles_m, ab, want):
    """With every launch choice automatic, B stored K x N with a partial last
    64-deep step on a grid of one round or less runs 32-deep steps; the other
    cases keep the 64-deep ring. Same bits either way."""
    print(f"case automatic pipeline {lay} K={K} tiles_m={tiles_m} {ab}", flush=True)
    M, N = 256 * tiles_m, 16384      # 64 tile columns: more than half of the compute units
    dt = torch.float16 if ab == "f16" else torch.bfloat16
    gen = inputs.random_f16 if ab == "f16" else inputs.random_bf16
    A = _dev16(gen((M, K), 7).view(np.uint16), dt)
    B = _dev16(gen((K, N) if lay == "KxN" else (N, K), 8).view(np.uint16), dt)
    C = torch.empty((M, N), dtype=dt, device=DEV)
    tg.tuning_clear()
    rc, plan = _plan(A, B, C, lay, ab, ab)
    assert rc == 0 and (plan["bk"], plan["stages"]) == want, plan
    auto = tg.gemm(A, B, lay)
    other = tg.gemm(A, B, lay, k_step=64 if want[0] == 32 else 32)
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int16), other.view(torch.int16))


@pytest.mark.parametrize("lay,cands", [("NxK", 12), ("KxN", 12)])
def test_tuning_binary32_operands(oracle_mod, lay, cands):
    """Binary32 operands (either B layout): the tuner tries the direct-to-LDS
    kernel's ring depths (2, 3 at 256 rows) and its 128- and 64-row tiles
    (4 pipelines x 3 group heights). The recorded choice (K step 16 floats)
    is used by later automatic calls and changes no bits."""
    print(f"case tuning f32 {lay}", flush=True)
    M, N, K = 3584, 4096, 1000          # 14 x 16 tiles of 256 x 256
    A = inputs.random_f32((M, K), 11)
    B = inputs.random_f32((N, K) if lay == "NxK" else (K, N), 12)
    Ad = torch.from_numpy(A).to(DEV)
    Bd = torch.from_numpy(B).to(DEV)
    base = tg.gemm(Ad, Bd, lay, out_dtype=torch.float32)
    C, chosen = tg.tune(Ad, Bd, lay, out_dtype=torch.float32, rounds=3)
    torch.cuda.synchronize()
    print(f"  chosen {chosen}", flush=True)
    assert chosen["candidates"] == cands and chosen["k_step"] == 16
    assert (chosen["stages"], chosen["tile_m"]) in {(2, 256), (3, 256), (3, 128), (3, 64)}
    assert torch.equal(C, base)
    rc, plan = _plan(Ad, Bd, C, lay, "f32", "f32")
    assert rc == 0
    assert (plan["bk"], plan["stages"], plan["group_m"], plan["bm"]) == \
        (chosen["k_step"], chosen["stages"], chosen["group_m"], chosen["tile_m"])
    again = tg.gemm(Ad, Bd, lay, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(again, base)
    got = again.cpu().numpy()
    I, J = inputs.sample_points(M, N, 4096, 13)
    ref, tol = oracle_mod.gemm_ex(A, B, lay, "f32", I=I, J=J)
    res = oracle_mod.check_ex(got[I, J], "f32", ref, tol)
    assert res["nfail"] == 0, res
