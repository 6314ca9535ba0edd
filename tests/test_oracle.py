"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: an exact rational brute force,
numpy's own binary16 implementation, a closed form, or a worked example the
pages print (fixtures under tests/golden/).
"""
from fractions import Fraction

import numpy as np
import pytest

from conftest import read_golden
from dense_tiled_gemm_tgemm_amd import inputs


# ---------------------------------------------------------------- binary16 --

def test_decode_all_bit_patterns_match_numpy(oracle_mod):
    """Exact decode of all 65536 binary16 patterns equals numpy's float16->float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.half_to_double(bits)
    theirs = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_ulp16_matches_numpy_spacing(oracle_mod):
    """ulp16 equals numpy's float16 spacing at every finite binary16 value."""
    vals = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16)
    with np.errstate(over="ignore"):
        sp = np.abs(np.spacing(vals).astype(np.float64))
    # np.spacing at 65504 is inf (next value overflows); the oracle keeps 32 there
    for v, s in zip(vals[::37].astype(np.float64), sp[::37]):
        if np.isfinite(s):
            assert oracle_mod.ulp16(v) == s, v
            assert oracle_mod.ulp16(-v) == s, v
    assert oracle_mod.ulp16(65504.0) == 32.0
    # between binary16 values: spacing of the binade that holds them
    assert oracle_mod.ulp16(4099.0) == 4.0
    assert oracle_mod.ulp16(1.5e-7) == 2.0 ** -24


# ----------------------------------------------------- exact brute force --

def _exact(A16, B16, b_layout):
    """Exact rational sum and sum of |products|; binary16 values are dyadic."""
    A = [[Fraction(float(x)) for x in row] for row in A16.astype(np.float64)]
    Bm = B16.astype(np.float64)
    if b_layout == "NxK":
        Bm = Bm.T
    B = [[Fraction(float(x)) for x in row] for row in Bm]
    M, K = len(A), len(A[0]) if A else 0
    N = len(B[0]) if B else 0
    ref = [[sum((A[i][k] * B[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    ab = [[sum((abs(A[i][k] * B[k][j]) for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    return ref, ab


def _wide_f16(shape, seed):
    """binary16 values spanning subnormals to large normals, both signs, zeros."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 0x7C00, size=shape).astype(np.uint16)       # finite magnitudes
    bits |= (rng.integers(0, 2, size=shape).astype(np.uint16) << 15)   # random sign
    return bits.view(np.float16)


@pytest.mark.parametrize("b_layout", ["KxN", "NxK"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 7, 5), (5, 1, 8)])
def test_brute_force_exact_rational(oracle_mod, M, N, K, b_layout):
    seed = M * 100 + N * 10 + K
    rng = np.random.default_rng(seed)
    # moderate-range values (include subnormals) so sums do not overflow
    A = (rng.uniform(-2, 2, (M, K)) * np.where(rng.random((M, K)) < 0.2, 2.0 ** -20, 1.0)).astype(np.float16)
    Bshape = (K, N) if b_layout == "KxN" else (N, K)
    B = rng.uniform(-2, 2, Bshape).astype(np.float16)
    ref, ab = oracle_mod.gemm(A, B, b_layout)
    eref, eab = _exact(A, B, b_layout)
    for i in range(M):
        for j in range(N):
            bound = K * 2.0 ** -53 * float(eab[i][j])
            assert abs(Fraction(ref[i, j]) - eref[i][j]) <= Fraction(bound), (i, j)
            assert abs(Fraction(ab[i, j]) - eab[i][j]) <= Fraction(bound), (i, j)


def test_brute_force_wide_exponents(oracle_mod):
    """Wide binary16 exponent range, strided operands: fp64 error stays within K*2^-53*sum|p|."""
    M, N, K = 4, 6, 8
    Afull = _wide_f16((M, K + 3), 11) * np.float16(2.0 ** -8)
    Bfull = _wide_f16((K, N + 5), 12) * np.float16(2.0 ** -8)
    A, B = Afull[:, :K], Bfull[:, :N]          # row strides K+3 and N+5
    ref, ab = oracle_mod.gemm(A, B, "KxN")
    eref, eab = _exact(np.ascontiguousarray(A), np.ascontiguousarray(B), "KxN")
    for i in range(M):
        for j in range(N):
            bound = K * 2.0 ** -53 * float(eab[i][j])
            assert abs(Fraction(ref[i, j]) - eref[i][j]) <= Fraction(bound)


def test_points_equal_full(oracle_mod):
    A = inputs.random_f16((37, 29), 5)
    B = inputs.random_f16((41, 29), 6)
    ref, ab = oracle_mod.gemm(A, B, "NxK")
    I = np.array([0, 36, 5, 17, 36], dtype=np.int64)
    J = np.array([0, 40, 13, 2, 0], dtype=np.int64)
    r2, a2 = oracle_mod.gemm_points(A, B, "NxK", I, J)
    assert np.array_equal(r2, ref[I, J]) and np.array_equal(a2, ab[I, J])


def test_layouts_agree_on_transposed_storage(oracle_mod):
    """B stored K x N and the same B stored N x K give the same product."""
    A = inputs.random_f16((9, 13), 7)
    B = inputs.random_f16((13, 11), 8)
    r1, a1 = oracle_mod.gemm(A, B, "KxN")
    r2, a2 = oracle_mod.gemm(A, np.ascontiguousarray(B.T), "NxK")
    assert np.array_equal(r1, r2) and np.array_equal(a1, a2)


# ------------------------------------------------------ printed example --

def test_page4_rowsum_example(oracle_mod):
    g = read_golden("rowsum_2x4.txt")
    A = np.array(g["A"], dtype=np.float16)
    B = np.array(g["B"], dtype=np.float16)
    C = np.array(g["C"], dtype=np.float64)
    ref, _ = oracle_mod.gemm(A, B, "KxN")
    assert np.array_equal(ref, C)


# ------------------------------------------------------------ closed forms --

@pytest.mark.parametrize("K", [1, 256, 4096, 4099, 8192])
def test_all_ones_gives_K(oracle_mod, K):
    A = np.ones((3, K), dtype=np.float16)
    B = np.ones((K, 5), dtype=np.float16)
    ref, ab = oracle_mod.gemm(A, B, "KxN")
    assert np.all(ref == K) and np.all(ab == K)


def test_all_ones_binary16_rounding_and_fp16_accumulation_discriminator(oracle_mod):
    """C = K rounds to the nearest binary16: 4099 -> 4100 (spacing 4 in [4096, 8192)).
    A kernel that accumulated in binary16 would stall at 2048 (2048 + 1 rounds back
    to 2048); the tolerance test must reject that output."""
    K = 4099
    A = np.ones((1, K), dtype=np.float16)
    B = np.ones((K, 1), dtype=np.float16)
    ref, ab = oracle_mod.gemm(A, B, "KxN")
    assert float(np.float16(ref[0, 0])) == 4100.0
    good = np.array([4100.0], dtype=np.float16)
    assert oracle_mod.check(good, ref, ab)["nfail"] == 0
    K = 4096
    ref, ab = oracle_mod.gemm(np.ones((1, K), np.float16), np.ones((K, 1), np.float16), "KxN")
    stalled = np.array([2048.0], dtype=np.float16)
    assert oracle_mod.check(stalled, ref, ab)["nfail"] == 1


@pytest.mark.parametrize("b_layout", ["KxN", "NxK"])
def test_identity_right_gives_A(oracle_mod, b_layout):
    A = inputs.random_f16((17, 24), 21)
    I = np.eye(24, dtype=np.float16)   # symmetric, same in both layouts
    ref, _ = oracle_mod.gemm(A, I, b_layout)
    assert np.array_equal(ref, A.astype(np.float64))


def test_identity_left_gives_B(oracle_mod):
    B = inputs.random_f16((24, 19), 22)
    ref, _ = oracle_mod.gemm(np.eye(24, dtype=np.float16), B, "KxN")
    assert np.array_equal(ref, B.astype(np.float64))
    ref2, _ = oracle_mod.gemm(np.eye(24, dtype=np.float16), np.ascontiguousarray(B.T), "NxK")
    assert np.array_equal(ref2, B.astype(np.float64))


def test_ternary_matches_integer_product(oracle_mod):
    """Entries in {-1,0,1}: every partial sum is an integer, so the fp64 sum is exact
    and equals numpy's int64 product."""
    A = inputs.ternary_f16((70, 333), 31)
    B = inputs.ternary_f16((333, 45), 32)
    ref, _ = oracle_mod.gemm(A, B, "KxN")
    exact = A.astype(np.int64) @ B.astype(np.int64)
    assert np.array_equal(ref, exact.astype(np.float64))


def test_K_zero_gives_zero(oracle_mod):
    ref, ab = oracle_mod.gemm(np.zeros((3, 0), np.float16), np.zeros((0, 4), np.float16), "KxN")
    assert ref.shape == (3, 4) and np.all(ref == 0) and np.all(ab == 0)


# ----------------------------------------------------- plausible mistakes --

def test_pins_catch_plausible_oracle_mistakes(oracle_mod):
    """Mistakes of the kind a buggy oracle could make change the brute-force
    answer: a transposed right operand, a dropped last k term, a sign flip."""
    M, N, K = 6, 6, 6
    A = inputs.random_f16((M, K), 41)
    B = inputs.random_f16((K, N), 42)
    eref, _ = _exact(A, B, "KxN")
    exact = np.array([[float(x) for x in r] for r in eref])
    ok, _ = oracle_mod.gemm(A, B, "KxN")
    assert np.allclose(ok, exact, rtol=0, atol=1e-12)
    transposed, _ = oracle_mod.gemm(A, B, "NxK")  # the K x N array read as N x K
    assert not np.allclose(transposed, exact, atol=1e-3)
    dropped, _ = oracle_mod.gemm(A[:, :K - 1], B[:K - 1], "KxN")
    assert not np.allclose(dropped, exact, atol=1e-3)
    flipped, _ = oracle_mod.gemm(A, -B, "KxN")
    assert not np.allclose(flipped, exact, atol=1e-3)


# ------------------------------------------------------------ tolerance --

def test_check_accepts_rounded_reference_and_rejects_errors(oracle_mod):
    A = inputs.random_f16((64, 128), 51)
    B = inputs.random_f16((128, 32), 52)
    ref, ab = oracle_mod.gemm(A, B, "KxN")
    good = ref.astype(np.float16)
    assert oracle_mod.check(good, ref, ab)["nfail"] == 0
    bad = good.copy()
    bad[3, 7] = np.float16(float(bad[3, 7]) + 0.01 * float(ab[3, 7]) + 1.0)
    bad[10, 0] = np.float16(np.nan)
    res = oracle_mod.check(bad, ref, ab)
    assert res["nfail"] == 2 and res["first_fail"] == [3 * 32 + 7, 10 * 32 + 0]


def test_check_tolerance_covers_fp32_any_order(oracle_mod):
    """fp32 sums of exact products in a shuffled order, rounded to binary16, pass."""
    rng = np.random.default_rng(61)
    A = inputs.random_f16((8, 4096), 62)
    B = inputs.random_f16((4096, 8), 63)
    ref, ab = oracle_mod.gemm(A, B, "KxN")
    out = np.empty((8, 8), dtype=np.float16)
    for i in range(8):
        for j in range(8):
            p = (A[i].astype(np.float32) * B[:, j].astype(np.float32))
            acc = np.float32(0)
            for v in p[rng.permutation(4096)]:
                acc = np.float32(acc + v)
            out[i, j] = np.float16(acc)
    assert oracle_mod.check(out, ref, ab)["nfail"] == 0


def test_sample_points_cover_tails():
    I, J = inputs.sample_points(3001, 5003, 4096, seed=7)
    assert set(range(2816, 3001)).issubset(set(I.tolist()))
    assert set(range(4864, 5003)).issubset(set(J.tolist()))
    assert I.max() < 3001 and J.max() < 5003 and len(I) >= 4096


def test_workload_registry_matches_stated_shapes():
    w = inputs.WORKLOADS
    assert (w["sq256"].M, w["sq256"].N, w["sq256"].K, w["sq256"].b_layout, w["sq256"].seed) == (256, 256, 256, "KxN", 0)
    assert (w["sq4096"].M, w["sq4096"].b_layout, w["sq4096"].seed) == (4096, "KxN", 1)
    assert (w["sq8192_nt"].M, w["sq8192_nt"].b_layout, w["sq8192_nt"].seed) == (8192, "NxK", 2)
    assert (w["ragged"].M, w["ragged"].N, w["ragged"].K, w["ragged"].seed) == (3001, 5003, 4099, 3)
    assert (w["qkv_proj"].M, w["qkv_proj"].N, w["qkv_proj"].K, w["qkv_proj"].b_layout) == (8192, 12288, 4096, "NxK")
    A, B = inputs.make_inputs(w["sq256"])
    assert A.shape == (256, 256) and B.shape == (256, 256) and A.dtype == np.float16
    assert np.abs(A.astype(np.float64)).max() <= 1.0
    A2, _ = inputs.make_inputs(w["sq256"])
    assert inputs.sha256(A) == inputs.sha256(A2)
