"""Pins of the extended oracle (bfloat16 inputs, binary16 / bfloat16 / binary32
outputs, scale, bias and rectifier on store) against facts that do not come
from the oracle: numpy's binary32 decoding, exact rational brute force,
closed forms and the plain fp16 oracle on the cases that reduce to it.
"""
from fractions import Fraction

import numpy as np
import pytest

from dense_tiled_gemm_tgemm_amd import inputs


# ------------------------------------------------------------ decoding --

def test_bf16_decode_all_bit_patterns_match_numpy_f32(oracle_mod):
    """bfloat16 is the upper half of a binary32: decoding all 65536 patterns
    equals numpy's decoding of the binary32 pattern with a zero lower half."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.bf16_to_double(bits)
    with np.errstate(invalid="ignore"):
        theirs = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_f32_decode_matches_numpy(oracle_mod):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x807fffff, 0x00800000, 0x7f7fffff, 0x7f800000, 0xff800000,
                        0x7fc00000, 0x3f800000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    ours = oracle_mod.f32_to_double(bits)
    with np.errstate(invalid="ignore"):
        theirs = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], theirs[~nan])


def test_ulp_type_matches_numpy_spacing(oracle_mod):
    """binary32: numpy's float32 spacing; bfloat16: 2^16 times the binary32
    spacing at bfloat16 normals, 2^-133 below them; binary16: as ulp16."""
    rng = np.random.default_rng(4)
    v32 = rng.integers(0, 0x7f7fffff, size=3000, dtype=np.int64).astype(np.uint32).view(np.float32)
    for v in v32[:1500]:
        s = float(np.spacing(v))
        assert oracle_mod.ulp_type(float(v), "f32") == s
        assert oracle_mod.ulp_type(-float(v), "f32") == s
    vb = oracle_mod.bf16_to_double(rng.integers(0x0080, 0x7f7f, size=1500).astype(np.uint16))
    for v in vb:
        assert oracle_mod.ulp_type(v, "bf16") == float(np.spacing(np.float32(v))) * 2.0 ** 16
    assert oracle_mod.ulp_type(1e-39, "bf16") == 2.0 ** -133
    assert oracle_mod.ulp_type(1e-39, "f32") == 2.0 ** -149
    for v in [0.0, 1e-6, 1.0, 3.0, 1000.0, 65504.0]:
        assert oracle_mod.ulp_type(v, "f16") == oracle_mod.ulp16(v)


# ----------------------------------------------------- exact brute force --

def _exact_ex(A, B, b_layout, decode, alpha, bias, act):
    """Exact rational act(alpha * sum + bias[j]) and |alpha| * sum|p| + |bias[j]|."""
    Ad = decode(A)
    Bd = decode(B)
    if b_layout == "NxK":
        Bd = Bd.T
    M, K = Ad.shape
    N = Bd.shape[1]
    fa = Fraction(float(alpha))
    out, mag = [], []
    for i in range(M):
        ro, rm = [], []
        for j in range(N):
            ps = [Fraction(float(Ad[i, k])) * Fraction(float(Bd[k, j])) for k in range(K)]
            bj = Fraction(float(bias[j])) if bias is not None else Fraction(0)
            v = fa * sum(ps, Fraction(0)) + bj
            if act == "relu" and v < 0:
                v = Fraction(0)
            ro.append(v)
            rm.append(abs(fa) * sum((abs(p) for p in ps), Fraction(0)) + abs(bj))
        out.append(ro)
        mag.append(rm)
    return out, mag


@pytest.mark.parametrize("b_layout", ["KxN", "NxK"])
@pytest.mark.parametrize("act", ["none", "relu"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (6, 4, 9), (5, 8, 3)])
def test_bf16_brute_force_with_epilogue(oracle_mod, M, N, K, b_layout, act):
    """bfloat16 operands over a wide exponent range, a non-unit scale and a
    per-column bias with M != N: a transposed operand, a dropped k term, a
    bias indexed by row, a scale applied to the bias or a rectifier applied
    before the bias all change this exact answer."""
    seed = 1000 + M * 100 + N * 10 + K
    rng = np.random.default_rng(seed)
    A = inputs.to_bf16_bits(rng.uniform(-2, 2, (M, K)) * 2.0 ** rng.integers(-30, 30, (M, K)))
    Bshape = (K, N) if b_layout == "KxN" else (N, K)
    B = inputs.to_bf16_bits(rng.uniform(-2, 2, Bshape) * 2.0 ** rng.integers(-30, 30, Bshape))
    bias = inputs.random_bias(N, seed, scale=4.0)
    alpha = -0.75
    ref, mag = oracle_mod.gemm_ex(A, B, b_layout, "bf16", alpha, bias, act)
    eref, emag = _exact_ex(A, B, b_layout, oracle_mod.bf16_to_double, alpha, bias, act)
    for i in range(M):
        for j in range(N):
            bound = Fraction((K + 2) * 2.0 ** -52) * emag[i][j]
            assert abs(Fraction(ref[i, j]) - eref[i][j]) <= bound, (i, j)
            assert abs(Fraction(mag[i, j]) - emag[i][j]) <= bound, (i, j)


def test_f16_brute_force_with_epilogue(oracle_mod):
    M, N, K = 4, 7, 6
    rng = np.random.default_rng(77)
    A = rng.uniform(-3, 3, (M, K)).astype(np.float16)
    B = rng.uniform(-3, 3, (K, N)).astype(np.float16)
    bias = inputs.random_bias(N, 78, scale=3.0)
    ref, mag = oracle_mod.gemm_ex(A, B, "KxN", "f16", 1.5, bias, "relu")
    eref, emag = _exact_ex(A.view(np.uint16), B.view(np.uint16), "KxN", oracle_mod.half_to_double, 1.5, bias,
                           "relu")
    for i in range(M):
        for j in range(N):
            bound = Fraction((K + 2) * 2.0 ** -52) * emag[i][j]
            assert abs(Fraction(ref[i, j]) - eref[i][j]) <= bound
    assert (ref == 0).any() and (ref > 0).any()          # the rectifier acted on some elements


def test_plausible_epilogue_mistakes_are_caught(oracle_mod):
    """Mistakes an epilogue could make change the brute-force answer: bias by
    row instead of column, scale applied to the bias, rectifier before the bias."""
    M, N, K = 3, 5, 4
    rng = np.random.default_rng(91)
    A = inputs.to_bf16_bits(rng.uniform(-1, 1, (M, K)))
    B = inputs.to_bf16_bits(rng.uniform(-1, 1, (K, N)))
    bias = np.array([0.5, -1.25, 2.0, -0.375, 1.0], dtype=np.float32)
    alpha = 2.0
    ref, _ = oracle_mod.gemm_ex(A, B, "KxN", "bf16", alpha, bias, "relu")
    s, _ = oracle_mod.gemm_ex(A, B, "KxN", "bf16")
    by_row = np.maximum(alpha * s + bias[:M, None].astype(np.float64), 0)
    scaled_bias = np.maximum(alpha * (s + bias.astype(np.float64)), 0)
    relu_first = np.maximum(alpha * s, 0) + bias.astype(np.float64)
    right = np.maximum(alpha * s + bias.astype(np.float64), 0)
    assert np.allclose(ref, right, rtol=0, atol=1e-12)
    for wrong in (by_row, scaled_bias, relu_first):
        assert not np.allclose(ref, wrong, atol=1e-3)


# ----------------------------------------------- reductions to the f16 oracle --

@pytest.mark.parametrize("b_layout", ["KxN", "NxK"])
def test_plain_case_equals_f16_oracle(oracle_mod, b_layout):
    """ab_type binary16, scale 1, no bias, no rectifier is the plain product."""
    A = inputs.random_f16((23, 41), 5)
    B = inputs.random_f16((41, 19) if b_layout == "KxN" else (19, 41), 6)
    r1, a1 = oracle_mod.gemm(A, B, b_layout)
    r2, a2 = oracle_mod.gemm_ex(A, B, b_layout, "f16")
    assert np.array_equal(r1, r2) and np.array_equal(a1, a2)
    I = np.array([0, 22, 7], dtype=np.int64)
    J = np.array([18, 0, 7], dtype=np.int64)
    r3, a3 = oracle_mod.gemm_ex(A, B, b_layout, "f16", I=I, J=J)
    assert np.array_equal(r3, r1[I, J]) and np.array_equal(a3, a1[I, J])


def test_bf16_values_equal_in_f16_give_the_f16_product(oracle_mod):
    """Small integers are exact in both formats: the bfloat16 product of their
    bfloat16 encodings equals the binary16 product of their binary16 ones."""
    rng = np.random.default_rng(8)
    Ai = rng.integers(-8, 9, (9, 30))
    Bi = rng.integers(-8, 9, (30, 11))
    r16, _ = oracle_mod.gemm(Ai.astype(np.float16), Bi.astype(np.float16), "KxN")
    rbf, _ = oracle_mod.gemm_ex(inputs.to_bf16_bits(Ai), inputs.to_bf16_bits(Bi), "KxN", "bf16")
    assert np.array_equal(r16, rbf)
    assert np.array_equal(rbf, (Ai @ Bi).astype(np.float64))


# ------------------------------------------------------------ closed forms --

def test_K_zero_gives_rectified_bias(oracle_mod):
    bias = np.array([-2.0, 0.0, 3.5, -0.25], dtype=np.float32)
    A = np.zeros((3, 0), dtype=np.uint16)
    B = np.zeros((0, 4), dtype=np.uint16)
    r, m = oracle_mod.gemm_ex(A, B, "KxN", "bf16", 3.0, bias, "none")
    assert np.array_equal(r, np.tile(bias.astype(np.float64), (3, 1)))
    assert np.array_equal(m, np.tile(np.abs(bias).astype(np.float64), (3, 1)))
    r, _ = oracle_mod.gemm_ex(A, B, "KxN", "bf16", 3.0, bias, "relu")
    assert np.array_equal(r, np.tile(np.maximum(bias, 0).astype(np.float64), (3, 1)))


def test_power_of_two_scale_of_integer_product(oracle_mod):
    """Ternary operands: the sum is an integer; a power-of-two scale and an
    integer bias keep it exact."""
    A = inputs.ternary_f16((20, 300), 31)
    B = inputs.ternary_f16((300, 13), 32)
    bias = np.arange(13, dtype=np.float32) - 6
    r, _ = oracle_mod.gemm_ex(A, B, "KxN", "f16", 0.125, bias, "relu")
    exact = np.maximum((A.astype(np.int64) @ B.astype(np.int64)) * 0.125 + bias, 0)
    assert np.array_equal(r, exact)


def test_bad_arguments_rejected(oracle_mod):
    A = np.zeros((2, 3), np.uint16)
    B = np.zeros((3, 2), np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.gemm_ex(A, B, "KxN", "f16", bias=np.zeros(3, np.float32))
    with pytest.raises(ValueError):
        oracle_mod.gemm_ex(A, B, "KxN", "f16", I=np.array([2]), J=np.array([0]))


# ------------------------------------------------------------ tolerance --

def test_check_f32_output_accepts_fp32_sums_any_order(oracle_mod):
    """fp32 sums of exact products in a shuffled order, scaled and biased in
    fp32, pass the binary32-output check; a 1% error fails it."""
    rng = np.random.default_rng(61)
    A = inputs.random_f16((6, 2048), 62)
    B = inputs.random_f16((2048, 6), 63)
    bias = inputs.random_bias(6, 64)
    alpha = 0.7
    ref, mag = oracle_mod.gemm_ex(A, B, "KxN", "f16", alpha, bias, "none")
    out = np.empty((6, 6), dtype=np.float32)
    for i in range(6):
        for j in range(6):
            p = A[i].astype(np.float32) * B[:, j].astype(np.float32)
            acc = np.float32(0)
            for v in p[rng.permutation(2048)]:
                acc = np.float32(acc + v)
            out[i, j] = np.float32(np.float32(alpha) * acc + bias[j])
    assert oracle_mod.check_ex(out, "f32", ref, mag)["nfail"] == 0
    bad = out.copy()
    bad[2, 3] = np.float32(bad[2, 3] + 0.01 * mag[2, 3] + 1e-3)
    res = oracle_mod.check_ex(bad, "f32", ref, mag)
    assert res["nfail"] == 1 and res["first_fail"] == [2 * 6 + 3]


def test_check_bf16_output_rounding(oracle_mod):
    """A bfloat16 output rounded from the reference passes; one 4 ulps off
    (where the sum term is negligible) fails; NaN fails."""
    ref = np.array([1.0, 3.0e5, -7.5e-3, 1.2e-39, 0.0])
    mag = np.zeros_like(ref)
    good = inputs.to_bf16_bits(ref)
    assert oracle_mod.check_ex(good, "bf16", ref, mag)["nfail"] == 0
    bad = good.copy()
    bad[1] += 4
    bad[4] = 0x7FC0
    res = oracle_mod.check_ex(bad, "bf16", ref, mag)
    assert res["nfail"] == 2 and res["first_fail"] == [1, 4]


def test_check_overflow_to_infinity(oracle_mod):
    """A reference past binary16's range must be stored as the infinity of
    its sign; a finite value there fails."""
    ref = np.array([70000.0, -70000.0, 65519.0])
    mag = np.zeros_like(ref)
    got = np.array([np.inf, -np.inf, 65504.0], dtype=np.float16)
    assert oracle_mod.check_ex(got, "f16", ref, mag)["nfail"] == 0
    got2 = np.array([65504.0, np.inf, 65504.0], dtype=np.float16)
    assert oracle_mod.check_ex(got2, "f16", ref, mag)["nfail"] == 2


def test_bf16_input_rounding_is_nearest_even():
    """The input generator's binary32 -> bfloat16 step: ties go to the even
    pattern, values between round to the nearer one."""
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.0 - 2.0 ** -7])
    assert [int(v) for v in inputs.to_bf16_bits(x)] == [0x3F80, 0x3F82, 0x3F81, 0xC000]


# ------------------------------------------------------------ binary32 inputs --

@pytest.mark.parametrize("b_layout", ["KxN", "NxK"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (6, 4, 9)])
def test_f32_inputs_brute_force_with_epilogue(oracle_mod, M, N, K, b_layout):
    """binary32 operands over a wide exponent range: exact rational answer."""
    seed = 2000 + M * 100 + N * 10 + K
    rng = np.random.default_rng(seed)
    A = (rng.uniform(-2, 2, (M, K)) * 2.0 ** rng.integers(-40, 40, (M, K))).astype(np.float32)
    Bshape = (K, N) if b_layout == "KxN" else (N, K)
    B = (rng.uniform(-2, 2, Bshape) * 2.0 ** rng.integers(-40, 40, Bshape)).astype(np.float32)
    bias = inputs.random_bias(N, seed, scale=4.0)
    ref, mag = oracle_mod.gemm_ex(A, B, b_layout, "f32", 1.25, bias, "relu")
    eref, emag = _exact_ex(A.view(np.uint32), B.view(np.uint32), b_layout, oracle_mod.f32_to_double, 1.25, bias,
                           "relu")
    for i in range(M):
        for j in range(N):
            bound = Fraction((K + 2) * 2.0 ** -52) * emag[i][j]
            assert abs(Fraction(ref[i, j]) - eref[i][j]) <= bound, (i, j)


def test_f32_inputs_reduce_to_f16_product(oracle_mod):
    """binary16 values widened to binary32 give the binary16 product exactly."""
    A = inputs.random_f16((13, 50), 81)
    B = inputs.random_f16((19, 50), 82)
    r16, a16 = oracle_mod.gemm(A, B, "NxK")
    r32, a32 = oracle_mod.gemm_ex(A.astype(np.float32), B.astype(np.float32), "NxK", "f32")
    assert np.array_equal(r16, r32) and np.array_equal(a16, a32)
