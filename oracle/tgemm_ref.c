/*
 * CPU oracle for the fp16 dense matrix product C = A*B.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the independent checker of the GPU
 * path. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it. The product library never links, includes or calls it, and
 * it shares no code, header or table with the GPU kernels.
 *
 * What it computes (page 1, "Using NVIDIA CUDA Tile to write a
 * high-performance matrix multiply", section "What is matrix multiplication?"):
 * each output element is the dot product of a row of A (M x K) with a column
 * of B (K x N):  C[i][j] = sum over k of A[i][k] * B[k][j].
 *
 * The tiled kernels on the pages accumulate in fp32 and convert to the output
 * type only at the store (page 1, sections 4 and 6; page 4, section 2.4.9.1
 * "Matrix multiplication"), and fill partial K tiles with zeros, which adds
 * only 0*0 terms (page 4, section 2.4.9.1). A tiled result therefore differs
 * from the definition only by rounding, so the oracle is the definition
 * itself, evaluated in fp64:
 *   - every binary16 input is decoded exactly to a double from the IEEE 754
 *     binary16 field definition (no compiler half type is used);
 *   - each product of two binary16 values is exact in fp64 (two 11-bit
 *     significands give at most 22 bits);
 *   - the products are summed in ascending k in fp64, and the sum of their
 *     absolute values is kept alongside for the tolerance.
 *
 * Tolerance (ref_check_f16): a GPU output g passes when
 *   |g - ref| <= rel * sum_k |A[i][k] B[k][j]| + ulp16(ref),
 * with rel = 1e-3 by default. Any order of fp32 summation of exact products
 * errs by at most about (K-1) * 2^-24 * sum|p| (the standard recursive
 * summation bound), which is below 1e-3 * sum|p| for every K <= 16777; the
 * final round-to-nearest into binary16 adds at most half a binary16 ulp.
 *
 * The second half of this file extends the same definition to bfloat16
 * inputs, binary16 / bfloat16 / binary32 outputs and a scale, bias and
 * rectifier applied to each sum before it is stored (ref_gemm_ex).
 *
 * Parallelism: OpenMP over output elements only. Each element's k order stays
 * sequential, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: sign s (1 bit), biased exponent e (5 bits), fraction f
 * (10 bits). e == 0: subnormal or zero, value f * 2^-24. 0 < e < 31: normal,
 * value (1024 + f) * 2^(e - 25). e == 31: infinity (f == 0) or NaN. */
double ref_half_to_double(uint16_t h) {
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e < 31) {
        v = ldexp((double)(1024 + f), e - 25);
    } else {
        v = (f == 0) ? INFINITY : NAN;
    }
    return s ? -v : v;
}

void ref_decode_f16(int64_t n, const uint16_t* src, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = ref_half_to_double(src[i]);
}

/* Spacing of binary16 numbers at the magnitude of x: 2^-24 below the
 * smallest normal 2^-14, else 2^(floor(log2|x|) - 10). frexp gives
 * |x| = m * 2^e with m in [0.5, 1), so floor(log2|x|) = e - 1. Above the
 * largest finite binary16 (65504) the spacing of the top binade, 32, is
 * returned. */
double ref_ulp16(double x) {
    double a = fabs(x);
    if (!(a >= ldexp(1.0, -14))) return ldexp(1.0, -24); /* also NaN */
    if (a > 65504.0) return 32.0;
    int e;
    (void)frexp(a, &e);
    return ldexp(1.0, e - 11);
}

int ref_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Decode A (M rows of K, row stride lda) into a dense M x K double array. */
static double* decode_a(int64_t M, int64_t K, const uint16_t* A, int64_t lda) {
    double* a = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    if (!a) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) a[i * K + k] = ref_half_to_double(A[i * lda + k]);
    return a;
}

/* Decode B into a dense N x K double array bt, so that bt[j*K + k] = B[k][j]
 * for both storage layouts:
 *   b_layout 0 (K x N): element (k, j) is B[k*ldb + j];
 *   b_layout 1 (N x K): element (k, j) is B[j*ldb + k]. */
static double* decode_bt(int64_t N, int64_t K, const uint16_t* B, int64_t ldb, int b_layout) {
    double* bt = (double*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!bt) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k) {
            uint16_t h = (b_layout == 0) ? B[k * ldb + j] : B[j * ldb + k];
            bt[j * K + k] = ref_half_to_double(h);
        }
    return bt;
}

/*
 * Reference values for a set of output elements.
 *   npts < 0 : every element of the M x N output, in row-major order
 *              (index i*N + j of ref/absum);
 *   npts >= 0: the elements (I[p], J[p]) for p < npts.
 * ref[p]   = sum_k A[i][k] * B[k][j]   (fp64, ascending k)
 * absum[p] = sum_k |A[i][k] * B[k][j]|
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int ref_gemm_f16(int64_t M, int64_t N, int64_t K,
                 const uint16_t* A, int64_t lda,
                 const uint16_t* B, int64_t ldb, int b_layout,
                 int64_t npts, const int64_t* I, const int64_t* J,
                 double* ref, double* absum) {
    if (M < 0 || N < 0 || K < 0 || (b_layout != 0 && b_layout != 1)) return -1;
    if (npts > 0 && (!I || !J)) return -1;
    double* a = decode_a(M, K, A, lda);
    double* bt = decode_bt(N, K, B, ldb, b_layout);
    if (!a || !bt) {
        free(a);
        free(bt);
        return -1;
    }
    const int64_t n_out = (npts < 0) ? M * N : npts;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 256) reduction(| : bad)
    for (int64_t p = 0; p < n_out; ++p) {
        const int64_t i = (npts < 0) ? p / N : I[p];
        const int64_t j = (npts < 0) ? p % N : J[p];
        if (i < 0 || i >= M || j < 0 || j >= N) {
            bad = 1;
            continue;
        }
        const double* ar = a + i * K;
        const double* br = bt + j * K;
        double acc = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double prod = ar[k] * br[k];
            acc += prod;
            s += fabs(prod);
        }
        ref[p] = acc;
        absum[p] = s;
    }
    free(a);
    free(bt);
    return bad ? -1 : 0;
}

/*
 * Tolerance check of n GPU outputs (binary16 bit patterns) against the
 * oracle. An element passes when
 *   - ref is finite and g is finite and |g - ref| <= rel*absum + ulp16(ref), or
 *   - |ref| rounds past the binary16 range (|ref| >= 65520) and g is the
 *     infinity of the same sign, or
 *   - ref is NaN and g is NaN, or ref is an infinity and g equals it.
 * Returns the number of failing elements; *worst receives the largest
 * |g - ref| / (rel*absum + ulp16(ref)) over finite pairs; the indices of the
 * first max_report failures (in index order) go to first_fail.
 */
int64_t ref_check_f16(int64_t n, const uint16_t* got, const double* ref, const double* absum,
                      double rel, double* worst, int64_t* first_fail, int64_t max_report) {
    int64_t nfail = 0;
    double w = 0.0;
    for (int64_t p = 0; p < n; ++p) {
        const double g = ref_half_to_double(got[p]);
        const double r = ref[p];
        int ok;
        if (isnan(r)) {
            ok = isnan(g);
        } else if (isinf(r)) {
            ok = (g == r);
        } else if (fabs(r) >= 65520.0) {
            ok = isinf(g) && ((g > 0) == (r > 0));
        } else if (!isfinite(g)) {
            ok = 0;
        } else {
            const double tol = rel * absum[p] + ref_ulp16(r);
            const double ratio = fabs(g - r) / tol;
            if (ratio > w) w = ratio;
            ok = fabs(g - r) <= tol;
        }
        if (!ok) {
            if (nfail < max_report && first_fail) first_fail[nfail] = p;
            ++nfail;
        }
    }
    if (worst) *worst = w;
    return nfail;
}


/* ------------------------------------------------------------------------
 * Extended operation: other element types and a fused epilogue.
 *
 * Element types (the pages' tile kernels take the element type as a
 * parameter: page 1, section 6 and its launcher, which picks tiles for 2-byte
 * and 4-byte inputs; page 2, section 7; page 4, section 2.4.9.1 accumulates in
 * fp32 and stores an fp32 C):
 *   type 0: IEEE 754 binary16 (decoded by ref_half_to_double above);
 *   type 1: bfloat16, the upper half of a binary32: sign (1 bit), biased
 *           exponent e (8 bits), fraction f (7 bits). e == 0: f * 2^-133;
 *           0 < e < 255: (128 + f) * 2^(e - 134); e == 255: inf / NaN;
 *   type 2: IEEE 754 binary32: sign, e (8 bits), f (23 bits). e == 0:
 *           f * 2^-149; 0 < e < 255: (2^23 + f) * 2^(e - 150); e == 255:
 *           inf / NaN.
 * Products of two values of any one of these types are exact in fp64 (at
 * most 24 + 24 significant bits).
 *
 * Epilogue (the reading of "scale, bias and activation on store"):
 *   C[i][j] = act(alpha * sum_k A[i][k] B[k][j] + bias[j]),
 * act(x) = x, or max(x, 0) for the rectifier. bias may be absent (zero).
 * The tolerance magnitude returned alongside is
 *   |alpha| * sum_k |A[i][k] B[k][j]| + |bias[j]|,
 * which bounds the fp32 rounding of the scale and the bias add as it bounds
 * the sum; the rectifier does not increase any difference.
 * ---------------------------------------------------------------------- */

double ref_bf16_to_double(uint16_t b) {
    const int s = (b >> 15) & 1;
    const int e = (b >> 7) & 255;
    const int f = b & 127;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);
    } else if (e < 255) {
        v = ldexp((double)(128 + f), e - 134);
    } else {
        v = (f == 0) ? INFINITY : NAN;
    }
    return s ? -v : v;
}

double ref_f32_to_double(uint32_t w) {
    const int s = (int)((w >> 31) & 1u);
    const int e = (int)((w >> 23) & 255u);
    const uint32_t f = w & 0x7fffffu;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -149);
    } else if (e < 255) {
        v = ldexp((double)((1u << 23) + f), e - 150);
    } else {
        v = (f == 0) ? INFINITY : NAN;
    }
    return s ? -v : v;
}

static double decode_elem(uint16_t h, int type) {
    return type == 1 ? ref_bf16_to_double(h) : ref_half_to_double(h);
}

/* Spacing of the output type at |x| (below the smallest normal: the subnormal
 * step; above the largest finite value: the top binade's spacing). */
double ref_ulp_type(double x, int type) {
    const int frac_bits = (type == 0) ? 10 : (type == 1) ? 7 : 23;
    const int emin = (type == 0) ? -14 : -126;        /* smallest normal 2^emin */
    const double a = fabs(x);
    if (!(a >= ldexp(1.0, emin))) return ldexp(1.0, emin - frac_bits); /* also NaN */
    int e;
    (void)frexp(a, &e);
    const int emax = (type == 0) ? 15 : 127;
    if (e - 1 > emax) e = emax + 1;
    return ldexp(1.0, e - 1 - frac_bits);
}

/* Smallest magnitude that rounds to infinity in the output type. */
static double overflow_threshold(int type) {
    if (type == 0) return 65520.0;                               /* 65504 + 16 */
    if (type == 1) return ldexp(2.0 - ldexp(1.0, -8), 127);      /* max bf16 + half ulp */
    return ldexp(2.0 - ldexp(1.0, -24), 127);                    /* max f32 + half ulp */
}

/* Element p of an operand of the given type (16-bit patterns for types 0
 * and 1, 32-bit patterns for type 2). */
static double elem_at(const void* X, int64_t p, int type) {
    return type == 2 ? ref_f32_to_double(((const uint32_t*)X)[p]) : decode_elem(((const uint16_t*)X)[p], type);
}

static double* decode_a_t(int64_t M, int64_t K, const void* A, int64_t lda, int type) {
    double* a = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    if (!a) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) a[i * K + k] = elem_at(A, i * lda + k, type);
    return a;
}

static double* decode_bt_t(int64_t N, int64_t K, const void* B, int64_t ldb, int b_layout, int type) {
    double* bt = (double*)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!bt) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            bt[j * K + k] = elem_at(B, (b_layout == 0) ? k * ldb + j : j * ldb + k, type);
    return bt;
}

/*
 * Reference values of the extended operation at a set of output elements
 * (npts < 0: all, row-major; else (I[p], J[p])). ab_type: 0 binary16,
 * 1 bfloat16, 2 binary32 for both operands (strides in elements of that
 * type). bias: N floats or NULL. act: 0 none,
 * 1 rectifier. ref[p] and tol_mag[p] as described above. Returns 0, or -1
 * on bad arguments or allocation failure.
 */
int ref_gemm_ex(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda, const void* B, int64_t ldb, int b_layout, int ab_type,
                double alpha, const float* bias, int act,
                int64_t npts, const int64_t* I, const int64_t* J, double* ref, double* tol_mag) {
    if (M < 0 || N < 0 || K < 0 || (b_layout != 0 && b_layout != 1)) return -1;
    if (ab_type < 0 || ab_type > 2 || (act != 0 && act != 1)) return -1;
    if (npts > 0 && (!I || !J)) return -1;
    double* a = decode_a_t(M, K, A, lda, ab_type);
    double* bt = decode_bt_t(N, K, B, ldb, b_layout, ab_type);
    if (!a || !bt) {
        free(a);
        free(bt);
        return -1;
    }
    const int64_t n_out = (npts < 0) ? M * N : npts;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 256) reduction(| : bad)
    for (int64_t p = 0; p < n_out; ++p) {
        const int64_t i = (npts < 0) ? p / N : I[p];
        const int64_t j = (npts < 0) ? p % N : J[p];
        if (i < 0 || i >= M || j < 0 || j >= N) {
            bad = 1;
            continue;
        }
        const double* ar = a + i * K;
        const double* br = bt + j * K;
        double acc = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double prod = ar[k] * br[k];
            acc += prod;
            s += fabs(prod);
        }
        const double bj = bias ? (double)bias[j] : 0.0;
        double v = alpha * acc + bj;
        if (act == 1 && v < 0.0) v = 0.0;
        ref[p] = v;
        tol_mag[p] = fabs(alpha) * s + fabs(bj);
    }
    free(a);
    free(bt);
    return bad ? -1 : 0;
}

/*
 * Tolerance check of n GPU outputs of type c_type (0 binary16, 1 bfloat16:
 * got16 holds the bit patterns; 2 binary32: got32 does). An element passes
 * when ref and g are finite and |g - ref| <= rel * tol_mag + ulp(ref) in the
 * output type, or |ref| rounds past the type's range and g is the infinity
 * of the same sign, or ref is NaN and g is NaN, or ref is an infinity and g
 * equals it. Returns the failure count; *worst and first_fail as in
 * ref_check_f16.
 */
int64_t ref_check_ex(int64_t n, int c_type, const uint16_t* got16, const uint32_t* got32, const double* ref,
                     const double* tol_mag, double rel, double* worst, int64_t* first_fail, int64_t max_report) {
    if (c_type < 0 || c_type > 2 || (c_type < 2 && !got16) || (c_type == 2 && !got32)) return -1;
    const double ovf = overflow_threshold(c_type);
    int64_t nfail = 0;
    double w = 0.0;
    for (int64_t p = 0; p < n; ++p) {
        const double g = (c_type == 2) ? ref_f32_to_double(got32[p]) : decode_elem(got16[p], c_type);
        const double r = ref[p];
        int ok;
        if (isnan(r)) {
            ok = isnan(g);
        } else if (isinf(r)) {
            ok = (g == r);
        } else if (fabs(r) >= ovf) {
            ok = isinf(g) && ((g > 0) == (r > 0));
        } else if (!isfinite(g)) {
            ok = 0;
        } else {
            const double tol = rel * tol_mag[p] + ref_ulp_type(r, c_type);
            const double ratio = fabs(g - r) / tol;
            if (ratio > w) w = ratio;
            ok = fabs(g - r) <= tol;
        }
        if (!ok) {
            if (nfail < max_report && first_fail) first_fail[nfail] = p;
            ++nfail;
        }
    }
    if (worst) *worst = w;
    return nfail;
}

/* Array decoders for the checks: n bfloat16 / binary32 bit patterns -> double. */
void ref_decode_bf16(int64_t n, const uint16_t* src, double* dst) {
    for (int64_t p = 0; p < n; ++p) dst[p] = ref_bf16_to_double(src[p]);
}

void ref_decode_f32(int64_t n, const uint32_t* src, double* dst) {
    for (int64_t p = 0; p < n; ++p) dst[p] = ref_f32_to_double(src[p]);
}
