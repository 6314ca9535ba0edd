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
