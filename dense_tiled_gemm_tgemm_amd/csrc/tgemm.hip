// Host entry points of the dense tiled GEMM for MI355X (gfx950): argument
// checks and planning (tgemm_plan.h), kernel choice among the instantiated
// combinations of element types and epilogue, and the launch. The kernels and
// their design are in tgemm_kernels.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tgemm.h"
#include "tgemm_kernels.h"
#include "tgemm_plan.h"

namespace tg {

static const void* pick_kernel(const Plan& pl) {
    const int ab = pl.ab_type, ct = pl.c_type;
    const bool e = pl.epi;
#define TG_PICK(a, c) \
    if (ab == a && ct == c) return e ? kernel_for<a, c, true>(pl) : kernel_for<a, c, false>(pl);
    TG_PICK(0, 0)
    TG_PICK(0, 1)
    TG_PICK(0, 2)
    TG_PICK(1, 0)
    TG_PICK(1, 1)
    TG_PICK(1, 2)
#undef TG_PICK
    return nullptr;
}

static thread_local int g_last_hip_error = 0;

// The direct-to-LDS kernel with 64-deep steps runs one workgroup per compute
// unit when a workgroup has at least two steps per tile (the cross-tile load
// stream reaches at most one tile ahead).
static bool persistent(const Plan& pl) {
    return (pl.variant & kDma) && pl.k_step == 64 && pl.K >= 2 * 64;
}

// Compute units of the current device (cached per device), or -hipError_t.
static int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return -(int)e;
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return -(int)e;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

static bool epilogue_requested(float alpha, const float* bias, int act) {
    return !(alpha == 1.0f) || bias != nullptr || act != TGEMM_ACT_NONE;
}

static int plan_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda, const void* B,
                     int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc, float alpha, const float* bias,
                     int act, int force_generic, int group_m, int num_xcd, int k_step, int stages, Plan* pl,
                     const void** fn) {
    if (act != TGEMM_ACT_NONE && act != TGEMM_ACT_RELU) return TGEMM_ERR_INVALID;
    const int rc = make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, force_generic, group_m, num_xcd, k_step,
                             stages, pl, ab_type, c_type, bias, epilogue_requested(alpha, bias, act));
    if (rc != TGEMM_OK) return rc;
    *fn = pick_kernel(*pl);
    return *fn ? TGEMM_OK : TGEMM_ERR_UNSUPPORTED;
}

}  // namespace tg

extern "C" int tgemm_gemm_config(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc,
                                 float alpha, const float* bias, int act, void* stream, int force_generic,
                                 int group_m, int num_xcd, int k_step, int stages) {
    tg::Plan pl;
    const void* fn = nullptr;
    const int rc = tg::plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act,
                                 force_generic, group_m, num_xcd, k_step, stages, &pl, &fn);
    if (rc != TGEMM_OK) return rc;
    if (pl.M == 0 || pl.N == 0) return TGEMM_OK;
    const int c_size = c_type == TGEMM_F32 ? 4 : 2;
    tg::Args args;
    args.A = static_cast<const uint16_t*>(A);
    args.B = static_cast<const uint16_t*>(B);
    args.C = C;
    args.bias = bias;
    args.alpha = alpha;
    args.relu = act == TGEMM_ACT_RELU;
    args.lda = pl.lda;
    args.ldb = pl.ldb;
    args.ldc = pl.ldc;
    args.M = pl.M;
    args.N = pl.N;
    args.K = pl.K;
    args.grid_m = pl.grid_m;
    args.grid_n = pl.grid_n;
    args.W = pl.W;
    args.group_m = pl.group_m;
    args.num_xcd = pl.num_xcd;
    args.grid = pl.W;
    args.c16 = ((uintptr_t)C % 16 == 0) && ((pl.ldc * c_size) % 16 == 0);
    args.c8 = (pl.variant & tg::kVecC) != 0;
    if (tg::persistent(pl)) {
        // one workgroup per compute unit, each walking several tiles
        const int ncu = tg::compute_units();
        if (ncu < 0) {
            tg::g_last_hip_error = -ncu;
            return TGEMM_ERR_HIP;
        }
        if (ncu > 0 && ncu < pl.W) args.grid = ncu;
    }
    void* kargs[] = {&args};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)args.grid), dim3(tg::NTHREADS), kargs, 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        tg::g_last_hip_error = (int)e;
        return TGEMM_ERR_HIP;
    }
    return TGEMM_OK;
}

extern "C" int tgemm_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc, float alpha,
                          const float* bias, int act, void* stream) {
    return tgemm_gemm_config(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act, stream,
                             0, 0, 0, 0, 0);
}

extern "C" int tgemm_f16_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, int b_layout, void* C, int64_t ldc,
                                void* stream, int force_generic, int group_m, int num_xcd, int k_step,
                                int stages) {
    return tgemm_gemm_config(M, N, K, TGEMM_F16, A, lda, B, ldb, b_layout, TGEMM_F16, C, ldc, 1.0f, nullptr,
                             TGEMM_ACT_NONE, stream, force_generic, group_m, num_xcd, k_step, stages);
}

extern "C" int tgemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                         int64_t ldb, int b_layout, void* C, int64_t ldc, void* stream) {
    return tgemm_f16_config(M, N, K, A, lda, B, ldb, b_layout, C, ldc, stream, 0, 0, 0, 0, 0);
}

extern "C" const char* tgemm_status_string(int status) {
    switch (status) {
        case TGEMM_OK: return "ok";
        case TGEMM_ERR_INVALID: return "invalid argument";
        case TGEMM_ERR_UNSUPPORTED: return "unsupported problem size";
        case TGEMM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int tgemm_last_hip_error(void) { return tg::g_last_hip_error; }

static void fill_info(const tg::Plan& pl, int64_t* info) {
    info[0] = pl.variant;
    info[1] = tg::BM;
    info[2] = tg::BN;
    info[3] = pl.k_step;
    info[4] = (pl.M == 0 || pl.N == 0) ? 0 : pl.W;
    info[5] = pl.group_m;
    info[6] = pl.num_xcd;
    info[7] = tg::NTHREADS;
    info[8] = pl.stages;
    info[9] = (int64_t)pl.stages * 2 * 256 * pl.k_step * 2;   // LDS bytes per workgroup
}

extern "C" int tgemm_plan_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda,
                               const void* B, int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc,
                               float alpha, const float* bias, int act, int force_generic, int group_m,
                               int num_xcd, int k_step, int stages, int64_t* info) {
    if (!info) return TGEMM_ERR_INVALID;
    tg::Plan pl;
    const void* fn = nullptr;
    const int rc = tg::plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act,
                                 force_generic, group_m, num_xcd, k_step, stages, &pl, &fn);
    if (rc != TGEMM_OK) return rc;
    fill_info(pl, info);
    return TGEMM_OK;
}

extern "C" int tgemm_plan_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, int b_layout, void* C, int64_t ldc, int force_generic,
                              int group_m, int num_xcd, int k_step, int stages, int64_t* info) {
    return tgemm_plan_gemm(M, N, K, TGEMM_F16, A, lda, B, ldb, b_layout, TGEMM_F16, C, ldc, 1.0f, nullptr,
                           TGEMM_ACT_NONE, force_generic, group_m, num_xcd, k_step, stages, info);
}

extern "C" int tgemm_tile_of(int64_t grid_m, int64_t grid_n, int group_m, int num_xcd, int64_t wid,
                             int64_t* tile_m, int64_t* tile_n) {
    if (!tile_m || !tile_n || grid_m <= 0 || grid_n <= 0 || group_m <= 0 || num_xcd <= 0)
        return TGEMM_ERR_INVALID;
    if (grid_m > 2147483647 || grid_n > 2147483647 || grid_m * grid_n > 2147483647 || wid < 0 ||
        wid >= grid_m * grid_n)
        return TGEMM_ERR_INVALID;
    const int g = group_m > grid_m ? (int)grid_m : group_m;
    int tm, tn;
    tg::tile_of((int)wid, (int)(grid_m * grid_n), (int)grid_m, (int)grid_n, g, num_xcd, &tm, &tn);
    *tile_m = tm;
    *tile_n = tn;
    return TGEMM_OK;
}
