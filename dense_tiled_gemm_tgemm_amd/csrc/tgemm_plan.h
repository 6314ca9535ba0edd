// Host-side planning for the tiled GEMM: argument checks, variant choice,
// grid size, and the workgroup -> output-tile map shared with the kernels.
// Plain C++ apart from the host/device qualifiers on tile_of().
#pragma once

#include <stdint.h>

#include "tgemm.h"

#if defined(__HIPCC__)
#define TG_HD __host__ __device__
#else
#define TG_HD
#endif

namespace tg {

// Workgroup tile: BM x BN outputs, K walked BK at a time (page 1, section
// "Step 2: set the tile size": each block owns one tm x tn output tile).
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 256;            // 4 waves of 64 lanes, 2 x 2 over the tile

// Raster group height in tiles. Page 1, section "Swizzle", groups 8 tile-rows
// of 128 rows (GROUP_SIZE_M = 8 with tm = 128): 1024 rows of A per group. With
// 256-row tiles the same 1024 rows are 4 tile-rows (on MI355X, 4 and 8 measure
// the same within noise at 8192^3 and on the projection shape).
constexpr int kDefaultGroupM = 4;
constexpr int kDefaultNumXcd = 8;        // MI355X: 8 accelerator dies of 32 CUs
constexpr int kCusPerXcd = 32;           // gfx950: compute units per accelerator die

// Dies the dispatcher deals workgroups over, for a device of `ncu` compute
// units: a whole MI355X has 8 dies of 32 compute units; a partitioned one
// exposes a whole number of dies per device (4, 2 or 1).
inline int num_xcd_for(int ncu) {
    const int x = ncu / kCusPerXcd;
    return x < 1 ? 1 : (x > kDefaultNumXcd ? kDefaultNumXcd : x);
}
// Direct-to-LDS pipeline: K step and LDS ring depth (a stage holds 64 KiB at
// K step 64, 32 KiB at K step 32). 64-deep steps take a 2-stage ring.
constexpr int kDefaultDmaKStep = 64;
constexpr int kDefaultDmaStages32 = 4;     // ring depth when the K step is 32
// Tiles of 128 or 64 rows (x 256 columns) run two workgroups per compute
// unit: 32-deep steps in a ring of at most 80 KiB (3 stages by default).
constexpr int kDefaultSmallStages = 3;
constexpr int kProducerWaves = 4;          // producer/consumer workgroups: 4 + 4 waves

// Automatic launches of 16-bit operands with B stored K x N, K not a multiple
// of 64 and no more tiles than compute units take 32-deep steps (default ring
// depth, built for every type combination): measured 2-4% ahead of the
// 64-deep default there (3001x5003x4099 and 3072x5120x4099), while with K a
// multiple of 64, or B stored N x K, the 64-deep ring is 3-9% ahead on every
// grid of one round or less measured.
constexpr int kPartialKxNKStep = 32;
constexpr int kF32KStep = 16;              // K step (floats) of the binary32-operand kernels

enum : int { kVecAB = 1, kVecC = 2, kLayoutNxK = 4, kDma = 8 };

// Largest row stride (elements) for the direct-to-LDS path: every in-range
// byte offset inside a 256-row panel, (255 * ld + K) * 2 with K <= ld, stays
// below 2^31, under the out-of-range offset the kernel uses for zero padding.
constexpr int64_t kMaxDmaLd = 4000000;

// Output tile computed by workgroup `wid` of W = grid_m * grid_n.
// Step 1 (die-aware renumbering): the dispatcher hands workgroup w to die
// w mod X. Renumber so die x receives one contiguous range of logical ids,
// in its own dispatch order, so neighbouring tiles share that die's L2.
// Step 2 (grouped order, page 1, section "Swizzle"): logical ids walk down
// group_m tile-rows before moving one tile-column right, so a die's
// concurrently running tiles reuse a few A row-panels and B column-panels.
// group_m must be <= grid_m (the host clamps it; larger values map the same).
TG_HD inline void tile_of(int wid, int W, int grid_m, int grid_n, int group_m, int num_xcd,
                          int* tile_m, int* tile_n) {
    int p = wid;
    if (num_xcd > 1) {
        const int q = W / num_xcd, r = W % num_xcd;
        const int x = wid % num_xcd, s = wid / num_xcd;
        p = (x < r) ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
    }
    const int in_group = group_m * grid_n;
    const int g = p / in_group;
    const int first = g * group_m;
    const int rows = (grid_m - first < group_m) ? grid_m - first : group_m;
    *tile_m = first + p % rows;
    *tile_n = (p - g * in_group) / rows;
}

struct Plan {
    int M, N, K;
    int64_t lda, ldb, ldc;
    int layout;        // 0 = KxN, 1 = NxK
    int ab_type;       // TGEMM_F16, TGEMM_BF16 or TGEMM_F32 (both operands)
    int c_type;        // TGEMM_F16, TGEMM_BF16 or TGEMM_F32
    bool epi;          // scale, bias or activation requested (else C = A * B as it is)
    int variant;       // kVecAB | kVecC | kLayoutNxK | kDma bits
    int bm;            // tile rows of the launched kernel (BM, or 128 / 64 for the small tiles)
    int bn;            // tile columns of the launched kernel (BN)
    int producers;     // producer waves per workgroup (0, or kProducerWaves)
    int threads;       // threads per workgroup
    int grid_m, grid_n, W;
    int group_m, num_xcd;
    int k_step, stages;   // K step per LDS stage and ring depth of the launched kernel
    int grid;             // workgroups launched (W, or the compute units for a persistent launch)
    bool c_stream;        // C's base and row pitch multiples of 128 bytes: its 16-byte stores are streamed
};

// Binary32 operands planned onto the direct-to-LDS kernel: it is launched
// with K and both row strides counted in 16-bit units.
inline bool f32_on_dma(const Plan& pl) { return pl.ab_type == TGEMM_F32 && (pl.variant & kDma); }

inline bool span_bytes(int64_t rows, int64_t cols, int64_t ld, uint64_t* bytes, int esize = 2) {
    // bytes covered by a row-major rows x cols array of esize-byte elements
    if (rows <= 0 || cols <= 0) {
        *bytes = 0;
        return true;
    }
    int64_t last;
    if (__builtin_mul_overflow(rows - 1, ld, &last)) return false;
    if (__builtin_add_overflow(last, cols, &last)) return false;
    if (last > INT64_MAX / 4) return false;
    *bytes = (uint64_t)last * (uint64_t)esize;
    return true;
}

inline bool overlaps(const void* p, uint64_t pn, const void* q, uint64_t qn) {
    if (pn == 0 || qn == 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + qn && b < a + pn;
}

// ab_type / c_type: element types; bias: N floats or null; alpha and act as
// in tgemm_gemm (epi: alpha != 1, a bias or an activation).
// tile_m: 0 (automatic: 256), 256, 128 or 64 tile rows; producers: 0, or 4
// (producer/consumer workgroups, 128-row tiles).
inline int make_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, int b_layout, void* C, int64_t ldc, int force_generic,
                     int group_m, int num_xcd, int k_step, int stages, Plan* pl,
                     int ab_type = TGEMM_F16, int c_type = TGEMM_F16, const void* bias = nullptr,
                     bool epi = false, int tile_m = 0, int producers = 0) {
    const int64_t kMaxDim = 2147483647;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return TGEMM_ERR_INVALID;
    if (b_layout != TGEMM_B_KxN && b_layout != TGEMM_B_NxK) return TGEMM_ERR_INVALID;
    if (ab_type != TGEMM_F16 && ab_type != TGEMM_BF16 && ab_type != TGEMM_F32) return TGEMM_ERR_INVALID;
    if (c_type != TGEMM_F16 && c_type != TGEMM_BF16 && c_type != TGEMM_F32) return TGEMM_ERR_INVALID;
    const int ab_size = ab_type == TGEMM_F32 ? 4 : 2;
    const int c_size = c_type == TGEMM_F32 ? 4 : 2;
    if (force_generic != 0 && force_generic != 1) return TGEMM_ERR_INVALID;
    if (group_m < 0 || group_m > 1024 || num_xcd < 0 || num_xcd > 64) return TGEMM_ERR_INVALID;
    // (binary32 operands always step 16 floats: 0 or 16, the value a plan reports)
    if (k_step != 0 && k_step != 32 && k_step != 64 && !(ab_type == TGEMM_F32 && k_step == kF32KStep))
        return TGEMM_ERR_INVALID;
    if (stages != 0 && (stages < 2 || stages > 5)) return TGEMM_ERR_INVALID;
    if (k_step == 64 && stages != 0 && stages != 2) return TGEMM_ERR_INVALID;  // 2 x 64 KiB fills LDS
    if (tile_m != 0 && tile_m != 256 && tile_m != 128 && tile_m != 64) return TGEMM_ERR_INVALID;
    if (producers != 0 && producers != kProducerWaves) return TGEMM_ERR_INVALID;
    if (producers && tile_m != 0 && tile_m != 128) return TGEMM_ERR_INVALID;
    const int bm = producers ? 128 : (tile_m ? tile_m : BM);
    // smaller tiles and producer/consumer workgroups: 32-deep steps, and a
    // ring of at most 80 KiB per workgroup (two per compute unit) for the
    // small tiles
    if (bm != BM && k_step == 64) return TGEMM_ERR_INVALID;
    if (bm != BM && !producers && stages > 3) return TGEMM_ERR_INVALID;
    const int64_t one = 1;
    if (lda < (K > one ? K : one)) return TGEMM_ERR_INVALID;
    const int64_t bmin = (b_layout == TGEMM_B_KxN) ? N : K;
    if (ldb < (bmin > one ? bmin : one)) return TGEMM_ERR_INVALID;
    if (ldc < (N > one ? N : one)) return TGEMM_ERR_INVALID;

    uint64_t na, nb, nc;
    if (!span_bytes(M, K, lda, &na, ab_size)) return TGEMM_ERR_INVALID;
    if (b_layout == TGEMM_B_KxN) {
        if (!span_bytes(K, N, ldb, &nb, ab_size)) return TGEMM_ERR_INVALID;
    } else {
        if (!span_bytes(N, K, ldb, &nb, ab_size)) return TGEMM_ERR_INVALID;
    }
    if (!span_bytes(M, N, ldc, &nc, c_size)) return TGEMM_ERR_INVALID;
    if ((na && !A) || (nb && !B) || (nc && !C)) return TGEMM_ERR_INVALID;
    if (((uintptr_t)A % ab_size) || ((uintptr_t)B % ab_size) || ((uintptr_t)C % c_size)) return TGEMM_ERR_INVALID;
    if (overlaps(C, nc, A, na) || overlaps(C, nc, B, nb)) return TGEMM_ERR_INVALID;
    // the bias is read while C is written: 4-byte aligned, apart from C
    const uint64_t nbias = bias ? (uint64_t)N * 4u : 0u;
    if (bias && ((uintptr_t)bias & 3)) return TGEMM_ERR_INVALID;
    if (overlaps(C, nc, bias, nbias)) return TGEMM_ERR_INVALID;

    // tile grid: fixed below once the kernel (and its tile width) is known
    const int64_t gm = (M + bm - 1) / bm;

    pl->M = (int)M;
    pl->N = (int)N;
    pl->K = (int)K;
    pl->lda = lda;
    pl->ldb = ldb;
    pl->ldc = ldc;
    pl->c_stream = ((uintptr_t)C % 128 == 0) && ((ldc * c_size) % 128 == 0);
    pl->layout = b_layout;
    pl->ab_type = ab_type;
    pl->c_type = c_type;
    pl->epi = epi;
    int g = group_m ? group_m : kDefaultGroupM;
    if (gm > 0 && g > gm) g = (int)gm;
    pl->group_m = g > 0 ? g : 1;
    pl->num_xcd = num_xcd ? num_xcd : kDefaultNumXcd;

    const bool vec_ab = !force_generic && ((uintptr_t)A % 16 == 0) && ((lda * ab_size) % 16 == 0) &&
                        ((uintptr_t)B % 16 == 0) && ((ldb * ab_size) % 16 == 0);
    // vector C stores: 8-byte runs of a 16-bit C, 16-byte runs of an fp32 C
    const int c_vec = c_type == TGEMM_F32 ? 16 : 8;
    const bool vec_c = ((uintptr_t)C % c_vec == 0) && ((ldc * c_size) % c_vec == 0);
    // direct-to-LDS (any 2-byte alignment: gfx950 buffer loads accept
    // unaligned addresses): row strides small enough for 32-bit panel
    // offsets (a K x N B is rebased at every K step, so its offsets stay
    // below 64 * ldb * 2 + 512 bytes whatever K is: the same stride limit).
    // (K == 0 only writes zeros: the register-staged kernel does that)
    // (row strides of at least 8 elements: then a 16-byte access can run past
    // the end of an operand only in its last row, which the kernel reloads
    // element by element; narrower operands take the register-staged kernel)
    // (binary32 operands run on the same kernel as pairs of 16-bit units: row
    // strides of at least 4 floats and at most half the 16-bit limit)
    const bool dma =
        ab_type == TGEMM_F32
            ? (!force_generic && K > 0 && lda >= 4 && ldb >= 4 && lda <= kMaxDmaLd / 2 && ldb <= kMaxDmaLd / 2)
            : (!force_generic && K > 0 && lda >= 8 && ldb >= 8 && lda <= kMaxDmaLd && ldb <= kMaxDmaLd);
    // binary32 operands on the direct-to-LDS kernel
    const bool f32_dma = ab_type == TGEMM_F32 && dma;
    pl->variant = (vec_ab ? kVecAB : 0) | (vec_c ? kVecC : 0) |
                  (b_layout == TGEMM_B_NxK ? kLayoutNxK : 0) | (dma ? kDma : 0);
    if (f32_dma) {
        // 16 floats per step whatever k_step asks; 2 stages (256-row tiles) or 3
        pl->k_step = kF32KStep;
        pl->stages = stages ? stages : (bm != BM ? kDefaultSmallStages : 2);
    } else if (ab_type == TGEMM_F32) {
        pl->k_step = kF32KStep;
        pl->stages = 2;
    } else if (dma) {
        // a ring deeper than 2 stages implies 32-deep steps; 64-deep steps
        // need at least two steps
        pl->k_step = k_step ? k_step : ((stages > 2 || K <= 64 || bm != BM) ? 32 : kDefaultDmaKStep);
        if (pl->k_step == 64 && K <= 64) return TGEMM_ERR_INVALID;
        pl->stages = pl->k_step == 64 ? 2 : (stages ? stages : (bm != BM ? kDefaultSmallStages : kDefaultDmaStages32));
    } else {
        pl->k_step = BK;
        pl->stages = 2;
    }
    // the small tiles and producer/consumer workgroups exist on the
    // direct-to-LDS path only
    if (bm != BM && !(dma && (ab_type != TGEMM_F32 || f32_dma))) return TGEMM_ERR_UNSUPPORTED;
    pl->bm = bm;
    pl->producers = producers;
    pl->threads = NTHREADS + producers * 64;
    pl->bn = BN;
    const int64_t gn = (N + pl->bn - 1) / pl->bn;
    if (gm * gn > kMaxDim) return TGEMM_ERR_UNSUPPORTED;
    pl->grid_m = (int)gm;
    pl->grid_n = (int)gn;
    pl->W = (int)(gm * gn);
    pl->grid = pl->W;
    return TGEMM_OK;
}

}  // namespace tg
