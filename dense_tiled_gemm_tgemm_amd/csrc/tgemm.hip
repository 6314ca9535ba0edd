// Host entry points of the dense tiled GEMM for MI355X (gfx950): argument
// checks and planning (tgemm_plan.h), kernel choice among the instantiated
// combinations of element types and epilogue, and the launch. The kernels and
// their design are in tgemm_kernels.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <unordered_map>
#include <vector>

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
    TG_PICK(2, 0)
    TG_PICK(2, 1)
    TG_PICK(2, 2)
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

// The current device's compute units into *ncu: TGEMM_OK, or TGEMM_ERR_HIP
// (hipError_t kept for tgemm_last_hip_error) when there is no usable device.
static int device_compute_units(int* ncu) {
    const int n = compute_units();
    if (n <= 0) {
        g_last_hip_error = n < 0 ? -n : (int)hipErrorInvalidDevice;
        return TGEMM_ERR_HIP;
    }
    *ncu = n;
    return TGEMM_OK;
}

static bool epilogue_requested(float alpha, const float* bias, int act) {
    return !(alpha == 1.0f) || bias != nullptr || act != TGEMM_ACT_NONE;
}

// ---------------------------------------------------------------------------
// Runtime tuning (page 2, "CUDA 13.1 new feature: the Tile programming model",
// section 7.4: several tile configurations are tried and the fastest is kept
// per problem shape, so later calls pay nothing). Here the choices are the
// launch parameters that leave the result unchanged bit for bit: K step and
// LDS ring depth of the direct-to-LDS pipeline, and the raster group height.
// The table is per device, keyed by everything that selects a kernel: sizes,
// strides, layout, types, epilogue on/off, the variant bits (alignment
// classes, load path) and the C store policy.
// ---------------------------------------------------------------------------
struct TuneKey {
    int dev;
    int64_t M, N, K, lda, ldb, ldc;
    int layout, ab, ct, epi, variant, c_stream;
    bool operator==(const TuneKey& o) const {
        return dev == o.dev && M == o.M && N == o.N && K == o.K && lda == o.lda && ldb == o.ldb && ldc == o.ldc &&
               layout == o.layout && ab == o.ab && ct == o.ct && epi == o.epi && variant == o.variant &&
               c_stream == o.c_stream;
    }
};

struct TuneKeyHash {
    size_t operator()(const TuneKey& k) const {
        uint64_t h = 1469598103934665603ull;
        const int64_t v[] = {k.dev, k.M,      k.N,  k.K,  k.lda,   k.ldb,    k.ldc,
                             k.layout, k.ab, k.ct, k.epi, k.variant, k.c_stream};
        for (int64_t x : v) h = (h ^ (uint64_t)x) * 1099511628211ull;    // FNV-1a over the fields
        return (size_t)h;
    }
};

struct TuneChoice {
    int k_step, stages, group_m, num_xcd, tile_m, producers;
};

constexpr float kTuneWarmupMs = 100.f;        // GPU time of the clock-settling launches
constexpr int kTuneWarmupMaxLaunches = 4096;
constexpr float kTuneMinGain = 0.99f;         // a choice must be at least 1% faster than the untuned launch

static std::mutex g_tune_mu;
static std::unordered_map<TuneKey, TuneChoice, TuneKeyHash> g_tuned;
static std::atomic<int> g_tuned_count{0};

static bool tune_key(const Plan& pl, TuneKey* k) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    *k = TuneKey{dev,        pl.M,       pl.N,        pl.K,      pl.lda,     pl.ldb,
                 pl.ldc,     pl.layout,  pl.ab_type,  pl.c_type, pl.epi ? 1 : 0, pl.variant,
                 pl.c_stream ? 1 : 0};
    return true;
}

static bool tuned_choice(const Plan& pl, TuneChoice* c) {
    if (g_tuned_count.load(std::memory_order_acquire) == 0) return false;   // nothing tuned: no runtime query
    TuneKey k;
    if (!tune_key(pl, &k)) return false;
    std::lock_guard<std::mutex> lock(g_tune_mu);
    const auto it = g_tuned.find(k);
    if (it == g_tuned.end()) return false;
    *c = it->second;
    return true;
}

// Plan and kernel for a call on a device with `ncu` compute units (0: the
// current device's, queried only once the arguments have passed and there is
// work to plan). With every launch choice automatic (all zero) the choice
// recorded by tgemm_tune_gemm for this problem, if any, is used.
static int plan_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda, const void* B,
                     int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc, float alpha, const float* bias,
                     int act, int force_generic, int group_m, int num_xcd, int k_step, int stages, int tile_m,
                     int producers, int ncu, Plan* pl, const void** fn, bool use_tuned = true) {
    if (act != TGEMM_ACT_NONE && act != TGEMM_ACT_RELU) return TGEMM_ERR_INVALID;
    const bool epi = epilogue_requested(alpha, bias, act);
    int rc = make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, force_generic, group_m, num_xcd, k_step, stages,
                       pl, ab_type, c_type, bias, epi, tile_m, producers);
    if (rc != TGEMM_OK) return rc;
    if (pl->M == 0 || pl->N == 0) {              // nothing to launch
        *fn = nullptr;
        pl->grid = 0;
        return TGEMM_OK;
    }
    if (!pick_kernel(*pl)) return TGEMM_ERR_UNSUPPORTED;   // before any device query
    if (ncu == 0) {
        rc = device_compute_units(&ncu);
        if (rc != TGEMM_OK) return rc;
    }
    TuneChoice t;
    const bool automatic = !force_generic && !group_m && !num_xcd && !k_step && !stages && !tile_m && !producers;
    const bool tuned = automatic && use_tuned && tuned_choice(*pl, &t);
    if (tuned) {
        Plan tp;
        rc = make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, 0, t.group_m, t.num_xcd, t.k_step, t.stages,
                       &tp, ab_type, c_type, bias, epi, t.tile_m, t.producers);
        if (rc == TGEMM_OK) *pl = tp;
    } else if (automatic && f32_on_dma(*pl)) {
        // binary32 operands: a 64-row tile keeps 96-98% of the 256-row tile's
        // rate (the matrix work per staged byte is 8 times that of 16-bit
        // operands), and its finer grid balances better, so it is taken
        // unless the 256-row tiles fill at least 7/8 of their rounds over the
        // compute units (measured at 256 units: 64 rows ahead by 23-54% with
        // 160, 192, 320 and 384 tiles and by 1.9-3.6x below half a round;
        // even at 224; 256-row tiles 2-4% ahead with 256, 1024 and 1536)
        const int64_t rounds = ((int64_t)pl->W + ncu - 1) / ncu;
        if ((int64_t)pl->W * 8 < rounds * ncu * 7) {
            Plan rp;
            rc = make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, 0, 0, 0, 0, 0, &rp, ab_type, c_type, bias, epi,
                           64, 0);
            if (rc == TGEMM_OK) *pl = rp;
        }
    } else if (automatic && (pl->variant & kDma) && ab_type != TGEMM_F32 && (int64_t)pl->W * 2 <= ncu) {
        // a grid of 256-row tiles filling at most half of the compute units:
        // smaller tiles spread the same work over more workgroups; 64-row
        // tiles when it fills a quarter or less (256^3: 3.0 -> 5.9 TFLOP/s,
        // 2048^3: 441 -> 613), 128-row tiles up to half (2560 x 2048 x 2048:
        // 545 -> 718, 4096 x 2048 x 2048: 872 -> 963); above half the
        // 256-row tile is ahead (2560 x 4096 x 2048: 1058 against 773)
        Plan rp;
        const int tm = (int64_t)pl->W * 4 <= ncu ? 64 : 128;
        rc = make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, 0, 0, 0, 0, 0, &rp, ab_type, c_type, bias, epi, tm, 0);
        if (rc == TGEMM_OK) *pl = rp;
    } else if (automatic && (pl->variant & kDma) && !(pl->variant & kLayoutNxK) && ab_type != TGEMM_F32 &&
               K > 64 && K % 64 != 0 && pl->W <= ncu) {
        Plan rp;
        rc = make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, 0, 0, 0, kPartialKxNKStep, 0, &rp, ab_type,
                       c_type, bias, epi);
        if (rc == TGEMM_OK) *pl = rp;
    }
    // one workgroup per compute unit, each walking several tiles
    if (persistent(*pl) && ncu < pl->W) pl->grid = ncu;
    if (!num_xcd && !tuned) pl->num_xcd = num_xcd_for(ncu);    // the tuned choice names its own
    *fn = pick_kernel(*pl);
    return *fn ? TGEMM_OK : TGEMM_ERR_UNSUPPORTED;
}

// Enqueue the planned kernel.
static int launch(const Plan& pl, const void* fn, const void* A, const void* B, void* C, int c_type, float alpha,
                  const float* bias, int act, void* stream) {
    const int c_size = c_type == TGEMM_F32 ? 4 : 2;
    Args args;
    args.A = static_cast<const uint16_t*>(A);
    args.B = static_cast<const uint16_t*>(B);
    args.C = C;
    args.bias = bias;
    args.alpha = alpha;
    args.relu = act == TGEMM_ACT_RELU;
    // binary32 operands on the direct-to-LDS kernel: K and the operand
    // strides in 16-bit units (the kernel moves bytes; its matrix
    // instructions read the 4-byte values)
    const int units = f32_on_dma(pl) ? 2 : 1;
    args.lda = pl.lda * units;
    args.ldb = pl.ldb * units;
    args.ldc = pl.ldc;
    args.M = pl.M;
    args.N = pl.N;
    args.K = pl.K * units;
    args.grid_m = pl.grid_m;
    args.grid_n = pl.grid_n;
    args.W = pl.W;
    args.group_m = pl.group_m;
    args.num_xcd = pl.num_xcd;
    args.grid = pl.grid;
    // 16-byte C stores at any alignment of the rows (gfx950 buffer stores
    // accept unaligned addresses, as its buffer loads do: on the 3001 x 5003
    // x 4099 workload, whose C rows are 2-byte aligned, 140.2 -> 130.8 us
    // against element stores), wherever every byte offset inside a wave's
    // 128 rows stays below 2^31 (they go through a 32-bit buffer offset)
    args.c16 = (127 * pl.ldc + (int64_t)pl.N) * c_size + 16 < (int64_t(1) << 31);
    args.c8 = (pl.variant & kVecC) != 0;
    // streamed 16-byte C stores where whole 128-byte lines are written
    args.c_stream = pl.c_stream;
    void* kargs[] = {&args};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)args.grid), dim3((unsigned)pl.threads), kargs, 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return TGEMM_ERR_HIP;
    }
    return TGEMM_OK;
}

}  // namespace tg

extern "C" int tgemm_gemm_config(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc,
                                 float alpha, const float* bias, int act, void* stream, int force_generic,
                                 int group_m, int num_xcd, int k_step, int stages, int tile_m, int producers) {
    tg::Plan pl;
    const void* fn = nullptr;
    const int rc = tg::plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act,
                                 force_generic, group_m, num_xcd, k_step, stages, tile_m, producers, 0, &pl, &fn);
    if (rc != TGEMM_OK) return rc;
    if (pl.M == 0 || pl.N == 0) return TGEMM_OK;
    return tg::launch(pl, fn, A, B, C, c_type, alpha, bias, act, stream);
}

extern "C" int tgemm_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc, float alpha,
                          const float* bias, int act, void* stream) {
    return tgemm_gemm_config(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act, stream,
                             0, 0, 0, 0, 0, 0, 0);
}

extern "C" int tgemm_f16_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, int b_layout, void* C, int64_t ldc,
                                void* stream, int force_generic, int group_m, int num_xcd, int k_step,
                                int stages, int tile_m, int producers) {
    return tgemm_gemm_config(M, N, K, TGEMM_F16, A, lda, B, ldb, b_layout, TGEMM_F16, C, ldc, 1.0f, nullptr,
                             TGEMM_ACT_NONE, stream, force_generic, group_m, num_xcd, k_step, stages, tile_m,
                             producers);
}

extern "C" int tgemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                         int64_t ldb, int b_layout, void* C, int64_t ldc, void* stream) {
    return tgemm_f16_config(M, N, K, A, lda, B, ldb, b_layout, C, ldc, stream, 0, 0, 0, 0, 0, 0, 0);
}

extern "C" int tgemm_tune_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda,
                               const void* B, int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc,
                               float alpha, const float* bias, int act, void* stream, int rounds, int64_t* info) {
    if (rounds < 1 || rounds > 100) return TGEMM_ERR_INVALID;
    tg::Plan base;
    const void* fn = nullptr;
    int rc = tg::plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act, 0, 0, 0, 0,
                           0, 0, 0, 0, &base, &fn, false);
    if (rc != TGEMM_OK) return rc;
    if (info)
        for (int i = 0; i < 8; ++i) info[i] = 0;
    if (base.M == 0 || base.N == 0) return TGEMM_OK;
    int ncu = 0;
    rc = tg::device_compute_units(&ncu);
    if (rc != TGEMM_OK) return rc;

    // candidates: tile rows x K step x ring depth (direct-to-LDS path only:
    // 256-row tiles with 64- or 32-deep steps, 128- and 64-row tiles at two
    // workgroups per compute unit, producer/consumer workgroups) x raster
    // group height; those not built for the types drop out
    struct Cand {
        tg::TuneChoice c;
        tg::Plan pl;
        const void* fn;
    };
    std::vector<Cand> cands;
    const int pipes16[][4] = {{64, 2, 256, 0}, {32, 4, 256, 0}, {32, 2, 256, 0}, {32, 3, 256, 0}, {32, 5, 256, 0},
                              {32, 3, 128, 0}, {32, 2, 128, 0}, {32, 3, 64, 0},  {32, 3, 128, 4}, {32, 5, 128, 4}};
    // binary32 operands: 16-deep steps only (the K step choice does not apply)
    const int pipes32[][4] = {{16, 2, 256, 0}, {16, 3, 256, 0}, {16, 3, 128, 0}, {16, 3, 64, 0}};
    const bool f32 = ab_type == TGEMM_F32;
    const int(*pipes)[4] = f32 ? pipes32 : pipes16;
    const int npipes = (base.variant & tg::kDma) ? (f32 ? 4 : (int)(sizeof(pipes16) / sizeof(pipes16[0]))) : 1;
    const int groups[] = {4, 8, 16};
    for (int ip = 0; ip < npipes; ++ip) {
        for (int g : groups) {
            const bool dma = (base.variant & tg::kDma) != 0;
            const int ks = dma ? pipes[ip][0] : 0;
            const int st = dma ? pipes[ip][1] : 0;
            const int tm = dma ? pipes[ip][2] : 0;
            const int pr = dma ? pipes[ip][3] : 0;
            Cand cd;
            cd.c = tg::TuneChoice{ks, st, g, tg::num_xcd_for(ncu), tm, pr};
            if (tg::plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act, 0, g,
                              tg::num_xcd_for(ncu), ks, st, tm, pr, ncu, &cd.pl, &cd.fn, false) != TGEMM_OK)
                continue;                                   // not built for these types, or invalid for this K
            bool dup = false;                               // group heights clamp to the tile rows
            for (const Cand& o : cands)
                dup = dup || (o.pl.k_step == cd.pl.k_step && o.pl.stages == cd.pl.stages &&
                              o.pl.group_m == cd.pl.group_m && o.pl.bm == cd.pl.bm &&
                              o.pl.producers == cd.pl.producers);
            if (!dup) cands.push_back(cd);
        }
    }
    if (cands.empty()) return TGEMM_ERR_UNSUPPORTED;
    const int nc = (int)cands.size();
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the launch the problem gets without tuning
    int def = 0;
    for (int i = 0; i < nc; ++i)
        if (cands[i].pl.k_step == base.k_step && cands[i].pl.stages == base.stages &&
            cands[i].pl.group_m == base.group_m && cands[i].pl.bm == base.bm &&
            cands[i].pl.producers == base.producers)
            def = i;
    // one event between consecutive launches; every round runs every candidate
    // once, round r starting at candidate r (so no candidate always runs first
    // or last in a round while the clock drifts)
    std::vector<hipEvent_t> ev((size_t)nc * rounds + 1, nullptr);
    hipError_t e = hipSuccess;
    for (auto& x : ev)
        if (e == hipSuccess) e = hipEventCreate(&x);
    for (int i = 0; i < nc && e == hipSuccess && rc == TGEMM_OK; ++i)       // one launch of each
        rc = tg::launch(cands[i].pl, cands[i].fn, A, B, C, c_type, alpha, bias, act, stream);
    // settle the clock first: the board's power-limited clock takes a fraction
    // of a second of sustained matrix work to reach its steady state, and
    // candidates timed before that differ by more than the choices do
    {
        float warm_ms = 0.f;
        int n = 0;
        while (e == hipSuccess && rc == TGEMM_OK && warm_ms < tg::kTuneWarmupMs && n < tg::kTuneWarmupMaxLaunches) {
            e = hipEventRecord(ev[0], st);
            for (int q = 0; q < 16 && e == hipSuccess && rc == TGEMM_OK; ++q, ++n)
                rc = tg::launch(cands[def].pl, cands[def].fn, A, B, C, c_type, alpha, bias, act, stream);
            if (e == hipSuccess && rc == TGEMM_OK) e = hipEventRecord(ev[1], st);
            if (e == hipSuccess && rc == TGEMM_OK) e = hipEventSynchronize(ev[1]);
            float ms = 0.f;
            if (e == hipSuccess && rc == TGEMM_OK) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
            warm_ms += ms;
        }
    }
    if (e == hipSuccess && rc == TGEMM_OK) e = hipEventRecord(ev[0], st);
    for (int r = 0; r < rounds && e == hipSuccess && rc == TGEMM_OK; ++r)
        for (int q = 0; q < nc && e == hipSuccess && rc == TGEMM_OK; ++q) {
            const int i = (q + r) % nc;
            rc = tg::launch(cands[i].pl, cands[i].fn, A, B, C, c_type, alpha, bias, act, stream);
            if (rc == TGEMM_OK) e = hipEventRecord(ev[(size_t)r * nc + q + 1], st);
        }
    if (e == hipSuccess && rc == TGEMM_OK) e = hipEventSynchronize(ev.back());
    std::vector<float> med(nc, 0.f);
    for (int i = 0; i < nc && e == hipSuccess && rc == TGEMM_OK; ++i) {
        std::vector<float> t(rounds);
        for (int r = 0; r < rounds && e == hipSuccess; ++r) {
            const int q = ((i - r) % nc + nc) % nc;   // position of candidate i in round r
            const size_t j = (size_t)r * nc + q;
            e = hipEventElapsedTime(&t[r], ev[j], ev[j + 1]);
        }
        std::sort(t.begin(), t.end());
        med[i] = t[rounds / 2];
    }
    for (auto& x : ev)
        if (x) (void)hipEventDestroy(x);
    if (rc != TGEMM_OK) return rc;
    if (e != hipSuccess) {
        tg::g_last_hip_error = (int)e;
        return TGEMM_ERR_HIP;
    }
    // the fastest median, unless it beats the untuned launch by too little to
    // tell from run-to-run noise
    int best = 0;
    for (int i = 1; i < nc; ++i)
        if (med[i] < med[best]) best = i;
    if (med[best] > tg::kTuneMinGain * med[def]) best = def;
    tg::TuneKey key;
    if (!tg::tune_key(base, &key)) return TGEMM_ERR_HIP;
    const tg::Plan& bp = cands[best].pl;
    {
        std::lock_guard<std::mutex> lock(tg::g_tune_mu);
        tg::g_tuned[key] = tg::TuneChoice{bp.k_step, bp.stages, bp.group_m, bp.num_xcd, bp.bm, bp.producers};
        tg::g_tuned_count.store((int)tg::g_tuned.size(), std::memory_order_release);
    }
    if (info) {
        info[0] = bp.k_step;
        info[1] = bp.stages;
        info[2] = bp.group_m;
        info[3] = bp.num_xcd;
        info[4] = (int64_t)(med[best] * 1e6f);   // median launch time, ns
        info[5] = nc;
        info[6] = bp.bm;
        info[7] = bp.producers;
    }
    return TGEMM_OK;
}

extern "C" int tgemm_tuning_entries(void) { return tg::g_tuned_count.load(std::memory_order_acquire); }

extern "C" void tgemm_tuning_clear(void) {
    std::lock_guard<std::mutex> lock(tg::g_tune_mu);
    tg::g_tuned.clear();
    tg::g_tuned_count.store(0, std::memory_order_release);
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
    info[1] = pl.bm;
    info[2] = pl.bn;
    info[3] = pl.k_step;
    info[4] = (pl.M == 0 || pl.N == 0) ? 0 : pl.grid;
    info[5] = pl.group_m;
    info[6] = pl.num_xcd;
    info[7] = pl.threads;
    info[8] = pl.stages;
    // LDS bytes per workgroup: stages x (A block + B block rows) x K step x element size
    info[9] = (int64_t)pl.stages * (pl.bm + pl.bn) * pl.k_step * (pl.ab_type == TGEMM_F32 ? 4 : 2);
}

extern "C" int tgemm_plan_gemm(int64_t M, int64_t N, int64_t K, int ab_type, const void* A, int64_t lda,
                               const void* B, int64_t ldb, int b_layout, int c_type, void* C, int64_t ldc,
                               float alpha, const float* bias, int act, int force_generic, int group_m,
                               int num_xcd, int k_step, int stages, int tile_m, int producers, int compute_units,
                               int64_t* info) {
    if (!info || compute_units < 0 || compute_units > 65536) return TGEMM_ERR_INVALID;
    tg::Plan pl;
    const void* fn = nullptr;
    const int rc = tg::plan_gemm(M, N, K, ab_type, A, lda, B, ldb, b_layout, c_type, C, ldc, alpha, bias, act,
                                 force_generic, group_m, num_xcd, k_step, stages, tile_m, producers, compute_units,
                                 &pl, &fn);
    if (rc != TGEMM_OK) return rc;
    fill_info(pl, info);
    return TGEMM_OK;
}

extern "C" int tgemm_plan_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, int b_layout, void* C, int64_t ldc, int force_generic,
                              int group_m, int num_xcd, int k_step, int stages, int tile_m, int producers,
                              int compute_units, int64_t* info) {
    return tgemm_plan_gemm(M, N, K, TGEMM_F16, A, lda, B, ldb, b_layout, TGEMM_F16, C, ldc, 1.0f, nullptr,
                           TGEMM_ACT_NONE, force_generic, group_m, num_xcd, k_step, stages, tile_m, producers,
                           compute_units, info);
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
