// Host planning code under AddressSanitizer and UndefinedBehaviorSanitizer
// (built with g++ by tests/test_sanitizers.py; no GPU, no HIP runtime).
// Runs make_plan over an argument table (every rejection rule, the edge
// values of each limit, the five workload shapes, both layouts, all element
// types) and tile_of over every workgroup of many grids, checking that the
// map is a bijection onto the tile grid. Any overflow, out-of-bounds access
// or undefined operation aborts the run; a wrong answer exits non-zero.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tgemm_plan.h"

using tg::make_plan;
using tg::Plan;

static int g_fail = 0;

#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
                         __LINE__, #cond);                                        \
            ++g_fail;                                                             \
        }                                                                         \
    } while (0)

static const uintptr_t PA = uintptr_t(1) << 40, PB = uintptr_t(2) << 40, PC = uintptr_t(3) << 40;

static int plan(int64_t M, int64_t N, int64_t K, uintptr_t A, int64_t lda, uintptr_t B, int64_t ldb, int lay,
                uintptr_t C, int64_t ldc, int fg = 0, int gm = 0, int nx = 0, int ks = 0, int st = 0,
                int ab = TGEMM_F16, int ct = TGEMM_F16, uintptr_t bias = 0, Plan* out = nullptr) {
    Plan p{};
    const int rc = make_plan(M, N, K, (const void*)A, lda, (const void*)B, ldb, lay, (void*)C, ldc, fg, gm, nx, ks,
                             st, &p, ab, ct, (const void*)bias, bias != 0);
    if (rc == TGEMM_OK) {
        // what a launch derives from a plan stays consistent
        EXPECT(p.W == p.grid_m * p.grid_n && p.grid == p.W);
        EXPECT(p.grid_m == (M + 255) / 256);
        EXPECT(p.k_step == 16 || p.k_step == 32 || p.k_step == 64);
        EXPECT(p.stages >= 2 && p.stages <= 5);
        EXPECT(p.group_m >= 1 && p.group_m <= 1024);
    }
    if (out) *out = p;
    return rc;
}

int main() {
    const int64_t big = int64_t(1) << 31;
    // rejections (nothing planned)
    EXPECT(plan(-1, 4, 4, PA, 4, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, -1, 4, PA, 4, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, -1, PA, 4, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(big, 4, 4, PA, 4, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, big, 4, PA, 4, PB, big, 0, PC, big) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 8, PA, 7, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 9, 8, PA, 8, PB, 8, 0, PC, 9) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 9, 8, PA, 8, PB, 7, 1, PC, 9) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 9, 8, PA, 8, PB, 9, 0, PC, 8) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, 0, 4, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, 0, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, 0, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA + 1, 4, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC + 3, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PA + 8, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PB, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 2, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 2) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, -1) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 1025) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 65) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 16) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 1) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 6) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 64, 3) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 16, 64, PA, 64, PB, 16, 0, PC, 16, 0, 0, 0, 64) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 0, 3) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 0, 0, 3) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA + 2, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 0, TGEMM_F32) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 0, 0, 0, PC + 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 0, 0, 0, PB + 1024 + 2) == TGEMM_ERR_INVALID);
    // spans whose byte count overflows int64 are rejected, not wrapped
    EXPECT(plan(big - 1, 4, 8, PA, int64_t(1) << 62, PB, 4, 0, PC, 4) == TGEMM_ERR_INVALID);
    EXPECT(plan(4, 4, big - 1, PA, big - 1, PB, int64_t(1) << 61, 1, PC, 4) == TGEMM_ERR_INVALID);

    // accepted plans: the five workloads and the stride limits
    Plan p;
    EXPECT(plan(8192, 8192, 8192, PA, 8192, PB, 8192, 1, PC, 8192, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT((p.variant & tg::kDma) && p.W == 1024 && p.k_step == 64 && p.stages == 2);
    EXPECT(plan(3001, 5003, 4099, PA, 4099, PB, 5003, 0, PC, 5003, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT((p.variant & tg::kDma) && p.W == 240);
    EXPECT(plan(256, 256, 256, PA, 256, PB, 256, 0, PC, 256, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT(plan(4096, 4096, 4096, PA, 4096, PB, 4096, 0, PC, 4096, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT(plan(8192, 12288, 4096, PA, 4096, PB, 4096, 1, PC, 12288, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT(p.W == 1536);
    EXPECT(plan(512, 512, 512, PA, tg::kMaxDmaLd, PB, 512, 1, PC, 512, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT(p.variant & tg::kDma);
    EXPECT(plan(512, 512, 512, PA, tg::kMaxDmaLd + 8, PB, 512, 1, PC, 512, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT(!(p.variant & tg::kDma) && (p.variant & tg::kVecAB));
    EXPECT(plan(8192, 152064, 8192, PA, 8192, PB, 152064, 0, PC, 152064, 0, 0, 0, 0, 0, 0, 0, 0, &p) == TGEMM_OK);
    EXPECT(p.variant & tg::kDma);
    EXPECT(plan(4, 4, 4, PA, 4, PB, 4, 0, PC, 4, 0, 0, 0, 0, 0, TGEMM_F32, TGEMM_F32, 0, &p) == TGEMM_OK);
    EXPECT(plan(0, 5, 7, 0, 7, PB, 5, 0, 0, 5) == TGEMM_OK);
    EXPECT(plan(5, 5, 0, 0, 1, 0, 5, 0, PC, 5) == TGEMM_OK);
    // every argument combination of a small sweep plans or is rejected cleanly
    for (int64_t M : {0, 1, 255, 256, 257, 70000})
        for (int64_t N : {0, 1, 7, 8, 300})
            for (int64_t K : {0, 1, 64, 65, 4099})
                for (int lay : {0, 1})
                    for (int ab : {0, 1, 2})
                        for (int ks : {0, 32, 64})
                            for (int64_t pad : {0, 1, 8}) {
                                const int64_t lda = (K > 0 ? K : 1) + pad;
                                const int64_t ldb = ((lay == 0 ? N : K) > 0 ? (lay == 0 ? N : K) : 1) + pad;
                                const int64_t ldc = (N > 0 ? N : 1) + pad;
                                const int rc = plan(M, N, K, PA, lda, PB, ldb, lay, PC, ldc, 0, 0, 0, ks, 0, ab);
                                EXPECT(rc == TGEMM_OK || rc == TGEMM_ERR_INVALID);
                            }

    // tile_of: a bijection onto the tile grid for every grid, group height and die count
    for (int gm = 1; gm <= 40; gm += 3)
        for (int gn = 1; gn <= 40; gn += 7)
            for (int g : {1, 2, 4, 8, 16})
                for (int x : {1, 3, 8}) {
                    const int W = gm * gn;
                    std::vector<char> seen((size_t)W, 0);
                    const int gc = g > gm ? gm : g;
                    for (int w = 0; w < W; ++w) {
                        int tm = -1, tn = -1;
                        tg::tile_of(w, W, gm, gn, gc, x, &tm, &tn);
                        if (tm < 0 || tm >= gm || tn < 0 || tn >= gn) {
                            EXPECT(false);
                            continue;
                        }
                        seen[(size_t)tm * gn + tn]++;
                    }
                    for (int i = 0; i < W; ++i) EXPECT(seen[(size_t)i] == 1);
                }
    if (g_fail) {
        std::fprintf(stderr, "%d expectations failed\n", g_fail);
        return 1;
    }
    std::printf("plan_check: all expectations held\n");
    return 0;
}
