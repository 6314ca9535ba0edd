// Kernel instantiations for one (input type, output type, epilogue), chosen
// when this file is compiled: TG_AB (0 binary16, 1 bfloat16, 2 binary32
// inputs), TG_CT (0 binary16, 1 bfloat16, 2 fp32 output), TG_EPI (0 sums
// stored as they are, 1 scale, bias and activation applied). The library links one object per
// combination, so the combinations compile in parallel.
#include "tgemm_kernels.h"

#if !defined(TG_AB) || !defined(TG_CT) || !defined(TG_EPI)
#error "TG_AB, TG_CT and TG_EPI select the instantiated kernels"
#endif

namespace tg {
namespace {

constexpr int kTy = ty_code(TG_AB, TG_CT, TG_EPI != 0);
// the plain binary16 product instantiates every ring depth of 32-deep
// steps, the 2-stage ring of 128 x 256 tiles and the producer/consumer
// workgroups; the other combinations the default depth of each tile only
constexpr bool kAllDepths = (kTy == ty_code(0, 0, false));

template <int NXK>
const void* dma_ptr(int k_step, int stages, int tile_m, int producers, bool c_stream) {
    if (producers) {
        // producer/consumer workgroups: 128 x 256 tiles, 32-deep steps
        if constexpr (kAllDepths) {
            if (tile_m == 128 && k_step == 32 && stages == 3)
                return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3, 4, true>);
            if (tile_m == 128 && k_step == 32 && stages == 5)
                return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 5, 4, true>);
        }
        return nullptr;
    }
    if (tile_m == 128) {
        if (k_step == 32 && stages == kDefaultSmallStages)
            return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3, 4>);
        if constexpr (kAllDepths)
            if (k_step == 32 && stages == 2) return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 2, 4>);
        return nullptr;
    }
    if (tile_m == 64) {
        if (k_step == 32 && stages == kDefaultSmallStages)
            return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3, 2>);
        return nullptr;
    }
    // 64-deep steps: one build per C store policy
    if (k_step == 64)
        return c_stream ? reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 64, 2, 8, false, 1>)
                        : reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 64, 2, 8, false, 0>);
    if (stages == kDefaultDmaStages32) return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 4>);
    if constexpr (kAllDepths) {
        switch (stages) {
            case 2: return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 2>);
            case 3: return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3>);
            case 5: return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 5>);
            default: break;
        }
    }
    return nullptr;
}
static_assert(kDefaultDmaStages32 == 4 && kDefaultSmallStages == 3,
              "the default ring depths are instantiated for every combination");

template <int NXK>
const void* rs_ptr(bool vec) {
    return vec ? reinterpret_cast<const void*>(&tgemm_rs_kernel<kTy, NXK, true>)
               : reinterpret_cast<const void*>(&tgemm_rs_kernel<kTy, NXK, false>);
}

// binary32 operands: the direct-to-LDS kernel on the operands' bytes,
// 16-deep steps (32 16-bit units); 256-row tiles with a 2-, 3- or 4-stage
// ring, the smaller tiles with 3 stages
template <int NXK>
const void* f32_dma_ptr(int stages, int tile_m) {
    if constexpr (TG_AB == 2) {
        if (tile_m == 256 && stages == 2) return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 2>);
        if (tile_m == 256 && stages == 3) return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3>);
        if (tile_m == 256 && stages == 4) return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 4>);
        if (tile_m == 128 && stages == kDefaultSmallStages)
            return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3, 4>);
        if (tile_m == 64 && stages == kDefaultSmallStages)
            return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 32, 3, 2>);
    }
    (void)stages;
    (void)tile_m;
    return nullptr;
}

// binary32 operands, general kernel
template <int NXK>
const void* f32in_ptr(bool vec) {
    return vec ? reinterpret_cast<const void*>(&tgemm_f32in_rs_kernel<kTy, NXK, true>)
               : reinterpret_cast<const void*>(&tgemm_f32in_rs_kernel<kTy, NXK, false>);
}

}  // namespace

template <>
const void* kernel_for<TG_AB, TG_CT, (TG_EPI != 0)>(const Plan& pl) {
    const bool nxk = (pl.variant & kLayoutNxK) != 0;
    const bool vec = (pl.variant & kVecAB) != 0;
    if constexpr (TG_AB == 2) {
        // binary32 operands: the direct-to-LDS kernel, or the general one
        if (pl.variant & kDma)
            return pl.producers ? nullptr : (nxk ? f32_dma_ptr<1>(pl.stages, pl.bm) : f32_dma_ptr<0>(pl.stages, pl.bm));
        return nxk ? f32in_ptr<1>(vec) : f32in_ptr<0>(vec);
    } else {
        if (pl.variant & kDma)
            return nxk ? dma_ptr<1>(pl.k_step, pl.stages, pl.bm, pl.producers, pl.c_stream)
                       : dma_ptr<0>(pl.k_step, pl.stages, pl.bm, pl.producers, pl.c_stream);
        return nxk ? rs_ptr<1>(vec) : rs_ptr<0>(vec);
    }
}

}  // namespace tg
