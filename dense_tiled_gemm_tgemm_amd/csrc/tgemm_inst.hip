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
// steps; the other combinations the default depth only
constexpr bool kAllDepths = (kTy == ty_code(0, 0, false));

template <int NXK>
const void* dma_ptr(int k_step, int stages) {
    if (k_step == 64) return reinterpret_cast<const void*>(&tgemm_dma_kernel<kTy, NXK, 64, 2>);
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
static_assert(kDefaultDmaStages32 == 4, "the default ring depth is instantiated for every combination");

template <int NXK>
const void* rs_ptr(bool vec) {
    return vec ? reinterpret_cast<const void*>(&tgemm_rs_kernel<kTy, NXK, true>)
               : reinterpret_cast<const void*>(&tgemm_rs_kernel<kTy, NXK, false>);
}

template <int NXK>
const void* f32in_ptr(bool pipelined, bool vec) {
    if (pipelined) return reinterpret_cast<const void*>(&tgemm_f32in_kernel<kTy, NXK>);
    return vec ? reinterpret_cast<const void*>(&tgemm_f32in_rs_kernel<kTy, NXK, true>)
               : reinterpret_cast<const void*>(&tgemm_f32in_rs_kernel<kTy, NXK, false>);
}

}  // namespace

template <>
const void* kernel_for<TG_AB, TG_CT, (TG_EPI != 0)>(const Plan& pl) {
    const bool nxk = (pl.variant & kLayoutNxK) != 0;
    const bool vec = (pl.variant & kVecAB) != 0;
    if constexpr (TG_AB == 2) {
        // binary32 operands: the pipelined kernel, or the general one
        const bool pipelined = (pl.variant & kDma) != 0;
        return nxk ? f32in_ptr<1>(pipelined, vec) : f32in_ptr<0>(pipelined, vec);
    } else {
        if (pl.variant & kDma) return nxk ? dma_ptr<1>(pl.k_step, pl.stages) : dma_ptr<0>(pl.k_step, pl.stages);
        return nxk ? rs_ptr<1>(vec) : rs_ptr<0>(vec);
    }
}

}  // namespace tg
