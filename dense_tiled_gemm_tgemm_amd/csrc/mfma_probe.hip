// Matrix-core issue probe: the GEMM kernel's MFMA stream without its memory
// traffic. Each wave (one per SIMD, as in the GEMM) runs `iters` rounds of
// 16 independent v_mfma_f32_32x32x16_f16 on register-resident binary16
// fragments whose bit patterns look like the benchmark's inputs (random sign
// and mantissa, magnitudes 2^-6 .. 2^-3). It measures what the matrix cores
// of this board sustain for such data; the result is written only so the
// work is not optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm.h"

namespace tg_probe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float acc16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ half8 pseudo_random_half8(unsigned s) {
    half8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s ^= s >> 13;
        s *= 0x5bd1e995u;
        s ^= s >> 15;
        const unsigned bits = ((s & 1u) << 15) | ((9u + ((s >> 1) & 3u)) << 10) | ((s >> 3) & 1023u);
        h[e] = __builtin_bit_cast(_Float16, (uint16_t)bits);
    }
    return h;
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_issue_kernel(float* out, int iters) {
    const unsigned t = threadIdx.x + blockIdx.x * 256u;
    half8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = pseudo_random_half8(t * 8u + i);
        b[i] = pseudo_random_half8(t * 8u + 4u + i);
    }
    acc16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = acc16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
    out[t] = sum;
}

}  // namespace tg_probe

extern "C" int tgemm_mfma_issue_probe(int64_t workgroups, int iters, float* out, void* stream) {
    if (workgroups <= 0 || workgroups > 65536 || iters <= 0 || !out) return TGEMM_ERR_INVALID;
    void* kargs[] = {&out, &iters};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&tg_probe::mfma_issue_kernel),
                                         dim3((unsigned)workgroups), dim3(256), kargs, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}
