// Measurement aids (not part of the product operation), built as a library
// of their own (libtgemm_probe.so, include/tgemm_probe.h).
//
// Matrix-core ceiling probe: the GEMM kernel's instruction stream without its
// synchronization, tile changes or C stores. Each wave (one per SIMD, as in
// the GEMM) runs `iters` rounds of two 64-instruction slices of independent
// v_mfma_f32_16x16x32_f16 on 8 x 8 accumulator blocks. After every even MFMA
// it reads one 128-bit fragment from LDS into the buffer the next slice
// consumes (16 reads per slice, as the GEMM does for B stored N x K), and
// after every eighth odd MFMA it issues one 16-byte-per-lane direct-to-LDS
// buffer load (8 per slice, the GEMM's 64-deep steps), waiting for its loads
// once per round. The operands come from `data` (binary16 values the caller
// chooses, such as the benchmark's inputs), so the matrix cores see fresh
// values every slice, as in the GEMM: MI355X is power-limited under MFMA load
// and the switching activity of the operands sets the clock. The result is
// written only so that the work is not optimized away.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm.h"
#include "tgemm_probe.h"

namespace tg_probe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS: chunks [0, 4096) are read as fragments, [4096, 8192) receive the loads.
constexpr int kChunks = 8192;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_ceiling_kernel(const uint16_t* data, unsigned data_bytes, float* out, uint64_t* clocks, int iters) {
    __shared__ u32x4 sm[kChunks];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const u32x4* dv = reinterpret_cast<const u32x4*>(data);
    const unsigned dmask = (data_bytes >> 4) - 1u;                 // data_bytes is a power of two
    for (int i = tid; i < kChunks; i += 256) sm[i] = dv[((unsigned)blockIdx.x * kChunks + (unsigned)i) & dmask];
    __syncthreads();
    half8 fa[2][8], fb[2][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fa[0][i] = __builtin_bit_cast(half8, sm[lane + 64 * i + 1024 * wave]);
        fb[0][i] = __builtin_bit_cast(half8, sm[lane + 64 * (i + 8) + 1024 * wave]);
        fa[1][i] = fa[0][i];
        fb[1][i] = fb[0][i];
    }
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)data, 0, (int)data_bytes, 0x00020000);
#endif
    const unsigned voff = (unsigned)tid * 16u;
    const unsigned smask = data_bytes - 65536u;                     // 64 KiB-aligned windows inside the data
    unsigned soff = (unsigned)blockIdx.x * 65536u;
    // shader clock and 100 MHz reference time at the start of the rounds
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int q = 0; q < 64; ++q) {
                const int i = q >> 3, j = q & 7;
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
                if ((q & 1) == 0) {
                    const int r = q >> 1;
                    if (r < 16) {
                        half8& d = (r & 1) ? fb[h ^ 1][r >> 1] : fa[h ^ 1][r >> 1];
                        d = __builtin_bit_cast(half8, sm[lane + 64 * r + 1024 * wave + 16 * (it & 3)]);
                    }
                } else if ((q & 7) == 7) {
#if defined(__HIP_DEVICE_COMPILE__)
                    const int l = q >> 3;
                    u32x4* dst = sm + 4096 + (l * 4 + wave) * 64;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff,
                                                             (soff + (unsigned)l * 4096u) & smask, 0, 0);
#endif
                }
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8) | (0 << 14));   // this wave's loads landed
        soff += 262144u;
    }
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8) | (0 << 14));
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (clocks && tid == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[i][j][e];
    out[blockIdx.x * 256 + tid] = s;
}

// Die probe: the first thread of each workgroup records the number of the
// accelerator die (XCD) it runs on, read from the XCC_ID hardware register
// (bits 3:0). The die-aware raster assumes that the dispatcher deals
// workgroups to the dies in turn, so that those sharing a die are the ones
// with equal w mod 8; this shows what the hardware does.
__global__ void __launch_bounds__(64) xcd_id_kernel(int* out, int64_t n) {
    const int64_t w = blockIdx.x;
    if (threadIdx.x == 0 && w < n) {
#if defined(__HIP_DEVICE_COMPILE__)
        // s_getreg_b32 hwreg(HW_REG_XCC_ID, 0, 4): register 20, offset 0, width 4
        out[w] = (int)__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11));
#endif
    }
}

}  // namespace tg_probe

extern "C" int tgemm_mfma_issue_probe(int64_t workgroups, int iters, const void* data, int64_t data_bytes,
                                      float* out, uint64_t* clocks, void* stream) {
    if (workgroups <= 0 || workgroups > 65536 || iters <= 0 || !out || !data) return TGEMM_ERR_INVALID;
    if (data_bytes < (1 << 20) || data_bytes > (1ll << 30) || (data_bytes & (data_bytes - 1)) != 0)
        return TGEMM_ERR_INVALID;
    if ((uintptr_t)data % 16 != 0) return TGEMM_ERR_INVALID;
    const uint16_t* d = static_cast<const uint16_t*>(data);
    unsigned nb = (unsigned)data_bytes;
    void* kargs[] = {&d, &nb, &out, &clocks, &iters};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&tg_probe::mfma_ceiling_kernel),
                                         dim3((unsigned)workgroups), dim3(256), kargs, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

extern "C" int tgemm_xcd_probe(int64_t workgroups, int* out, void* stream) {
    if (workgroups <= 0 || workgroups > (1 << 20) || !out) return TGEMM_ERR_INVALID;
    int64_t n = workgroups;
    void* kargs[] = {&out, &n};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&tg_probe::xcd_id_kernel),
                                         dim3((unsigned)workgroups), dim3(64), kargs, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}
