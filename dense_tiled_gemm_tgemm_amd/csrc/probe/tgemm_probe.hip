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
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
    [[maybe_unused]] const unsigned voff = (unsigned)tid * 16u;
    [[maybe_unused]] const unsigned smask = data_bytes - 65536u;                     // 64 KiB-aligned windows inside the data
    [[maybe_unused]] unsigned soff = (unsigned)blockIdx.x * 65536u;
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


// ---------------------------------------------------------------------------
// Instruction-stream probes (tgemm_mfma_stream_probe): the GEMM's steady-state
// instruction stream taken apart, to see what each part costs the matrix
// cores on this board. Common to all: workgroups of 256 threads (one wave per
// SIMD) or 512 (two per SIMD); per round the work of one 64-deep step of a
// 256 x 256 tile (2^23 flops per workgroup; the binary32 kind half of that);
// fragments read from LDS as in the GEMM; loads from 4 KiB windows that four
// workgroups of one die share per round (8 KiB for 512 threads), as the
// GEMM's concurrently running tiles share panels in L2; shader-clock and
// reference-time stamps around the rounds.
// ---------------------------------------------------------------------------

constexpr unsigned kWaitVm0 = (0) | (7 << 4) | (15 << 8) | (0 << 14);    // s_waitcnt vmcnt(0)
constexpr unsigned kWaitLgkm0 = (15) | (7 << 4) | (0 << 8) | (3 << 14);  // s_waitcnt lgkmcnt(0)

__device__ __forceinline__ void fill_lds(u32x4* sm, const uint16_t* data, unsigned data_bytes, int nthreads) {
    const u32x4* dv = reinterpret_cast<const u32x4*>(data);
    const unsigned dmask = (data_bytes >> 4) - 1u;
    for (int i = threadIdx.x; i < kChunks; i += nthreads)
        sm[i] = dv[((unsigned)blockIdx.x * kChunks + (unsigned)i) & dmask];
    __syncthreads();
}

// first byte of this workgroup's load window in round 0: four workgroups of
// a die (equal w mod 8, consecutive w / 8) share one 64 KiB-spaced window
__device__ __forceinline__ unsigned window0() {
    const unsigned w = blockIdx.x;
    return ((w & 7u) * 8u + ((w >> 3) & 31u) / 4u) * 65536u;
}

__device__ __forceinline__ void stamp(uint64_t* clocks, uint64_t t0, uint64_t r0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (clocks && threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// 16x16x32 fp16, 8 x 8 blocks per wave, two 32-deep slices per round, blocks
// in serpentine order. READS: 16 fragment reads per slice (after the even
// MFMAs) into the buffer the next slice uses. LOADS, after every fourth MFMA
// of the second slice: 1 = 16 direct-to-LDS loads, 2 = 8 of them (every
// eighth), 3 = 16 loads into registers (each written back once a round
// later, by an empty asm that reads them), 4 = 16 ds_write_b128 of register
// values (no global load). WAIT: vmcnt(0), then (BAR) lgkmcnt(0) and a
// workgroup barrier, before the second slice (the GEMM's step boundary).
template <bool READS, int LOADS, bool BAR>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
stream16_kernel(const uint16_t* data, unsigned data_bytes, float* out, uint64_t* clocks, int iters) {
    __shared__ u32x4 sm[kChunks];
    fill_lds(sm, data, data_bytes, 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    half8 fa[2][8], fb[2][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fa[0][i] = __builtin_bit_cast(half8, sm[lane + 64 * i + 1024 * wave]);
        fb[0][i] = __builtin_bit_cast(half8, sm[lane + 64 * (i + 8) + 1024 * wave]);
        fa[1][i] = __builtin_bit_cast(half8, sm[lane + 64 * i + 1024 * wave + 16]);
        fb[1][i] = __builtin_bit_cast(half8, sm[lane + 64 * (i + 8) + 1024 * wave + 16]);
    }
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
    u32x4 stg[16];
#pragma unroll
    for (int l = 0; l < 16; ++l) stg[l] = LOADS == 4 ? sm[lane + 64 * l] : u32x4{};
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)data, 0, (int)data_bytes, 0x00020000);
#endif
    [[maybe_unused]] const unsigned voff = (unsigned)tid * 16u;
    [[maybe_unused]] const unsigned wmask = data_bytes - 4096u;
    [[maybe_unused]] unsigned soff = window0();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h == 1 && (LOADS == 1 || LOADS == 2)) {
                if (BAR) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                if (BAR) __builtin_amdgcn_s_barrier();
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < 64; ++q) {
                const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
                if (READS && (q & 1) == 0 && (q >> 1) < 16) {
                    const int r = q >> 1;
                    half8& d = (r & 1) ? fb[h ^ 1][r >> 1] : fa[h ^ 1][r >> 1];
                    d = __builtin_bit_cast(half8, sm[lane + 64 * r + 1024 * wave + 16 * (it & 3)]);
                } else if (LOADS && h == 1 && (q & 3) == 3 && (LOADS != 2 || (q & 7) == 7)) {
                    const int l = q >> 2;
                    [[maybe_unused]] const unsigned so = (soff + (unsigned)l * 4096u) & wmask;
                    if (LOADS == 1 || LOADS == 2) {
#if defined(__HIP_DEVICE_COMPILE__)
                        u32x4* dst = sm + 4096 + (l * 4 + wave) * 64;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff, so, 0, 0);
#endif
                    } else if (LOADS == 3) {
#if defined(__HIP_DEVICE_COMPILE__)
                        __asm__ __volatile__("" ::"v"(stg[l]));
                        stg[l] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)so, 0));
#endif
                    } else {
                        sm[4096 + (l * 4 + wave) * 64 + lane] = stg[l];
                    }
                }
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        soff += 64u * 65536u;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stamp(clocks, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[i][j][e];
#pragma unroll
    for (int l = 0; l < 16; ++l) s += __builtin_bit_cast(float, stg[l][0] & 0x3f800000u);
    out[blockIdx.x * 256 + tid] = s;
}

// 32x32x16 fp16, 4 x 4 blocks per wave (the same 128 x 128), two 32-deep
// slices of 32 MFMAs per round; GEMM: the 16 reads per slice (one after each
// of its first 16 MFMAs) and the loads and waits of stream16_kernel<true, 1, true>.
template <bool GEMM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
stream32x32_kernel(const uint16_t* data, unsigned data_bytes, float* out, uint64_t* clocks, int iters) {
    __shared__ u32x4 sm[kChunks];
    fill_lds(sm, data, data_bytes, 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    half8 fa[2][2][4], fb[2][2][4];     // [buffer][16-deep half][block]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[b][k][i] = __builtin_bit_cast(half8, sm[lane + 64 * (4 * k + i) + 1024 * wave + 16 * b]);
                fb[b][k][i] = __builtin_bit_cast(half8, sm[lane + 64 * (8 + 4 * k + i) + 1024 * wave + 16 * b]);
            }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)data, 0, (int)data_bytes, 0x00020000);
#endif
    [[maybe_unused]] const unsigned voff = (unsigned)tid * 16u;
    [[maybe_unused]] const unsigned wmask = data_bytes - 4096u;
    [[maybe_unused]] unsigned soff = window0();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (GEMM && h == 1) {
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                __builtin_amdgcn_s_barrier();
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                const int k = q >> 4, x = q & 15, i = x >> 2, j = (i & 1) ? 3 - (x & 3) : (x & 3);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[h][k][j], fa[h][k][i], acc[i][j], 0, 0, 0);
                if (GEMM && q < 16) {
                    half8& d = (q & 1) ? fb[h ^ 1][q >> 3][(q >> 1) & 3] : fa[h ^ 1][q >> 3][(q >> 1) & 3];
                    d = __builtin_bit_cast(half8, sm[lane + 64 * q + 1024 * wave + 16 * (it & 3)]);
                }
                if (GEMM && h == 1 && (q & 1) == 1) {
#if defined(__HIP_DEVICE_COMPILE__)
                    const int l = q >> 1;
                    u32x4* dst = sm + 4096 + (l * 4 + wave) * 64;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff,
                                                             (soff + (unsigned)l * 4096u) & wmask, 0, 0);
#endif
                }
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        soff += 64u * 65536u;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stamp(clocks, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[i][j][e];
    out[blockIdx.x * 256 + tid] = s;
}

// 16x16x32 fp16 with 8 waves of 64 x 128 (two per SIMD, 4 x 8 blocks each),
// the same 256 x 256 tile: two 32-deep slices of 32 MFMAs per round. GEMM:
// 12 fragment reads per slice, 8 direct-to-LDS loads per wave in the second
// slice (the workgroup's 64 KiB per step), waits and barrier before it.
template <bool GEMM>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
stream8w_kernel(const uint16_t* data, unsigned data_bytes, float* out, uint64_t* clocks, int iters) {
    __shared__ u32x4 sm[kChunks];
    fill_lds(sm, data, data_bytes, 512);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    half8 fa[2][4], fb[2][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[0][i] = __builtin_bit_cast(half8, sm[lane + 64 * i + 1024 * (wave & 3)]);
        fa[1][i] = __builtin_bit_cast(half8, sm[lane + 64 * i + 1024 * (wave & 3) + 16]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        fb[0][j] = __builtin_bit_cast(half8, sm[lane + 64 * (4 + j) + 1024 * (wave & 3)]);
        fb[1][j] = __builtin_bit_cast(half8, sm[lane + 64 * (4 + j) + 1024 * (wave & 3) + 16]);
    }
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)data, 0, (int)data_bytes, 0x00020000);
#endif
    [[maybe_unused]] const unsigned voff = (unsigned)tid * 16u;
    [[maybe_unused]] const unsigned wmask = data_bytes - 8192u;          // 8 KiB windows: 512 threads x 16 bytes
    [[maybe_unused]] unsigned soff = window0();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (GEMM && h == 1) {
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                __builtin_amdgcn_s_barrier();
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
                if (GEMM && (q & 1) == 0 && (q >> 1) < 12) {
                    const int r = q >> 1;
                    half8& d = r < 4 ? fa[h ^ 1][r] : fb[h ^ 1][r - 4];
                    d = __builtin_bit_cast(half8, sm[lane + 64 * r + 1024 * (wave & 3) + 16 * (it & 3)]);
                } else if (GEMM && h == 1 && (q & 3) == 3) {
#if defined(__HIP_DEVICE_COMPILE__)
                    const int l = q >> 2;
                    u32x4* dst = sm + 4096 + (l * 8 + wave) * 64;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff,
                                                             (soff + (unsigned)l * 8192u) & wmask, 0, 0);
#endif
                }
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        soff += 64u * 65536u;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    stamp(clocks, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[i][j][e];
    out[blockIdx.x * 512 + tid] = s;
}

// 16x16x4 binary32, 8 x 8 blocks per wave, 16-byte fragments (4 consecutive
// k per lane), the binary32 GEMM's order: per 16-deep slice each block's four
// MFMAs back to back on its accumulator, 16 fragment reads spread over the
// slice; two slices per round (2^22 flops per workgroup).
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
stream_f32_kernel(const uint16_t* data, unsigned data_bytes, float* out, uint64_t* clocks, int iters) {
    __shared__ u32x4 sm[kChunks];
    fill_lds(sm, data, data_bytes, 256);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    f32x4 fa[2][8], fb[2][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        fa[0][i] = __builtin_bit_cast(f32x4, sm[lane + 64 * i + 1024 * wave]);
        fb[0][i] = __builtin_bit_cast(f32x4, sm[lane + 64 * (i + 8) + 1024 * wave]);
        fa[1][i] = fa[0][i];
        fb[1][i] = fb[0][i];
    }
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(0.0f, 0.0f, f32x4{}, 0, 0, 0);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int q = 0; q < 64; ++q) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 4 * q + e;
                    const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[h][j][e], fa[h][i][e], acc[i][j], 0, 0, 0);
                    if ((m & 15) == 15) {
                        const int r = m >> 4;
                        f32x4& d = (r & 1) ? fb[h ^ 1][r >> 1] : fa[h ^ 1][r >> 1];
                        d = __builtin_bit_cast(f32x4, sm[lane + 64 * r + 1024 * wave + 16 * (it & 3)]);
                    }
                    __asm__ __volatile__("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    stamp(clocks, t0, r0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[i][j][e];
    out[blockIdx.x * 256 + tid] = s;
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

extern "C" int tgemm_mfma_stream_probe(int kind, int64_t workgroups, int iters, const void* data,
                                       int64_t data_bytes, float* out, uint64_t* clocks, void* stream) {
    if (workgroups <= 0 || workgroups > 65536 || iters <= 0 || !out || !data) return TGEMM_ERR_INVALID;
    if (data_bytes < (1 << 20) || data_bytes > (1ll << 30) || (data_bytes & (data_bytes - 1)) != 0)
        return TGEMM_ERR_INVALID;
    if ((uintptr_t)data % 16 != 0) return TGEMM_ERR_INVALID;
    using namespace tg_probe;
    const void* k = nullptr;
    unsigned threads = 256;
    switch (kind) {
        case TGEMM_STREAM_F16_MFMA: k = reinterpret_cast<const void*>(&stream16_kernel<false, 0, false>); break;
        case TGEMM_STREAM_F16_READS: k = reinterpret_cast<const void*>(&stream16_kernel<true, 0, false>); break;
        case TGEMM_STREAM_F16_GEMM: k = reinterpret_cast<const void*>(&stream16_kernel<true, 1, true>); break;
        case TGEMM_STREAM_F16_GEMM_NO_BARRIER:
            k = reinterpret_cast<const void*>(&stream16_kernel<true, 1, false>);
            break;
        case TGEMM_STREAM_F16_HALF_LOADS: k = reinterpret_cast<const void*>(&stream16_kernel<true, 2, true>); break;
        case TGEMM_STREAM_F16_VGPR_LOADS: k = reinterpret_cast<const void*>(&stream16_kernel<true, 3, false>); break;
        case TGEMM_STREAM_F16_LDS_WRITES: k = reinterpret_cast<const void*>(&stream16_kernel<true, 4, false>); break;
        case TGEMM_STREAM_F16_32X32: k = reinterpret_cast<const void*>(&stream32x32_kernel<false>); break;
        case TGEMM_STREAM_F16_32X32_GEMM: k = reinterpret_cast<const void*>(&stream32x32_kernel<true>); break;
        case TGEMM_STREAM_F16_8W_MFMA:
            k = reinterpret_cast<const void*>(&stream8w_kernel<false>);
            threads = 512;
            break;
        case TGEMM_STREAM_F16_8W_GEMM:
            k = reinterpret_cast<const void*>(&stream8w_kernel<true>);
            threads = 512;
            break;
        case TGEMM_STREAM_F32_GEMM: k = reinterpret_cast<const void*>(&stream_f32_kernel); break;
        default: return TGEMM_ERR_INVALID;
    }
    const uint16_t* d = static_cast<const uint16_t*>(data);
    unsigned nb = (unsigned)data_bytes;
    void* kargs[] = {&d, &nb, &out, &clocks, &iters};
    const hipError_t e = hipLaunchKernel(k, dim3((unsigned)workgroups), dim3(threads), kargs, 0,
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
