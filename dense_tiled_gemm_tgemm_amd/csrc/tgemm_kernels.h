// Device code of the dense tiled GEMM for MI355X (gfx950):
// C = act(alpha * A * B + bias), binary16, bfloat16 or binary32 in, fp32
// accumulate, binary16, bfloat16 or fp32 out (the plain product is alpha = 1,
// no bias, no activation). Included by the translation units that
// instantiate the kernels, one per (input type, output type).
//
// One workgroup owns one BM x BN output tile and walks K in steps (page 1,
// "Using NVIDIA CUDA Tile to write a high-performance matrix multiply",
// sections 1-6; page 4, CUDA programming guide 13.4.2, section 2.4.9.1).
// Per K step the tile's A and B blocks are staged from HBM/L2 into LDS while
// earlier steps run on the matrix cores (the load / barrier / compute /
// overlap / write-back lifecycle of page 3, "Why GEMM", section 2.2).
// Partial K tiles are padded with zeros and C elements outside M x N are
// never written (page 4, section 2.4.6.1.3).
//
// gfx950 mapping:
//  * 256 threads = 4 waves of 64 lanes in a 2 x 2 grid; each wave owns a
//    128 x 128 sub-tile held as 8 x 8 blocks of 16 x 16 fp32 accumulators
//    (256 accumulator registers per lane).
//  * Inner product: v_mfma_f32_16x16x32_f16 (bf16 for bfloat16 inputs), one
//    per 16 x 16 block and 32-deep K slice. Each lane supplies 8 consecutive-k
//    16-bit values of
//    one row of each operand (row = lane mod 16, k = 8 * (lane / 16) + 0..7),
//    read from LDS as one 128-bit word. The B fragment is passed as the
//    instruction's first operand and the A fragment as its second, so the
//    16 x 16 result block is C transposed: lane l holds C row (l mod 16) and
//    its four accumulator registers hold the four consecutive C columns
//    4 * (l / 16) + 0..3.
//    (This shape keeps the matrix cores busier between the interleaved LDS
//    and load instructions than the 32 x 32 x 16 one, which needs twice the
//    cycles per instruction but issues less evenly.)
//  * Every path multiplies the same operand values in the same 32-deep K
//    slices in ascending order, so all of them produce the same bits.
//  * Binary32 operands run on the direct-to-LDS kernel as pairs of 16-bit
//    units (K and the strides doubled): a 32-unit step is 16 floats, a
//    128-bit A (and N x K B) fragment 4 consecutive-k floats, a K x N B kept
//    [k][n] (F32KnLds) and read as four floats, and each block takes four
//    v_mfma_f32_16x16x4_f32 (slice()). The k each instruction and lane sums
//    are those of the binary32 general kernel below, so both binary32 paths
//    produce the same bits too.
//  * Workgroup -> tile: die-aware renumbering, then the grouped order of
//    page 1, section "Swizzle" (tile_of in tgemm_plan.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm.h"
#include "tgemm_plan.h"

namespace tg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Kernel type code TY: input type (bit 0: bfloat16, bit 4: binary32, neither:
// binary16), output type (bits 1-2: 0 binary16, 1 bfloat16, 2 fp32),
// epilogue (bit 3: scale, bias and activation applied; clear: the sums are
// stored as they are).
constexpr int ty_code(int ab, int ct, bool epi) {
    return (ab == 1 ? 1 : 0) | (ct << 1) | (epi ? 8 : 0) | (ab == 2 ? 16 : 0);
}
constexpr int ab_of(int ty) { return (ty & 16) ? 2 : (ty & 1); }
constexpr int ct_of(int ty) { return (ty >> 1) & 3; }
constexpr bool epi_of(int ty) { return (ty & 8) != 0; }

static_assert(BM == 256 && BN == 256 && BK == 64 && NTHREADS == 256,
              "the staging maps below assume a 256 x 256 tile, 64-deep register staging and 256 threads");

struct Args {
    const uint16_t* A;
    const uint16_t* B;
    void* C;              // binary16 / bfloat16 bits or fp32 (output type of the kernel)
    const float* bias;    // N values, or null (epilogue kernels only)
    float alpha;          // scale of the sums (epilogue kernels only)
    int relu;             // 1: negative results stored as zero (epilogue kernels only)
    int64_t lda, ldb, ldc;
    int M, N, K;
    int grid_m, grid_n, W, group_m, num_xcd;
    int grid;             // workgroups launched; workgroup b computes tiles b, b + grid, ...
    int c16;              // 16-byte C stores (any alignment): every offset in a wave's rows below 2^31
    int c8;               // the same for 8 bytes
    int c_stream;         // 1: C rows 128-byte aligned, 16-byte stores streamed (nt sc1); 0: default policy
};

// LDS layout of one staged K-contiguous operand block (256 rows x KS halves)
// as 16-byte chunks, CPR = KS / 8 per row, chunk c of row r at slot
// r * CPR + (c ^ f(r)):
//   KS = 64: f(r) = r & 7
//   KS = 32: f(r) = (r >> 1) & 3
// A fragment read takes 16 consecutive rows at one chunk per 16-lane group
// (4 groups = 4 consecutive chunks). The direct-to-LDS loads write each
// instruction's 1 KiB linearly, so only the reads can collide. Measured on
// gfx950 (LDS conflict counters of a read-only probe): both maps serve each
// 16-byte read in 4 LDS cycles, the rate of a plain linear read, while the
// earlier maps (r & 7) ^ ((r >> 3) & 1) and (r ^ (r >> 2)) & 3, conflict-free
// on paper for 16-lane groups, took 8 (page 3, sections 3.1 and 5.3; page 5,
// "Why swizzle matters"). Both maps depend on r mod 16 only, so the fragment
// of 16-row block i sits 16 * CPR slots after that of block 0.
template <int KS>
struct Lds {
    static constexpr int kCpr = KS / 8;
    static constexpr int kBlock = 256 * kCpr;          // chunks per operand block
    static constexpr int kStage = 2 * kBlock;          // A block then B block
    __device__ static __forceinline__ int swz(int r) {
        return KS == 64 ? (r & 7) : ((r >> 1) & 3);
    }
    __device__ static __forceinline__ int slot(int r, int c) { return r * kCpr + (c ^ swz(r)); }
};

// Fragment of the 16-row block `blk` of a K-contiguous LDS block for the
// 32-deep slice `s`: lane l gets row 16 * blk + (l mod 16) of the wave's
// 128-row half `half`, k = 32 s + 8 (l / 16) + 0..7.
template <int KS>
__device__ __forceinline__ half8 read_kc(const u32x4* __restrict__ s_blk, int half, int blk, int lane, int s) {
    return __builtin_bit_cast(half8, s_blk[Lds<KS>::slot(half * 128 + blk * 16 + (lane & 15), s * 4 + (lane >> 4))]);
}

// Eight binary16 values from p[0..nv-1]; lanes at or past nv read as zero.
__device__ __forceinline__ u32x4 load8_elems(const uint16_t* __restrict__ p, int nv) {
    unsigned w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const unsigned lo = (2 * q < nv) ? (unsigned)p[2 * q] : 0u;
        const unsigned hi = (2 * q + 1 < nv) ? (unsigned)p[2 * q + 1] : 0u;
        w[q] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Fragments are carried as 8 x 16-bit bit patterns; AB selects how the
// matrix core reads them (16-bit types; slice() takes binary32 fragments
// apart into four v_mfma_f32_16x16x4_f32).
template <int AB>
__device__ __forceinline__ f32x4 mfma16(const half8& b, const half8& a, const f32x4& c) {
    static_assert(AB == 0 || AB == 1, "16-bit operand types");
    if constexpr (AB == 0)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                       c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> two 16-bit outputs packed in one word, round to nearest even (page
// 1, section 6: the fp32 accumulator is converted to C's type when it is
// stored); one packed conversion instruction for either type.
template <int CT>
__device__ __forceinline__ unsigned pack2(float a, float b) {
    if constexpr (CT == 0)
        return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, half2));
    else
        return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Epilogue of one sum x in fp32: alpha * x + bias as one fused multiply-add
// (one rounding), then the rectifier (a NaN passes through, as it compares
// false). Without the epilogue the sum is stored as it is.
template <bool EPI>
__device__ __forceinline__ float epi(float x, float alpha, float b, bool relu) {
    if constexpr (!EPI) {
        return x;
    } else {
        const float v = __builtin_fmaf(alpha, x, b);
        return (relu && v < 0.f) ? 0.f : v;
    }
}

// Bias values of this lane's 32 columns (column n0 + 128 wn + 16 j + 4 (l / 16)
// + e in bv[j][e]); zeros past N or without a bias.
template <int NJ>
__device__ __forceinline__ void load_bias(float (&bv)[NJ][4], const Args& a, int n0, int wn, int lane) {
    const int colb = n0 + wn * 16 * NJ + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = colb + 16 * j + e;
            bv[j][e] = (a.bias && col < a.N) ? a.bias[col] : 0.f;
        }
}

// 16-byte C stores go through a buffer resource over the wave's 128 C rows
// (the host keeps this path only where every byte offset in those rows fits
// in 31 bits). Where C's rows are 128-byte aligned (base and row pitch) they
// use the streaming policy nt sc1: C is written once and never read back,
// every workgroup stores its tile at about the same time, and whole lines
// drain faster when they bypass the caches' normal replacement (8192^3:
// 1.8% against the default policy with a 16-bit C, 2.8% with an fp32 C).
// Rows at any other alignment split their 128-byte pieces over two lines,
// which streamed stores then write as partial lines; there the default
// (write-back) policy is faster, as the L2 merges the halves: 3001 x 5003 x
// 4099 (2-byte-aligned rows) 121.9 -> 116.8 us with a 16-bit C and 142.2 ->
// 118.3 with an fp32 C; 8192 x 12288 x 4096 with ldc 12289 648.7 -> 636.4
// and 728.8 -> 628.9. The persistent 64-deep kernel is built once per policy
// (the host picks by C's alignment); elsewhere the choice is a uniform flag
// (Args::c_stream), one scalar branch per store.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t BufRsrc;
#else
typedef int BufRsrc;                                  // host pass: never used
#endif
constexpr int kCStorePolicy = 2 | 16;                 // nt | sc1

__device__ __forceinline__ BufRsrc c_rows_rsrc(void* C, int64_t byte_offset) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(C) + byte_offset, 0, 0x7fffffff, 0x00020000);
#else
    (void)C; (void)byte_offset;
    return 0;
#endif
}

__device__ __forceinline__ void store16_c(const u32x4& v, const BufRsrc& r, int64_t byte_offset, bool stream) {
#if defined(__HIP_DEVICE_COMPILE__)
    if (stream)
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_offset, 0, kCStorePolicy);
    else
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_offset, 0, 0);
#else
    (void)v; (void)r; (void)byte_offset; (void)stream;
#endif
}

// A 16-byte store that only lanes with `ok` perform, without a branch: the
// other lanes present an offset at or beyond the resource's record count
// (0x7fffffff), which the hardware drops. The empty asm hands the selected
// offset to the store as it is, so no constant part of it is moved into the
// instruction's immediate offset (which would shift the dropped lanes' offset
// back into range).
constexpr unsigned kCOob = 0x80000000u;
__device__ __forceinline__ void store16_lanes(const u32x4& v, const BufRsrc& r, bool ok, int64_t byte_offset,
                                              bool stream) {
    unsigned o = ok ? (unsigned)byte_offset : kCOob;
    asm volatile("" : "+v"(o));
    store16_c(v, r, (int)o, stream);
}

// Lane l of wave (wm, wn) holds, in acc[i][j], C row m0 + 16 NI wm + 16 i + (l mod 16)
// at columns n0 + 16 NJ wn + 16 j + 4 (l / 16) + 0..3 (NI = 8 row blocks and
// NJ = 8 column blocks per wave; NI = 4 or 2 in the smaller tiles, NJ = 4 in
// the two-workgroups-per-unit binary32 kernel).
//  * 16-bit outputs: for each pair of 16-column blocks (j, j+1),
//    v_permlane16_swap exchanges the converted words between 16-lane rows so
//    that a lane in row g then holds the 8 consecutive columns
//    16 (j + (g & 1)) + 8 (g >> 1) .. +7 of its C row; a DPP rotation then
//    trades such 16-byte pieces between lanes l and l + 8 of each 16-lane row,
//    so that each store instruction writes 8 rows x 128 contiguous bytes
//    rather than 16 rows x 64 (3001 x 5003 x 4099, rows 2-byte aligned:
//    132.9 -> 125.1 us; no change at the aligned workloads). One 16-byte
//    store per lane at whatever alignment the row has (gfx950 buffer stores
//    accept unaligned addresses; against element stores for 2-byte-aligned
//    rows, 140.2 -> 130.8 us on the same workload); element stores where the
//    8 columns straddle N, and 8-byte or element stores when C's offsets
//    exceed 31 bits.
//  * fp32 output: each block's four columns are 16 contiguous bytes of the
//    lane's row; the same DPP trade between lanes l and l + 8 over pairs of
//    blocks makes each store instruction write 8 rows x 128 bytes, element
//    stores where the four columns straddle N (an 8-byte path here made the
//    register allocator move the accumulators around in the main loop of the
//    binary32-operand kernel).
// All lanes run the exchange; only the stores are predicated: the 16-byte store
// on its own condition, the 8-byte and element stores behind one uniform test
// (`whole`: the wave's rows lie inside C and its columns end at or before
// N, with 16-byte stores available), so an interior wave skips them with one scalar branch
// per store instead of a chain of exec-mask branches, which took longer than
// the conversions themselves. One 16-row block
// at a time (pinned), so the temporaries stay few when this runs between two
// tiles with the next tile's fragments already in registers. The 16-byte
// stores take the policy store16_c chooses from C's alignment; the 8-byte
// path is non-temporal.
// POL: 1 streamed stores, 0 default policy, -1 chosen at run time by a.c_stream.
template <int TY, int NJ = 8, int NI = 8, int POL = -1>
__device__ __forceinline__ void store_c(const f32x4 (&acc)[NI][NJ], const Args& a, int m0, int n0, int wm,
                                        int wn, int lane) {
    static_assert(NJ == 8 || NJ == 4, "a wave owns 8 or 4 blocks of 16 columns");
    static_assert(NI == 8 || NI == 4 || NI == 2 || NI == 1, "a wave owns 8, 4, 2 or 1 blocks of 16 rows");
    constexpr int kWr = 16 * NI;                      // C rows of a wave
    constexpr int CT = ct_of(TY);
    constexpr bool EPI = epi_of(TY);
    const int r16 = lane & 15, g = lane >> 4;
    const BufRsrc crs = c_rows_rsrc(a.C, (int64_t)(m0 + wm * kWr) * a.ldc * (CT == 2 ? 4 : 2));
    float bv[NJ][4];
    float alpha = 1.f;
    bool relu = false;
    if constexpr (EPI) {
        load_bias(bv, a, n0, wn, lane);
        alpha = a.alpha;
        relu = a.relu != 0;
    }
    const bool whole = __builtin_amdgcn_readfirstlane(
        (int)(a.c16 && m0 + wm * kWr + kWr <= a.M && n0 + wn * 16 * NJ + 16 * NJ <= a.N)) != 0;
    const bool stream = POL < 0 ? __builtin_amdgcn_readfirstlane(a.c_stream) != 0 : POL == 1;
    if constexpr (CT == 2) {
        // pairs (2q, 2q + 1) of 16-column blocks: lanes 8-15 of each 16-lane
        // row trade block 2q of their C row for block 2q + 1 of the row 8
        // above (DPP rotation by 8 inside the row), so that one store writes
        // rows 0-7 and the next rows 8-15 of the block, each row 32 contiguous
        // floats (128 bytes). A lane stores row rl (+ 8 h + 16 i) at columns
        // colq (+ 32 q); the row parts of the byte offsets are uniform.
        const bool hi = r16 >= 8;
        const int rl = r16 & 7;
        const int colq = n0 + wn * 16 * NJ + 4 * g + (hi ? 16 : 0);
        const int rowl = m0 + wm * kWr + rl;
        const int64_t lane_off = ((int64_t)rl * a.ldc + colq) * 4;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < NJ / 2; ++q) {
                u32x4 vs[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // the block's values enter vector registers here and not
                    // earlier: left to itself the compiler copied all 256
                    // accumulators out at the top of the store (ahead of the
                    // per-block branches), ran out of registers, and its spill
                    // code then stored one lane value from the wrong register
                    f32x4 x = acc[i][2 * q + h];
                    asm volatile("" : "+v"(x));
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = epi<EPI>(x[e], alpha, EPI ? bv[2 * q + h][e] : 0.f, relu);
                    vs[h] = __builtin_bit_cast(u32x4, v);
                }
                u32x4 d[2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned u = hi ? vs[0][e] : vs[1][e];
                    const unsigned w = (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0x128, 0xf, 0xf, false);
                    d[0][e] = hi ? w : vs[0][e];
                    d[1][e] = hi ? vs[1][e] : w;
                }
                const int col = colq + 32 * q;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ru = i * 16 + 8 * h;                 // uniform part of the row
                    const bool rok = rowl + ru < a.M;
                    const bool ok16 = rok & (col + 4 <= a.N) & (a.c16 != 0);
                    store16_lanes(d[h], crs, ok16, lane_off + 128 * q + (int64_t)ru * a.ldc * 4, stream);
                    if (__builtin_expect(!whole, 0)) {
                        asm volatile("");             // a scalar branch of its own, not merged into the lane mask
                        if (!ok16 && rok && col < a.N) {
                            float* dst = static_cast<float*>(a.C) + (int64_t)(rowl + ru) * a.ldc + col;
                            const f32x4 v = __builtin_bit_cast(f32x4, d[h]);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (col + e < a.N) dst[e] = v[e];
                        }
                    }
                }
            }
        }
    } else {
        // pairs (2q, 2q + 1) of 32-column groups: after the conversion,
        // lanes 8-15 of each 16-lane row trade group 2q of their C row for
        // group 2q + 1 of the row 8 above (DPP rotation by 8 inside the row),
        // so that one store writes rows 0-7 and the next rows 8-15 of the
        // block, each row 64 contiguous columns (128 bytes). A lane stores
        // row rl (+ 8 h + 16 i) at columns colq (+ 64 q); the row parts of
        // the byte offsets are uniform (scalar registers).
        const bool hi = r16 >= 8;
        const int rl = r16 & 7;
        const int colq = n0 + wn * 16 * NJ + (g & 1) * 16 + (g >> 1) * 8 + (hi ? 32 : 0);
        const int rowl = m0 + wm * kWr + rl;
        const int64_t lane_off = ((int64_t)rl * a.ldc + colq) * 2;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < NJ / 4; ++q) {
                u32x4 vs[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int pr = 2 * q + h;
                    const f32x4& x = acc[i][2 * pr];
                    const f32x4& y = acc[i][2 * pr + 1];
                    const float* bx = bv[2 * pr];
                    const float* by = bv[2 * pr + 1];
                    const unsigned x01 = pack2<CT>(epi<EPI>(x[0], alpha, EPI ? bx[0] : 0.f, relu),
                                                   epi<EPI>(x[1], alpha, EPI ? bx[1] : 0.f, relu));
                    const unsigned x23 = pack2<CT>(epi<EPI>(x[2], alpha, EPI ? bx[2] : 0.f, relu),
                                                   epi<EPI>(x[3], alpha, EPI ? bx[3] : 0.f, relu));
                    const unsigned y01 = pack2<CT>(epi<EPI>(y[0], alpha, EPI ? by[0] : 0.f, relu),
                                                   epi<EPI>(y[1], alpha, EPI ? by[1] : 0.f, relu));
                    const unsigned y23 = pack2<CT>(epi<EPI>(y[2], alpha, EPI ? by[2] : 0.f, relu),
                                                   epi<EPI>(y[3], alpha, EPI ? by[3] : 0.f, relu));
                    const auto s0 = __builtin_amdgcn_permlane16_swap(x01, y01, false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(x23, y23, false, false);
                    vs[h] = u32x4{s0[0], s1[0], s0[1], s1[1]};
                }
                u32x4 d[2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned u = hi ? vs[0][e] : vs[1][e];
                    const unsigned w = (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0x128, 0xf, 0xf, false);
                    d[0][e] = hi ? w : vs[0][e];
                    d[1][e] = hi ? vs[1][e] : w;
                }
                const int col = colq + 64 * q;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ru = i * 16 + 8 * h;                 // uniform part of the row
                    const bool rok = rowl + ru < a.M;
                    const bool ok16 = rok & (col + 8 <= a.N) & (a.c16 != 0);
                    store16_lanes(d[h], crs, ok16, lane_off + 128 * q + (int64_t)ru * a.ldc * 2, stream);
                    if (__builtin_expect(!whole, 0)) {
                        asm volatile("");             // a scalar branch of its own, not merged into the lane mask
                        uint16_t* dst = static_cast<uint16_t*>(a.C) + (int64_t)(rowl + ru) * a.ldc + col;
                        const u32x4& v = d[h];
                        if (ok16 || !rok) {
                        } else if (col + 8 <= a.N && a.c8) {
                            __builtin_nontemporal_store(u32x2{v[0], v[1]}, (u32x2*)dst);
                            __builtin_nontemporal_store(u32x2{v[2], v[3]}, (u32x2*)(dst + 4));
                        } else if (col < a.N) {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                if (col + e < a.N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                        }
                    }
                }
            }
        }
    }
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[8][8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};
}

// Zero accumulators produced by a matrix instruction (0 * 0 + 0 = +0, the
// same bits as zero_acc). Sums that start from plain zero moves make the
// register allocator keep some of them in vector registers across the K loop
// and copy them into the accumulator file at every step; starting from a
// matrix result keeps all of them in the accumulator file.
template <int AB, int NI = 8>
__device__ __forceinline__ void zero_acc_mma(f32x4 (&acc)[NI][8]) {
    const half8 z{};
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (AB == 2)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(0.0f, 0.0f, f32x4{}, 0, 0, 0);
            else
                acc[i][j] = mfma16<AB>(z, z, f32x4{});
        }
}

// ---------------------------------------------------------------------------
// Register-staged path (any stride, element-wise or 128-bit global loads):
// both operands are written K-contiguous into a BK = 64 deep LDS block with
// the KS = 64 map above, double-buffered.
// ---------------------------------------------------------------------------
using LdsR = Lds<BK>;

// Stage one BK-wide block of a K-contiguous operand (A, or B stored N x K):
// rows row0 .. row0+255, k = k0 .. k0+63. Thread t loads chunk (t & 7) of
// rows (t >> 3) + 32p: eight threads cover one 128-byte row segment.
// MASK: rows >= nrows and k >= K read as zero (page 4, section 2.4.6.1.3).
template <bool VEC, bool MASK>
__device__ __forceinline__ void load_kcontig(u32x4 (&r)[8], const uint16_t* __restrict__ X,
                                             int64_t ld, int nrows, int K, int row0, int k0,
                                             int tid) {
    const int gk = k0 + (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int gr = row0 + (tid >> 3) + 32 * p;
        if (!MASK) {
            const uint16_t* src = X + (int64_t)gr * ld + gk;
            r[p] = VEC ? *(const u32x4*)src : load8_elems(src, 8);
        } else {
            const int rem = K - gk;
            const int nv = (gr < nrows) ? (rem < 0 ? 0 : (rem > 8 ? 8 : rem)) : 0;
            const int grc = gr < nrows ? gr : nrows - 1;
            const uint16_t* src = X + (int64_t)grc * ld + (nv > 0 ? gk : 0);
            if (VEC && nv == 8)
                r[p] = *(const u32x4*)src;
            else
                r[p] = load8_elems(src, nv);
        }
    }
}

__device__ __forceinline__ void store_kcontig(u32x4* __restrict__ s, const u32x4 (&r)[8], int tid) {
    const int c = tid & 7;
#pragma unroll
    for (int p = 0; p < 8; ++p) s[LdsR::slot((tid >> 3) + 32 * p, c)] = r[p];
}

// Stage one BK-deep block of B stored K x N: k = k0 .. k0+63, n = n0 .. n0+255.
// Thread t owns the 8 x 8 block k = k0 + 8*(t & 7) + 0..7, n = n0 + 8*(t >> 3) + 0..7
// and loads it as eight 128-bit row pieces.
template <bool VEC, bool MASK>
__device__ __forceinline__ void load_kxn(u32x4 (&r)[8], const uint16_t* __restrict__ B, int64_t ldb,
                                         int N, int K, int n0, int k0, int tid) {
    const int gn = n0 + (tid >> 3) * 8;
    const int gk0 = k0 + (tid & 7) * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int gk = gk0 + kk;
        if (!MASK) {
            const uint16_t* src = B + (int64_t)gk * ldb + gn;
            r[kk] = VEC ? *(const u32x4*)src : load8_elems(src, 8);
        } else {
            const int rem = N - gn;
            const int nv = (gk < K) ? (rem < 0 ? 0 : (rem > 8 ? 8 : rem)) : 0;
            const int gkc = gk < K ? gk : K - 1;
            const uint16_t* src = B + (int64_t)gkc * ldb + (nv > 0 ? gn : 0);
            if (VEC && nv == 8)
                r[kk] = *(const u32x4*)src;
            else
                r[kk] = load8_elems(src, nv);
        }
    }
}

// Transpose the 8 x 8 block in registers and write it K-contiguous: LDS row
// n0' + nn receives k = 8*(t & 7) + 0..7 as logical chunk (t & 7). Threads
// with odd column-block index write their rows in swapped pair order so that
// the 16 lanes of a bank-group pass touch rows of both parities.
__device__ __forceinline__ void store_kxn(u32x4* __restrict__ s, const u32x4 (&r)[8], int tid) {
    const int kb = tid & 7;
    const int nb = tid >> 3;
    u32x4 t[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {       // word q of a row holds columns 2q (low) and 2q+1 (high)
#pragma unroll
        for (int p = 0; p < 4; ++p) {   // word p of a column holds rows 2p (low) and 2p+1 (high)
            const unsigned lo = r[2 * p][q], hi = r[2 * p + 1][q];
            t[2 * q][p] = (lo & 0xffffu) | (hi << 16);
            t[2 * q + 1][p] = (lo >> 16) | (hi & 0xffff0000u);
        }
    }
    const int odd = nb & 1;
#pragma unroll
    for (int sidx = 0; sidx < 8; ++sidx) {
        const u32x4 v = odd ? t[sidx ^ 1] : t[sidx];
        s[LdsR::slot(nb * 8 + (sidx ^ odd), kb)] = v;
    }
}

// One BK step of the wave's 128 x 128 sub-tile: 2 k32 slices x 8 x 8 MFMAs.
template <int AB>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[8][8], const u32x4* __restrict__ sA,
                                         const u32x4* __restrict__ sB, int wm, int wn, int lane) {
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
        half8 af[8], bf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) af[i] = read_kc<BK>(sA, wm, i, lane, s);
#pragma unroll
        for (int j = 0; j < 8; ++j) bf[j] = read_kc<BK>(sB, wn, j, lane, s);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = mfma16<AB>(bf[j], af[i], acc[i][j]);
    }
}

template <int NXK, bool VEC, bool MASK>
__device__ __forceinline__ void load_stage(u32x4 (&ra)[8], u32x4 (&rb)[8], const Args& a, int m0, int n0,
                                           int k0, int tid) {
    load_kcontig<VEC, MASK>(ra, a.A, a.lda, a.M, a.K, m0, k0, tid);
    if (NXK)
        load_kcontig<VEC, MASK>(rb, a.B, a.ldb, a.N, a.K, n0, k0, tid);
    else
        load_kxn<VEC, MASK>(rb, a.B, a.ldb, a.N, a.K, n0, k0, tid);
}

template <int NXK>
__device__ __forceinline__ void store_stage(u32x4* __restrict__ sA, u32x4* __restrict__ sB,
                                            const u32x4 (&ra)[8], const u32x4 (&rb)[8], int tid) {
    store_kcontig(sA, ra, tid);
    if (NXK)
        store_kcontig(sB, rb, tid);
    else
        store_kxn(sB, rb, tid);
}

template <int TY, int NXK, bool VEC>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(1, 1)))
tgemm_rs_kernel(Args a) {
    __shared__ u32x4 smem[2][2][LdsR::kBlock];   // [stage][A | B], 128 KiB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_of((int)blockIdx.x, a.W, a.grid_m, a.grid_n, a.group_m, a.num_xcd, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
    const int nk = (a.K + BK - 1) / BK;

    f32x4 acc[8][8];
    zero_acc(acc);

    u32x4 ra[8], rb[8];
    if (nk > 0) {
        if (interior && BK <= a.K)
            load_stage<NXK, VEC, false>(ra, rb, a, m0, n0, 0, tid);
        else
            load_stage<NXK, VEC, true>(ra, rb, a, m0, n0, 0, tid);
        store_stage<NXK>(smem[0][0], smem[0][1], ra, rb, tid);
        __syncthreads();
    }
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nk;
        if (more) {
            const int k0 = (t + 1) * BK;
            if (interior && k0 + BK <= a.K)
                load_stage<NXK, VEC, false>(ra, rb, a, m0, n0, k0, tid);
            else
                load_stage<NXK, VEC, true>(ra, rb, a, m0, n0, k0, tid);
        }
        mma_step<ab_of(TY)>(acc, smem[cur][0], smem[cur][1], wm, wn, lane);
        if (more) store_stage<NXK>(smem[cur ^ 1][0], smem[cur ^ 1][1], ra, rb, tid);
        __syncthreads();
    }
    store_c<TY>(acc, a, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Direct HBM/L2 -> LDS staging (any 2-byte alignment; row strides below the
// limits the host checks).
//
// buffer_load_dwordx4 ... lds writes lane L of a wave instruction to LDS
// bytes [base + 16L, base + 16L + 16): the destination slot is fixed by the
// lane, so the XOR swizzle is applied on the source side instead.
//
// Zero padding (page 4, section 2.4.6.1.3): a lane whose byte offset (vector
// + scalar part) reaches the buffer resource's record count reads zeros, and
// the zeros are what it writes into its LDS slot. A tile's resource ends at
// its operand's last element, so rows past the operand (and, for B stored
// K x N, rows past K) read zeros; steps past the last tile use a scalar
// offset of kOob and touch no memory at all. The one remaining case, chunks
// at or past K on the last, partial K step, is rewritten in LDS before that
// step is published. Each lane's load offsets are computed once and do not
// depend on the tile: with one wave per SIMD, a vector ALU write into a
// register a matrix instruction has just read stalls the matrix cores, so
// the main loop carries no per-load arithmetic.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) const char lds_cchar;

constexpr unsigned kOob = 0x80000000u;       // record counts stay below this

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    // s_waitcnt fields: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Compiler-level fence: no memory access is moved across it. The hardware
// ordering comes from the explicit s_waitcnt and s_barrier around it.
#define TG_COMPILER_FENCE() __asm__ __volatile__("" ::: "memory")

__device__ __forceinline__ void block_barrier() {
    TG_COMPILER_FENCE();
    __builtin_amdgcn_s_barrier();
    TG_COMPILER_FENCE();
}

// Base pointer and record count of the buffer resource over operand rows
// row0 .. nrows-1 (row stride ld): the byte span from the first of these rows
// to the operand's last element. Every offset a tile forms inside its 256
// rows stays below 2^31 (host stride limit); the span is capped below kOob,
// which only shortens it for tiles far from the operand's end.
struct Rsrc {
    const uint16_t* base;
    int nrec;
};

__device__ __forceinline__ Rsrc operand_rsrc(const uint16_t* X, int64_t ld, int nrows, int ncols, int row0) {
    int64_t span = ((int64_t)(nrows - row0 - 1) * ld + ncols) * 2;
    if (span > (int64_t)kOob - 1) span = (int64_t)kOob - 1;
    return Rsrc{X + (int64_t)row0 * ld, (int)span};
}

// B stored K x N is kept N-contiguous in LDS, [k][n] (512 bytes per k row):
// 16-byte chunk c (n = 8c .. 8c+7) of k row k sits at physical chunk
// c ^ h(k), h(k) = 2 (k & 3) ^ 8 ((k >> 3) & 1) ^ 16 ((k >> 4) & 1). A
// transposing fragment read has each 16-lane group read 4 consecutive k rows
// x 32 contiguous bytes, the four groups 8 rows apart; h spreads every 16-
// and 32-lane part of such a read over distinct banks. h ignores k bits 2
// and 5, so the second half of a fragment (k + 4) and the next 32-deep slice
// (k + 32) sit at fixed byte distances from the first.
struct KnLds {
    __device__ static __forceinline__ int h(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)) ^ (16 * ((k >> 4) & 1)); }
    __device__ static __forceinline__ int phys(int c, int k) { return c ^ h(k); }
    __device__ static __forceinline__ int logical(int p, int k) { return p ^ h(k); }
};

// Binary32 B stored K x N, [k][n] in LDS: a 16-deep step is 16 k rows of 256
// floats (1 KiB, 64 chunks of 4 floats); chunk c of k row k sits at physical
// chunk c ^ 4 ((k >> 2) & 3). A 16x16x4 fragment takes float e of block j
// for lane l from k row 4 (l / 16) + e, column 128 wn + 16 j + (l mod 16):
// four 32-bit reads whose 16-lane groups (k rows 4 apart) fall in four
// distinct 16-bank windows. Load instruction j of wave w fills k row 4j + w
// linearly, lane t taking logical chunk t ^ 4j. B's rows past K read zeros
// (they lie past the per-step range); a chunk straddling column N reads the
// next row's first floats, which reach only output columns that are never
// stored, except in B's last row, where the range check zeroes the whole
// chunk and fix_last_step reloads its valid floats.
struct F32KnLds {
    // byte offset in the B block of block jl (0..3; jl + 4 is 256 bytes on),
    // float e = 0 (e adds 1024 bytes), for lane group g, wave column wn, lane r16
    __device__ static __forceinline__ int frag_byte(int g, int wn, int jl, int r16) {
        return 4096 * g + 512 * wn + 64 * (jl ^ g) + 4 * r16;
    }
};

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four k values (4 consecutive k rows) of one n column of B stored [k][n],
// by the transposing read ds_read_b64_tr_b16: in each 16-lane group, lane i
// points at k row k0 + i/4, columns n0 + 4(i % 4) .. +3, and lane j receives
// column n0 + j.
__device__ __forceinline__ s16x4 read_tr(lds_cchar* __restrict__ p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
#else
    (void)p;
    return s16x4{};
#endif
}

__device__ __forceinline__ half8 join_halves(const s16x4& lo, const s16x4& hi) {
    return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// This lane's LDS read positions in stage 0 (stage st's A and B blocks sit
// st * CPR * 256 slots after stage 0's, within 64 KiB, so a read is one base
// register plus an immediate offset):
//  a[s], b[s]: the A and (K-contiguous) B fragments of 16-row block 0 for
//              slice s; block i lies 16 * CPR slots further.
//  tr[blk]:    for B stored [k][n], the transposing read of 16-column block
//              blk, slice 0, k rows +0..3 of the lane's 8 (lane l needs
//              column 128 wn + 16 blk + (l mod 16), k = 8 (l / 16) + 0..7);
//              k + 4 adds 2 KiB and slice s adds 16 KiB * s.
template <int KS, int NXK>
struct FragPtrs {
    const u32x4* a[KS / 32];
    const u32x4* b[KS / 32];
    lds_cchar* tr[8];
};

template <int KS, int NXK, int I = 8, int AB = 0>
__device__ __forceinline__ FragPtrs<KS, NXK> frag_ptrs(const u32x4* a_blk, const u32x4* b_blk, int wm, int wn,
                                                        int lane) {
    using L = Lds<KS>;
    FragPtrs<KS, NXK> f;
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS / 32; ++s) {
        f.a[s] = a_blk + L::slot(wm * 16 * I + r16, s * 4 + g);
        f.b[s] = b_blk + L::slot(wn * 128 + r16, s * 4 + g);
    }
    if constexpr (AB == 2 && !NXK) {
        // binary32 B stored K x N (F32KnLds): block j's float e of this lane
        // sits at tr[j & 3] + 256 (j >> 2) + 1024 e bytes
#pragma unroll
        for (int jl = 0; jl < 8; ++jl)
            f.tr[jl] = jl < 4 ? (lds_cchar*)b_blk + F32KnLds::frag_byte(g, wn, jl, r16) : nullptr;
    } else {
        const int krow = 8 * g + (r16 >> 2);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            const int ncol = wn * 128 + blk * 16 + 4 * (r16 & 3);
            const int byte = krow * 512 + KnLds::phys(ncol >> 3, krow) * 16 + (ncol & 7) * 2;
            f.tr[blk] = NXK ? nullptr : (lds_cchar*)b_blk + byte;
        }
    }
    return f;
}

// The read positions `so` slots further (those of another stage).
template <int KS, int NXK>
__device__ __forceinline__ FragPtrs<KS, NXK> shifted(const FragPtrs<KS, NXK>& f, int so) {
    FragPtrs<KS, NXK> g;
#pragma unroll
    for (int s = 0; s < KS / 32; ++s) {
        g.a[s] = f.a[s] + so;
        g.b[s] = f.b[s] + so;
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) g.tr[blk] = NXK ? nullptr : f.tr[blk] + so * 16;
    return g;
}

// Fragment reads; `so` is the stage's offset in slots from stage 0.
template <int KS, int NXK>
__device__ __forceinline__ half8 frag_a(const FragPtrs<KS, NXK>& f, int so, int s, int i) {
    return __builtin_bit_cast(half8, f.a[s][so + i * 16 * (KS / 8)]);
}

template <int KS, int NXK>
__device__ __forceinline__ half8 frag_b_kc(const FragPtrs<KS, NXK>& f, int so, int s, int j) {
    return __builtin_bit_cast(half8, f.b[s][so + j * 16 * (KS / 8)]);
}

template <int KS, int NXK>
__device__ __forceinline__ s16x4 frag_b_tr(const FragPtrs<KS, NXK>& f, int so, int s, int blk, int hh) {
    return read_tr(f.tr[blk] + so * 16 + s * 16384 + hh * 2048);
}

// Binary32 B stored K x N: float e of block j's fragment (F32KnLds).
template <int KS, int NXK>
__device__ __forceinline__ unsigned frag_b_f32kn(const FragPtrs<KS, NXK>& f, int so, int j, int e) {
    return *reinterpret_cast<const __attribute__((address_space(3))) unsigned*>(f.tr[j & 3] + so * 16 +
                                                                                (j >> 2) * 256 + e * 1024);
}

// Per-lane source offsets of the 2 * CPR load instructions of a K step (A's
// CPR, then B's). A wave instruction j fills LDS slots (4j + w) * 64 + L.
//  * K-contiguous operand (A; B stored N x K): slot -> row (256 / CPR) * j +
//    tid / CPR, physical chunk tid % CPR, which must hold logical chunk
//    (tid % CPR) ^ f(row); f(row) does not depend on j. The K step advances
//    the scalar offset by KS * 2 bytes.
//  * B stored K x N ([k][n], 32 chunks per k row): slot -> k row 8j +
//    (tid >> 5), physical chunk tid & 31, holding logical chunk
//    (tid & 31) ^ h(k row). Each K step loads through a resource based at
//    its own first k row (b_step_rsrc), so these offsets stay below
//    KS * ldb * 2 + 512 bytes for every K.
// voff[idx] is the row's byte offset plus the chunk's, relative to the
// tile's resource base; it is the same for every tile.
// An A block of 32 * I rows takes LA = I * CPR / 8 load instructions per
// step (the first LA of the step), B's 256 rows or columns CPR more.
template <int KS, int LA = KS / 8>
struct LaneLoads {
    static constexpr int kCpr = KS / 8;
    static constexpr int kLa = LA;                    // A loads per step
    static constexpr int kL = LA + kCpr;              // loads per step
    unsigned voff[kL];
    unsigned kchunk;      // k offset (elements) of this lane's K-contiguous chunk inside a K step
};

template <int KS, int NXK, int LA = KS / 8, int AB = 0>
__device__ __forceinline__ LaneLoads<KS, LA> lane_loads(const Args& a, int tid) {
    constexpr int kCpr = KS / 8;
    LaneLoads<KS, LA> p;
    const int r = tid / kCpr;
    const unsigned chunk = (unsigned)((tid % kCpr) ^ Lds<KS>::swz(r));
#pragma unroll
    for (int j = 0; j < kCpr; ++j) {
        const int row = r + (256 / kCpr) * j;
        if (j < LA) p.voff[j] = (unsigned)row * (unsigned)a.lda * 2u + chunk * 16u;
        if (NXK) {
            p.voff[LA + j] = (unsigned)row * (unsigned)a.ldb * 2u + chunk * 16u;
        } else if (AB == 2) {
            // binary32 [k][n] (F32KnLds): k row 4j + wave, logical chunk lane ^ 4j
            const unsigned krow = (unsigned)(4 * j + (tid >> 6));
            const unsigned c = (unsigned)((tid & 63) ^ (4 * j));
            p.voff[LA + j] = krow * (unsigned)a.ldb * 2u + c * 16u;
        } else {
            const int krow = 8 * j + (tid >> 5);
            const unsigned c = (unsigned)KnLds::logical(tid & 31, krow);
            p.voff[LA + j] = (unsigned)krow * (unsigned)a.ldb * 2u + c * 16u;
        }
    }
    p.kchunk = chunk * 8u;
    return p;
}

// Load instruction `idx` (0 .. 2*CPR-1) of a K step into the stage whose A
// and B blocks are a_blk and b_blk, with the step's scalar offsets (soa for
// A, sob for B).
template <int KS, int NXK, int LA>
__device__ __forceinline__ void issue_load(const Rsrc& ra, const Rsrc& rb, const LaneLoads<KS, LA>& p, int idx,
                                           unsigned soa, unsigned sob, u32x4* __restrict__ a_blk,
                                           u32x4* __restrict__ b_blk, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass cannot instantiate these target builtins
    const bool isb = idx >= LA;
    const int j = isb ? idx - LA : idx;
    const Rsrc& rs = isb ? rb : ra;
    // word 3 = 0x00020000: raw (untyped) access, 32-bit data format
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)rs.base, 0, rs.nrec, 0x00020000);
    u32x4* dst = (isb ? b_blk : a_blk) + (j * 4 + wave) * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, p.voff[idx], isb ? sob : soa, 0, 0);
#endif
}

// Elements at or past nv of an 8-element chunk set to zero (nv in 1..7).
__device__ __forceinline__ u32x4 keep_first(const u32x4& v, int nv) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const unsigned lo = (2 * q < nv) ? 0x0000ffffu : 0u;
        const unsigned hi = (2 * q + 1 < nv) ? 0xffff0000u : 0u;
        r[q] = v[q] & (lo | hi);
    }
    return r;
}

// Last K step when it is partial (k0 = its first k). Its K-contiguous chunks
// at or past K were loaded as whatever lies there. Every row stride is at
// least 8 elements on this path, so in every row but the operand's last the
// 16-byte access stayed inside the operand's range and read the next bytes of
// memory (the rest of the row, or the next row): a chunk straddling K holds
// its valid elements and only the rest is cleared, by a read-modify-write of
// the lane's own LDS slot; chunks wholly past K are cleared. In the operand's
// last row the range check zeroed the whole straddling access, so that chunk
// is loaded element by element (in a branch only the waves holding that row
// take, so other waves never wait on memory here). B stored K x N straddles
// only at column N, and only its final row K - 1 loses data the same way
// (other rows read the next row past N, which lands in output columns that
// are never stored). This runs after the lane's loads of the stage have
// landed and before the barrier that publishes it.
template <int KS, int NXK, int LA, int AB = 0>
__device__ __forceinline__ void fix_last_step(u32x4* __restrict__ a_blk, u32x4* __restrict__ b_blk,
                                              const LaneLoads<KS, LA>& p, const Args& a, int m0, int n0, int k0,
                                              int tid, int wave, int lane) {
    constexpr int kCpr = KS / 8;
    constexpr int kRowStep = 256 / kCpr;              // rows between a lane's chunks
    const int r = tid / kCpr;
    const int kc = k0 + (int)p.kchunk;
    const int nv = a.K - kc;                          // valid elements of this lane's K chunks (may be <= 0)
    if (nv < 8) {
        // one chunk at a time (not unrolled): this runs once per tile, inside a
        // loop whose fragments hold most of the registers
#pragma unroll 1
        for (int j = 0; j < kCpr; ++j) {
            const int row = r + kRowStep * j;
            const int slot = (j * 4 + wave) * 64 + lane;
            if (j < LA && m0 + row < a.M) {
                if (nv <= 0)
                    a_blk[slot] = u32x4{};
                else if (m0 + row == a.M - 1)
                    a_blk[slot] = load8_elems(a.A + (int64_t)(a.M - 1) * a.lda + kc, nv);
                else
                    a_blk[slot] = keep_first(a_blk[slot], nv);
            }
            if (NXK && n0 + row < a.N) {
                if (nv <= 0)
                    b_blk[slot] = u32x4{};
                else if (n0 + row == a.N - 1)
                    b_blk[slot] = load8_elems(a.B + (int64_t)(a.N - 1) * a.ldb + kc, nv);
                else
                    b_blk[slot] = keep_first(b_blk[slot], nv);
            }
        }
    }
    if (!NXK && AB == 2) {
        // binary32 [k][n] (F32KnLds): load j of this wave holds k row 4j + wave,
        // logical chunk lane ^ 4j; B's last row is k0 / 2 + krow == K / 2 - 1
        // (k0 and K in 16-bit units)
#pragma unroll 1
        for (int j = 0; j < kCpr; ++j) {
            const int krow = 4 * j + wave;
            const int nc = n0 + 4 * (lane ^ (4 * j));
            const int nvn = a.N - nc;                   // valid floats of the chunk
            if (k0 / 2 + krow == a.K / 2 - 1 && nvn > 0 && nvn < 4)
                b_blk[(j * 4 + wave) * 64 + lane] =
                    load8_elems(a.B + (int64_t)(a.K / 2 - 1) * a.ldb + 2 * (int64_t)nc, 2 * nvn);
        }
    } else if (!NXK) {
#pragma unroll 1
        for (int j = 0; j < kCpr; ++j) {
            const int krow = 8 * j + (tid >> 5);
            const int c = KnLds::logical(tid & 31, krow);
            const int nc = n0 + 8 * c;
            const int nvn = a.N - nc;
            if (k0 + krow == a.K - 1 && nvn > 0 && nvn < 8)
                b_blk[(j * 4 + wave) * 64 + lane] = load8_elems(a.B + (int64_t)(a.K - 1) * a.ldb + nc, nvn);
        }
    }
    TG_COMPILER_FENCE();
    wait_lgkmcnt0();                                  // this lane's LDS writes done before the barrier
    TG_COMPILER_FENCE();
}

// All fragments of slice `s` of stage 0 (used once, before the main loop).
template <int KS, int NXK, int I = 8, int AB = 0>
__device__ __forceinline__ void read_frags(half8 (&fa)[I], half8 (&fb)[8], const FragPtrs<KS, NXK>& f, int s) {
#pragma unroll
    for (int i = 0; i < I; ++i) fa[i] = frag_a(f, 0, s, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if constexpr (AB == 2 && !NXK)
            fb[j] = __builtin_bit_cast(half8, u32x4{frag_b_f32kn(f, 0, j, 0), frag_b_f32kn(f, 0, j, 1),
                                                    frag_b_f32kn(f, 0, j, 2), frag_b_f32kn(f, 0, j, 3)});
        else
            fb[j] = NXK ? frag_b_kc(f, 0, s, j) : join_halves(frag_b_tr(f, 0, s, j, 0), frag_b_tr(f, 0, s, j, 1));
    }
}

// One k32 slice: 8 I MFMAs (I x 8 blocks, serpentine by row) on the current
// fragments, with the next slice's fragment reads (slice next_s of the
// stage `so` slots from stage 0) and, when LOADS, the load instructions of
// one K step placed between them, in the order the next slice consumes them
// (A0, B0..B7, A1..; a [k][n] B fragment is two transposing reads). With
// I = 8 (64 MFMAs): reads after every even-numbered MFMA, loads spread evenly
// over the odd-numbered ones. Other I: the reads and loads together spread
// evenly over the MFMAs (several after one MFMA when there are more of them
// than MFMAs), the loads evenly among them. One instruction per MFMA keeps
// the matrix core fed; with one wave per SIMD every other instruction
// competes with MFMA issue, so the order is pinned at both the IR and the
// machine level.
template <int AB, int KS, int NXK, bool LOADS, bool ZC = false, bool READS = true, int I = 8, int LA = KS / 8>
__device__ __forceinline__ void slice(f32x4 (&acc)[I][8], const half8 (&fa)[I], const half8 (&fb)[8],
                                      half8 (&na)[I], half8 (&nb)[8], const FragPtrs<KS, NXK>& f, int so,
                                      int next_s, const Rsrc& ra, const Rsrc& rb, const LaneLoads<KS, LA>& p,
                                      unsigned soa, unsigned sob, u32x4* __restrict__ ld_a, u32x4* __restrict__ ld_b,
                                      int wave) {
    constexpr bool kF32Kn = AB == 2 && !NXK;
    constexpr int kNb = NXK ? 8 : (kF32Kn ? 32 : 16);   // B read instructions
    constexpr int kReads = I + kNb;
    s16x4 lo[8];
    // read number rq of the next slice's fragments (consumption order)
    auto read = [&](int rq) {
        if (rq >= 1 && rq <= kNb) {
            if (kF32Kn) {
                const int blk = (rq - 1) >> 2, e = (rq - 1) & 3;
                u32x4 v = __builtin_bit_cast(u32x4, nb[blk]);
                v[e] = frag_b_f32kn(f, so, blk, e);
                nb[blk] = __builtin_bit_cast(half8, v);
            } else if (NXK) {
                nb[rq - 1] = frag_b_kc(f, so, next_s, rq - 1);
            } else {
                const int blk = (rq - 1) >> 1, hh = (rq - 1) & 1;
                const s16x4 v = frag_b_tr(f, so, next_s, blk, hh);
                if (hh == 0)
                    lo[blk] = v;
                else
                    nb[blk] = join_halves(lo[blk], v);
            }
        } else {
            const int ai = rq == 0 ? 0 : rq - kNb;
            na[ai] = frag_a(f, so, next_s, ai);
        }
    };
    if constexpr (AB == 2) {
        // binary32 operands: a 16-byte fragment holds 4 floats of one row,
        // k = 4 (l / 16) + e within the 16-deep step, and v_mfma_f32_16x16x4_f32
        // e (e = 0..3) takes float e of every lane, so it sums the products of
        // k = e, 4 + e, 8 + e, 12 + e. A block's four instructions run back to
        // back on its accumulator (the matrix core chains them; spread over
        // the slice instead, the register allocator moves the accumulators
        // between register files at every step), so each accumulator takes
        // e = 0..3, step after step. A slice is 32 I instructions of 32
        // cycles: the step's loads go first, one after every fourth
        // instruction, so they have most of the slice to land, and the next
        // slice's fragment reads spread evenly over the rest.
        static_assert(KS == 32, "binary32 operands: 16-deep steps (32 16-bit units)");
        constexpr int kQ = 8 * I;                      // blocks
        constexpr int kM = 4 * kQ;                     // matrix instructions
        constexpr int kR = READS ? kReads : 0;
        constexpr int kLd = LOADS ? LaneLoads<KS, LA>::kL : 0;
        constexpr int kLoadEnd = 4 * kLd;              // instructions that carry the loads
        static_assert(kLoadEnd + kR <= kM, "at most one read or load after each matrix instruction");
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = q * 4 + e;
                const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
                const f32x4 av = __builtin_bit_cast(f32x4, fa[i]);
                const f32x4 bv = __builtin_bit_cast(f32x4, fb[j]);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[e], av[e],
                                                                (ZC && e == 0) ? f32x4{} : acc[i][j], 0, 0, 0);
                if (m < kLoadEnd) {
                    if ((m & 3) == 3) issue_load<KS, NXK>(ra, rb, p, m >> 2, soa, sob, ld_a, ld_b, wave);
                } else if (kR) {
                    const int u = m - kLoadEnd, span = kM - kLoadEnd;
                    if ((u + 1) * kR / span > u * kR / span) read(u * kR / span);
                }
                TG_COMPILER_FENCE();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else if constexpr (I == 8) {
        constexpr int kLps = KS / 4;
        constexpr int kGap = 64 / kLps;                // MFMAs per load
        static_assert(2 * kReads <= 64, "reads must fit the even MFMA slots");
        static_assert(LA == KS / 8, "a 256-row A block takes CPR loads");
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            // serpentine over the 8 x 8 blocks: a row change keeps the B fragment,
            // so one operand changes per MFMA throughout (less switching power)
            const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
            // ZC: a tile's first slice starts the sums from zero (inline constant C)
            acc[i][j] = mfma16<AB>(fb[j], fa[i], ZC ? f32x4{} : acc[i][j]);
            if (READS && (q & 1) == 0 && q / 2 < kReads) {
                read(q / 2);
            } else if (LOADS && q % kGap == kGap - 1) {
                issue_load<KS, NXK>(ra, rb, p, q / kGap, soa, sob, ld_a, ld_b, wave);
            }
            TG_COMPILER_FENCE();
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        constexpr int kQ = 8 * I;                      // MFMAs
        constexpr int kR = READS ? kReads : 0;
        constexpr int kLd = LOADS ? LaneLoads<KS, LA>::kL : 0;
        constexpr int kT = kR + kLd;                   // instructions placed between them
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int i = q >> 3, j = (i & 1) ? 7 - (q & 7) : (q & 7);
            acc[i][j] = mfma16<AB>(fb[j], fa[i], ZC ? f32x4{} : acc[i][j]);
#pragma unroll
            for (int e = q * kT / kQ; e < (q + 1) * kT / kQ; ++e) {
                const int before = kT ? e * kLd / kT : 0;       // loads among events 0 .. e-1
                if (kT && (e + 1) * kLd / kT > before)
                    issue_load<KS, NXK>(ra, rb, p, before, soa, sob, ld_a, ld_b, wave);
                else
                    read(e - before);
                TG_COMPILER_FENCE();
            }
            TG_COMPILER_FENCE();
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One output tile: its origin and its operands' buffer resources. For B
// stored K x N, rb.base is column n0 of k row 0 and bspan the byte span from
// there to B's last element; each K step gets a resource of its own
// (b_step_rsrc), so the offsets a step forms cover only its KS rows of B.
struct Tile {
    Rsrc ra, rb;
    int64_t bspan;
    int m0, n0;
};

template <int NXK, int TBM = BM, int AB = 0>
__device__ __forceinline__ Tile make_tile(const Args& a, int wid) {
    int tm, tn;
    tile_of(wid, a.W, a.grid_m, a.grid_n, a.group_m, a.num_xcd, &tm, &tn);
    Tile t;
    t.m0 = tm * TBM;
    t.n0 = tn * BN;
    t.ra = operand_rsrc(a.A, a.lda, a.M, a.K, t.m0);
    // B: N x K rows n0.. ; K x N columns n0.. of all K rows
    if (NXK) {
        t.rb = operand_rsrc(a.B, a.ldb, a.N, a.K, t.n0);
        t.bspan = 0;
    } else if (AB == 2) {
        // binary32 (K, lda and ldb in 16-bit units, N in floats): K / 2 rows of B
        t.rb = Rsrc{a.B + 2 * t.n0, 0};
        t.bspan = ((int64_t)(a.K / 2 - 1) * a.ldb + 2 * (int64_t)(a.N - t.n0)) * 2;
    } else {
        t.rb = Rsrc{a.B + t.n0, 0};
        t.bspan = ((int64_t)(a.K - 1) * a.ldb + (a.N - t.n0)) * 2;
    }
    return t;
}

// B's resource for data step d of tile t (B stored N x K: the tile's own,
// the step is a scalar offset). B stored K x N: based at k row d * KS, with
// the record count running to B's last element (rows past K read zeros),
// capped below kOob; the lane offsets then stay below KS rows of B, so any
// K works with a row stride up to the K-contiguous limit. Scalar arithmetic
// only (d is uniform); a step that loads nothing passes d = 0.
template <int KS, int NXK, int AB = 0>
__device__ __forceinline__ Rsrc b_step_rsrc(const Tile& t, int d, int64_t ldb) {
    if (NXK) return t.rb;
    const int64_t rows = (int64_t)d * (AB == 2 ? KS / 2 : KS);   // binary32: two 16-bit units per k
    int64_t span = t.bspan - rows * ldb * 2;
    span = span < 0 ? 0 : (span > (int64_t)kOob - 1 ? (int64_t)kOob - 1 : span);
    return Rsrc{t.rb.base + rows * ldb, (int)span};
}

// Per-workgroup constants of the direct-to-LDS kernel. With 256-row A
// blocks (I = 8) LDS holds the S stages' A blocks, then their B blocks; with
// smaller A blocks each stage holds its A block then its B block. Either way
// stage st's blocks sit st * kShift slots after stage 0's.
template <int KS, int NXK, int S, int I = 8>
struct DmaCtx {
    static constexpr int kLa = I * (KS / 8) / 8;                    // A loads per step
    static constexpr int kABlk = 32 * I * (KS / 8);                 // slots of an A block
    static constexpr int kBBlk = Lds<KS>::kBlock;                   // slots of a B block (256 rows / columns)
    static constexpr int kShift = I == 8 ? kBBlk : kABlk + kBBlk;   // slots between stages
    static constexpr int kSlots = S * (kABlk + kBBlk);
    LaneLoads<KS, kLa> p;
    unsigned bstep;       // scalar-offset advance of B per K step (B stored N x K; K x N rebases instead)
    int nk, klast;        // K steps per tile; first k of a tile's last step
    int lead;             // leading empty steps (0 or 1): data step of step t is t - lead
    bool fixup;           // a tile's last step needs fix_last_step
    int tid, wave, lane;  // of the loading waves (the producers' own numbering with PC)
    u32x4* smem;
    FragPtrs<KS, NXK> fp; // read positions in stage 0
    __device__ __forceinline__ u32x4* a_blk(int st) const { return smem + st * kShift; }
    __device__ __forceinline__ u32x4* b_blk(int st) const {
        return I == 8 ? smem + (S + st) * kBBlk : smem + st * kShift + kABlk;
    }
};

// K step t of tile tc, in stage st (FIRST: the tile's first step, whose
// first slice starts the sums from zero; LAST: its last step, which leaves
// the next step's first fragments unread so that they are not held in
// registers while the tile's C is stored). The steps a workgroup walks form one
// stream over its tiles: the loads issued here are for the step S further on,
// which is step t + S of tc or, near the end of tc, a first step of the
// workgroup's next tile tn (none when !has_next: those loads read nothing
// and write zeros); with a leading empty step (c.lead = 1, 32-deep rings)
// step u holds data step u - 1. Its first slice's fragments are in buffer F0 of fa/fb;
// the next step's first fragments end up in buffer F0 ^ (KS / 32 odd).
// `cur` holds the read positions of stage st on entry and those of the next
// stage on return; they are derived once per step, before the barrier wait,
// into registers no matrix instruction reads (a vector ALU write into a
// just-read MFMA operand register stalls the matrix cores).
// CONSUMER (producer/consumer workgroups): the step without its loads, wait
// counts or fix-up, which the producer waves do (producer_step).
template <int AB, int NXK, int KS, int S, int F0, bool FIRST = false, bool LAST = false, int I = 8,
          bool CONSUMER = false>
__device__ __forceinline__ void dma_step(f32x4 (&acc)[I][8], half8 (&fa)[2][I], half8 (&fb)[2][8], int st, int t,
                                         const Args& a, const DmaCtx<KS, NXK, S, I>& c, FragPtrs<KS, NXK>& cur,
                                         const Tile& tc, const Tile& tn, bool has_next) {
    using Ctx = DmaCtx<KS, NXK, S, I>;
    constexpr int kSlices = KS / 32;
    constexpr int kL = Ctx::kLa + KS / 8;             // loads per step
    constexpr int FL = (F0 + kSlices - 1) & 1;       // buffer of the last slice
    const int nst = (st + 1 == S) ? 0 : st + 1;
    static_assert(!FIRST || kSlices > 1, "the zero-start slice is the first of a 2-slice step");
#pragma unroll
    for (int s = 0; s + 1 < kSlices; ++s) {
        if (FIRST && s == 0)
            slice<AB, KS, NXK, false, true, true, I>(acc, fa[F0 & 1], fb[F0 & 1], fa[(F0 + 1) & 1], fb[(F0 + 1) & 1],
                                                    cur, 0, 1, tc.ra, tc.rb, c.p, 0u, 0u, c.smem, c.smem, c.wave);
        else
            slice<AB, KS, NXK, false, false, true, I>(acc, fa[(F0 + s) & 1], fb[(F0 + s) & 1], fa[(F0 + s + 1) & 1],
                                                     fb[(F0 + s + 1) & 1], cur, 0, s + 1, tc.ra, tc.rb, c.p, 0u, 0u,
                                                     c.smem, c.smem, c.wave);
    }
    cur = shifted(c.fp, nst * Ctx::kShift);
    if constexpr (CONSUMER) {
        TG_COMPILER_FENCE();
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkmcnt0();                              // this wave's reads of stage st returned
        block_barrier();                              // the producers published step t + 1
        slice<AB, KS, NXK, false, false, !LAST, I>(acc, fa[FL], fb[FL], fa[FL ^ 1], fb[FL ^ 1], cur, 0, 0, tc.ra,
                                                  tc.rb, c.p, 0u, 0u, c.smem, c.smem, c.wave);
    } else {
        // the step these loads are for (uniform: scalar selects)
        const int tl = t + S;
        const bool in_next = tl >= c.nk;
        const int ls = in_next ? tl - c.nk : tl;
        const bool live = !in_next || has_next;
        const int ld = KS == 32 ? ls - c.lead : ls;      // >= 0: tl >= S > lead
        const unsigned soa = live ? (unsigned)ld * (unsigned)(KS * 2) : kOob;
        const unsigned sob = live ? (NXK ? (unsigned)ld * c.bstep : 0u) : kOob;
        const Rsrc lra = in_next ? tn.ra : tc.ra;
        const Rsrc lrb = b_step_rsrc<KS, NXK, AB>(in_next ? tn : tc, live ? ld : 0, a.ldb);
        TG_COMPILER_FENCE();
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkmcnt0();                                  // this wave's reads of stage st returned
        wait_vmcnt<(S - 2) * kL>();                       // step t + 1 landed
        // rare (once per tile at most): laid out of line, so that an ordinary step
        // falls through to its last slice and the step loop takes one branch per
        // step, its back edge (+0.9% at 8192^3)
        if (__builtin_expect(c.fixup && t + 2 == c.nk, 0))
            fix_last_step<KS, NXK, Ctx::kLa, AB>(c.a_blk(nst), c.b_blk(nst), c.p, a, tc.m0, tc.n0, c.klast, c.tid,
                                                 c.wave, c.lane);
        block_barrier();
        // the loads go into the stage just released
        slice<AB, KS, NXK, true, false, !LAST, I>(acc, fa[FL], fb[FL], fa[FL ^ 1], fb[FL ^ 1], cur, 0, 0, lra, lrb,
                                                 c.p, soa, sob, c.a_blk(st), c.b_blk(st), c.wave);
    }
}

// A producer wave's part of K step t (producer/consumer workgroups, one tile
// per workgroup): wait for its own loads of step t + 1, fix up a partial last
// step, meet the consumers at the step's barrier (which publishes step t + 1
// and releases stage st), then load step t + S into stage st.
template <int NXK, int KS, int S, int I>
__device__ __forceinline__ void producer_step(int st, int t, const Args& a, const DmaCtx<KS, NXK, S, I>& c,
                                              const Tile& tc) {
    using Ctx = DmaCtx<KS, NXK, S, I>;
    constexpr int kL = Ctx::kLa + KS / 8;
    const int nst = (st + 1 == S) ? 0 : st + 1;
    const int tl = t + S;
    const bool live = tl < c.nk;
    const int ld = KS == 32 ? tl - c.lead : tl;
    const unsigned soa = live ? (unsigned)ld * (unsigned)(KS * 2) : kOob;
    const unsigned sob = live ? (NXK ? (unsigned)ld * c.bstep : 0u) : kOob;
    const Rsrc lrb = b_step_rsrc<KS, NXK>(tc, live ? ld : 0, a.ldb);
    wait_vmcnt<(S - 2) * kL>();                       // step t + 1 landed
    if (__builtin_expect(c.fixup && t + 2 == c.nk, 0))
        fix_last_step<KS, NXK>(c.a_blk(nst), c.b_blk(nst), c.p, a, tc.m0, tc.n0, c.klast, c.tid, c.wave, c.lane);
    block_barrier();
#pragma unroll
    for (int idx = 0; idx < kL; ++idx)
        issue_load<KS, NXK>(tc.ra, lrb, c.p, idx, soa, sob, c.a_blk(st), c.b_blk(st), c.wave);
}

// The steps 0 .. nk-1 (an even count) of a one-slice ring, in pairs: such
// steps alternate fragment buffers, so the pair's two steps are two fixed
// variants. One loop with nothing before or after it in the tile: a second
// path into store_c (an odd step taken apart from the pairs) made the register
// allocator split the accumulators between the two register files and move
// them every step.
template <int AB, int NXK, int S, int I = 8, bool CONSUMER = false>
__device__ __forceinline__ void step_pairs(f32x4 (&acc)[I][8], half8 (&fa)[2][I], half8 (&fb)[2][8],
                                           const Args& a, const DmaCtx<32, NXK, S, I>& c, FragPtrs<32, NXK>& cur,
                                           const Tile& tc) {
    int st = 0;
    for (int t = 0; t < c.nk; t += 2) {
        dma_step<AB, NXK, 32, S, 0, false, false, I, CONSUMER>(acc, fa, fb, st, t, a, c, cur, tc, tc, false);
        st = (st + 1 == S) ? 0 : st + 1;
        dma_step<AB, NXK, 32, S, 1, false, false, I, CONSUMER>(acc, fa, fb, st, t + 1, a, c, cur, tc, tc, false);
        st = (st + 1 == S) ? 0 : st + 1;
    }
}

// Tile kernel with both operands streamed straight into an S-stage LDS ring
// of KS-deep K steps (KS / 32 slices each): A K-contiguous, B either
// K-contiguous (stored N x K, NXK = 1) or kept [k][n] and transposed on read
// (stored K x N). The tile is 32 I x 256 (I = 8: 256 x 256, one workgroup
// per compute unit; I = 4 or 2: 128 x 256 or 64 x 256, two per compute unit),
// four waves in a 2 x 2 grid, each 16 I x 128 as I x 8 blocks of 16 x 16.
// Workgroup b computes tiles b, b + grid, ... (grid = the
// workgroups launched: one per compute unit for 64-deep steps, else one per
// tile). Its K steps form one stream across those tiles; step g lives in
// stage g mod S. The barrier of a step sits before its last slice: it
// follows every wave's last fragment read of the step's stage (so the loads
// for the step S further on go into that stage during the last slice) and
// every wave's loads of the next step (whose first fragments that slice
// reads). A step's loads thus have S - 1 steps less one slice to land, and
// the next tile's first steps load while the current tile finishes, so a
// tile's C stores drain while the next tile computes. Every step issues the
// same number of loads (steps past the last tile, and the leading step of an
// odd 32-deep step count, read nothing and write zeros), so all wait counts
// are constants.
// PC (producer/consumer, page 5's warp specialisation: one tile per
// workgroup, 32-deep steps, I = 4): eight waves, two per SIMD; waves 0-3
// compute as above but issue no loads and wait on nothing but their own LDS
// reads and the step barrier; waves 4-7 issue every load, wait for them, fix
// up a partial last step and meet the consumers at the same barriers.
// POL (64-deep steps): the C store policy fixed at compile time (store_c).
template <int TY, int NXK, int KS, int S, int I = 8, bool PC = false, int POL = -1>
__global__ void __launch_bounds__(PC ? 2 * NTHREADS : NTHREADS)
__attribute__((amdgpu_waves_per_eu((I == 8 && !PC) ? 1 : 2, (I == 8 && !PC) ? 1 : 2)))
tgemm_dma_kernel(Args a) {
    constexpr int AB = ab_of(TY);
    using Ctx = DmaCtx<KS, NXK, S, I>;
    static_assert(KS == 64 || KS == 32, "K step");
    static_assert(KS == 32 || S == 2, "64-deep steps use a 2-stage ring");
    static_assert(I == 8 || I == 4 || I == 2, "A blocks of 256, 128 or 64 rows");
    static_assert(Ctx::kLa >= 1, "the A block takes at least one load per step");
    static_assert(!PC || (KS == 32 && I == 4), "producer/consumer workgroups: 32-deep steps, 128 x 256 tiles");
    static_assert(AB != 2 || (KS == 32 && !PC), "binary32 operands: 16-deep steps (32 16-bit units)");
    static_assert(POL < 0 || KS == 64, "a fixed store policy for the persistent kernel only");
    static_assert(S >= 2 && S <= 6 && Ctx::kSlots * 16 <= 160 * 1024, "LDS ring must fit 160 KiB");
    static_assert(I == 8 || PC || Ctx::kSlots * 16 <= 80 * 1024, "two workgroups per compute unit");
    constexpr int kL = Ctx::kLa + KS / 8;             // load instructions per step per loading wave
    constexpr int kBm = 32 * I;                       // tile rows
    __shared__ u32x4 smem[Ctx::kSlots];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = PC && wave >= 4;
    const int wm = PC ? (wave & 3) >> 1 : wave >> 1, wn = wave & 1;
    const int nkd = (a.K + KS - 1) / KS;              // K steps holding data
    // 32-deep steps go in pairs: an odd count gets one leading step whose
    // loads all fall out of range (zeros), so that every tile runs one loop
    const int lead = KS == 32 ? (nkd & 1) : 0;
    const int nk = nkd + lead;

    int wid = (int)blockIdx.x;
    Tile tc = make_tile<NXK, kBm, AB>(a, wid);
    bool has_next = wid + a.grid < a.W;              // K == 0: one tile per workgroup
    Tile tn = has_next ? make_tile<NXK, kBm, AB>(a, wid + a.grid) : tc;
    f32x4 acc[I][8];
    if (KS == 32) zero_acc_mma<AB, I>(acc);

    Ctx c;
    const int ltid = PC ? tid - NTHREADS : tid;       // numbering of the loading waves
    const int lwave = PC ? wave - 4 : wave;
    c.p = lane_loads<KS, NXK, Ctx::kLa, AB>(a, ltid);
    c.bstep = (unsigned)(KS * 2);
    c.nk = nk;
    c.lead = lead;
    c.klast = (nkd - 1) * KS;
    c.fixup = (a.K % KS) != 0 || (!NXK && (a.N % (AB == 2 ? 4 : 8)) != 0);
    c.tid = ltid;
    c.wave = lwave;
    c.lane = lane;
    c.smem = smem;
    c.fp = frag_ptrs<KS, NXK, I, AB>(c.a_blk(0), c.b_blk(0), wm, wn, lane);
    if (producer) {
        if (nk > 0) {
            for (int t = 0; t < S; ++t) {
                const int d = t - lead;
                const bool live = d >= 0 && t < nk;
                for (int idx = 0; idx < kL; ++idx)
                    issue_load<KS, NXK>(tc.ra, b_step_rsrc<KS, NXK, AB>(tc, live ? d : 0, a.ldb), c.p, idx,
                                        live ? (unsigned)d * (unsigned)(KS * 2) : kOob,
                                        live ? (NXK ? (unsigned)d * c.bstep : 0u) : kOob, c.a_blk(t), c.b_blk(t),
                                        lwave);
            }
            wait_vmcnt<(S - 1) * kL>();               // step 0 landed
            if (c.fixup && nk == 1)
                fix_last_step<KS, NXK, Ctx::kLa, AB>(c.a_blk(0), c.b_blk(0), c.p, a, tc.m0, tc.n0, c.klast, ltid, lwave,
                                                     lane);
            block_barrier();
            int st = 0;
            for (int t = 0; t < nk; ++t) {
                producer_step<NXK, KS, S, I>(st, t, a, c, tc);
                st = (st + 1 == S) ? 0 : st + 1;
            }
        }
        wait_vmcnt<0>();                              // no load may still be writing LDS at exit
        return;
    }
    half8 fa[2][I], fb[2][8];
    if (nk > 0) {
        if constexpr (!PC) {
            // prologue: steps 0 .. S-1 of the first tile (a workgroup with more
            // than one tile has nk >= S); step t holds data step t - lead
            for (int t = 0; t < S; ++t) {
                const int d = t - lead;                   // data step
                const bool live = d >= 0 && t < nk;
                for (int idx = 0; idx < kL; ++idx)
                    issue_load<KS, NXK>(tc.ra, b_step_rsrc<KS, NXK, AB>(tc, live ? d : 0, a.ldb), c.p, idx,
                                        live ? (unsigned)d * (unsigned)(KS * 2) : kOob,
                                        live ? (NXK ? (unsigned)d * c.bstep : 0u) : kOob, c.a_blk(t), c.b_blk(t),
                                        wave);
            }
            wait_vmcnt<(S - 1) * kL>();                   // step 0 landed
            if (c.fixup && nk == 1)
                fix_last_step<KS, NXK, Ctx::kLa, AB>(c.a_blk(0), c.b_blk(0), c.p, a, tc.m0, tc.n0, c.klast, tid, wave,
                                                     lane);
        }
        block_barrier();
        read_frags<KS, NXK, I, AB>(fa[0], fb[0], c.fp, 0);
    }
    FragPtrs<KS, NXK> cur = c.fp;                     // read positions of the current stage
    if constexpr (KS == 64) {
        // tile after tile (two slices per step: every step starts on
        // fragment buffer 0). A tile's first slice starts its sums from zero
        // and its C is stored after the last step, so the accumulators carry
        // nothing from one tile to the next; only the next tile's first
        // fragments and the load stream do.
        // (64-deep steps are used with nk >= 2)
        int st = 0;
        for (;;) {
            dma_step<AB, NXK, KS, S, 0, true, false, I>(acc, fa, fb, st, 0, a, c, cur, tc, tn, has_next);
            st ^= 1;
            for (int t = 1; t + 1 < nk; ++t) {
                dma_step<AB, NXK, KS, S, 0, false, false, I>(acc, fa, fb, st, t, a, c, cur, tc, tn, has_next);
                st ^= 1;
            }
            dma_step<AB, NXK, KS, S, 0, false, true, I>(acc, fa, fb, st, nk - 1, a, c, cur, tc, tn, has_next);
            st ^= 1;
            store_c<TY, 8, I, POL>(acc, a, tc.m0, tc.n0, wm, wn, lane);
            if (!has_next) break;
            read_frags<KS, NXK, I, AB>(fa[0], fb[0], cur, 0);   // the next tile's first fragments
            wid += a.grid;
            tc = tn;
            has_next = wid + a.grid < a.W;
            if (has_next) tn = make_tile<NXK, kBm, AB>(a, wid + a.grid);
        }
    } else {
        // one tile per workgroup, its steps (an even count) in pairs
        step_pairs<AB, NXK, S, I, PC>(acc, fa, fb, a, c, cur, tc);
        store_c<TY, 8, I>(acc, a, tc.m0, tc.n0, wm, wn, lane);
    }
    // no load may still be writing this workgroup's LDS when it exits
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// binary32 operands, general kernel (for strides, alignments and a K x N B
// with N not a multiple of 4 that the direct-to-LDS kernel does not take; it
// runs binary32 operands on the same tiles with the fragment layout below).
// Page 1's launcher gives 4-byte inputs a tile configuration of their own;
// here the output tile and the wave grid stay those of the 16-bit kernels
// (256 x 256, 2 x 2 waves of 128 x 128 as 8 x 8 blocks of 16 x 16 fp32
// accumulators, so store_c is shared) and the K step is 16 floats. The inner
// product is v_mfma_f32_16x16x4_f32 (one float of each operand per lane, 32
// cycles): operands are staged through registers (any stride and alignment
// of 4 bytes) into a 2-stage LDS ring.
//
// LDS: per stage an A block and a B block of 256 rows x 4 chunks of 4 floats
// (k 4c .. 4c+3 in chunk c), chunk c of row r at slot r * 4 + (c ^ f(r)),
// f(r) = (r ^ (r >> 2)) & 3 (the 64-byte-row map of Lds<32>: conflict-free
// fragment reads and chunk writes).
//
// Fragments: lane l (row l mod 16 of a 16-row block, group g = l / 16) reads
// chunk g, i.e. k = k0 + 4g + 0..3. MFMA e (0..3) takes element e of the A
// and B chunks: its four lane groups cover k0 + e, k0 + 4 + e, k0 + 8 + e,
// k0 + 12 + e, so the four MFMAs together sum the 16 k of the step.
// ---------------------------------------------------------------------------
constexpr int kF32Ks = kF32KStep;               // K step (floats)
using LdsF = Lds<32>;                           // 4 chunks of 16 bytes per row
static_assert(LdsF::kCpr == 4 && LdsF::kBlock == 1024, "fp32 LDS blocks: 256 rows x 4 chunks");

// Four floats at p[0..nv-1]; the rest read as zero.
__device__ __forceinline__ u32x4 load4_f32(const uint32_t* __restrict__ p, int nv) {
    unsigned w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (q < nv) ? p[q] : 0u;
    return u32x4{w[0], w[1], w[2], w[3]};
}

// K-contiguous operand (A, or B stored N x K): thread t loads chunk (t & 3) of
// rows (t >> 2) + 64 p, p = 0..3, for k = k0 .. k0 + 15. MASK: rows >= nrows
// and k >= K read as zero (page 4, section 2.4.6.1.3).
template <bool VEC, bool MASK>
__device__ __forceinline__ void f32_load_kc(u32x4 (&r)[4], const uint32_t* __restrict__ X, int64_t ld, int nrows,
                                            int K, int row0, int k0, int tid) {
    const int gk = k0 + (tid & 3) * 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int gr = row0 + (tid >> 2) + 64 * p;
        if (!MASK) {
            const uint32_t* src = X + (int64_t)gr * ld + gk;
            r[p] = VEC ? *(const u32x4*)src : load4_f32(src, 4);
        } else {
            const int rem = K - gk;
            const int nv = (gr < nrows) ? (rem < 0 ? 0 : (rem > 4 ? 4 : rem)) : 0;
            const int grc = gr < nrows ? gr : nrows - 1;
            const uint32_t* src = X + (int64_t)grc * ld + (nv > 0 ? gk : 0);
            r[p] = (VEC && nv == 4) ? *(const u32x4*)src : load4_f32(src, nv);
        }
    }
}

__device__ __forceinline__ void f32_store_kc(u32x4* __restrict__ s, const u32x4 (&r)[4], int tid) {
#pragma unroll
    for (int p = 0; p < 4; ++p) s[LdsF::slot((tid >> 2) + 64 * p, tid & 3)] = r[p];
}

// B stored K x N: thread t owns the 4 x 4 block k = k0 + 4 (t >> 6) + 0..3,
// n = n0 + 4 (t & 63) + 0..3, loaded as four 16-byte row pieces.
template <bool VEC, bool MASK>
__device__ __forceinline__ void f32_load_kxn(u32x4 (&r)[4], const uint32_t* __restrict__ B, int64_t ldb, int N,
                                             int K, int n0, int k0, int tid) {
    const int gn = n0 + (tid & 63) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int gk = k0 + (tid >> 6) * 4 + q;
        if (!MASK) {
            const uint32_t* src = B + (int64_t)gk * ldb + gn;
            r[q] = VEC ? *(const u32x4*)src : load4_f32(src, 4);
        } else {
            const int rem = N - gn;
            const int nv = (gk < K) ? (rem < 0 ? 0 : (rem > 4 ? 4 : rem)) : 0;
            const int gkc = gk < K ? gk : K - 1;
            const uint32_t* src = B + (int64_t)gkc * ldb + (nv > 0 ? gn : 0);
            r[q] = (VEC && nv == 4) ? *(const u32x4*)src : load4_f32(src, nv);
        }
    }
}

// Transpose the 4 x 4 block: LDS row n0' + v receives k = 4 (t >> 6) + 0..3
// as chunk (t >> 6).
__device__ __forceinline__ void f32_store_kxn(u32x4* __restrict__ s, const u32x4 (&r)[4], int tid) {
    const int kc = tid >> 6, nb = tid & 63;
#pragma unroll
    for (int v = 0; v < 4; ++v) s[LdsF::slot(nb * 4 + v, kc)] = u32x4{r[0][v], r[1][v], r[2][v], r[3][v]};
}

template <int NXK, bool VEC, bool MASK>
__device__ __forceinline__ void f32_load_stage(u32x4 (&ra)[4], u32x4 (&rb)[4], const Args& a, int m0, int n0,
                                               int k0, int tid) {
    const uint32_t* A = reinterpret_cast<const uint32_t*>(a.A);
    const uint32_t* B = reinterpret_cast<const uint32_t*>(a.B);
    f32_load_kc<VEC, MASK>(ra, A, a.lda, a.M, a.K, m0, k0, tid);
    if (NXK)
        f32_load_kc<VEC, MASK>(rb, B, a.ldb, a.N, a.K, n0, k0, tid);
    else
        f32_load_kxn<VEC, MASK>(rb, B, a.ldb, a.N, a.K, n0, k0, tid);
}

template <int NXK>
__device__ __forceinline__ void f32_store_stage(u32x4* __restrict__ sA, u32x4* __restrict__ sB,
                                                const u32x4 (&ra)[4], const u32x4 (&rb)[4], int tid) {
    f32_store_kc(sA, ra, tid);
    if (NXK)
        f32_store_kc(sB, rb, tid);
    else
        f32_store_kxn(sB, rb, tid);
}

__device__ __forceinline__ f32x4 read_f32_frag(const u32x4* __restrict__ s_blk, int half, int blk, int lane) {
    return __builtin_bit_cast(f32x4, s_blk[LdsF::slot(half * 128 + blk * 16 + (lane & 15), lane >> 4)]);
}

// One 16-deep K step of the wave's 128 x 128 sub-tile from LDS: 4 x 8 x 8 MFMAs.
__device__ __forceinline__ void f32_mma_step(f32x4 (&acc)[8][8], const u32x4* __restrict__ sA,
                                             const u32x4* __restrict__ sB, int wm, int wn, int lane) {
    f32x4 af[8], bf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = read_f32_frag(sA, wm, i, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) bf[j] = read_f32_frag(sB, wn, j, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j][e], af[i][e], acc[i][j], 0, 0, 0);
}



// General kernel (any 4-byte alignment and stride, any K): one workgroup per
// output tile; the next step's operands are loaded into registers (masked at
// the edges) while the current step runs on the matrix cores, then written to
// the other LDS stage (one barrier per step).
template <int TY, int NXK, bool VEC>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(1, 1)))
tgemm_f32in_rs_kernel(Args a) {
    static_assert(ab_of(TY) == 2, "binary32 operands");
    __shared__ u32x4 smem[2][2][LdsF::kBlock];   // [stage][A | B], 64 KiB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_of((int)blockIdx.x, a.W, a.grid_m, a.grid_n, a.group_m, a.num_xcd, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
    const int nk = (a.K + kF32Ks - 1) / kF32Ks;

    f32x4 acc[8][8];
    zero_acc(acc);

    u32x4 ra[4], rb[4];
    if (nk > 0) {
        if (interior && kF32Ks <= a.K)
            f32_load_stage<NXK, VEC, false>(ra, rb, a, m0, n0, 0, tid);
        else
            f32_load_stage<NXK, VEC, true>(ra, rb, a, m0, n0, 0, tid);
        f32_store_stage<NXK>(smem[0][0], smem[0][1], ra, rb, tid);
        __syncthreads();
    }
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nk;
        if (more) {
            const int k0 = (t + 1) * kF32Ks;
            if (interior && k0 + kF32Ks <= a.K)
                f32_load_stage<NXK, VEC, false>(ra, rb, a, m0, n0, k0, tid);
            else
                f32_load_stage<NXK, VEC, true>(ra, rb, a, m0, n0, k0, tid);
        }
        f32_mma_step(acc, smem[cur][0], smem[cur][1], wm, wn, lane);
        if (more) f32_store_stage<NXK>(smem[cur ^ 1][0], smem[cur ^ 1][1], ra, rb, tid);
        __syncthreads();
    }
    store_c<TY>(acc, a, m0, n0, wm, wn, lane);
}

// Kernel for a plan, per (input type, output type, epilogue): each is
// instantiated in a translation unit of its own. Returns null for a K step /
// ring depth that combination does not instantiate.
template <int AB, int CT, bool EPI>
const void* kernel_for(const Plan& pl);
#define TG_DECLARE_KERNEL_FOR(ab, ct) \
    template <> const void* kernel_for<ab, ct, false>(const Plan& pl); \
    template <> const void* kernel_for<ab, ct, true>(const Plan& pl);
TG_DECLARE_KERNEL_FOR(0, 0)
TG_DECLARE_KERNEL_FOR(0, 1)
TG_DECLARE_KERNEL_FOR(0, 2)
TG_DECLARE_KERNEL_FOR(1, 0)
TG_DECLARE_KERNEL_FOR(1, 1)
TG_DECLARE_KERNEL_FOR(1, 2)
TG_DECLARE_KERNEL_FOR(2, 0)
TG_DECLARE_KERNEL_FOR(2, 1)
TG_DECLARE_KERNEL_FOR(2, 2)
#undef TG_DECLARE_KERNEL_FOR

}  // namespace tg
