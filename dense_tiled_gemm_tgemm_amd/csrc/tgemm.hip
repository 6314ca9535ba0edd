// fp16 dense tiled GEMM for MI355X (gfx950): C = A * B, binary16 in, fp32
// accumulate, binary16 out.
//
// One workgroup owns one BM x BN output tile and walks K in BK steps (page 1,
// "Using NVIDIA CUDA Tile to write a high-performance matrix multiply",
// sections 1-6; page 4, CUDA programming guide 13.4.2, section 2.4.9.1).
// Per K step the tile's A (BM x BK) and B (BK x BN) blocks are staged from
// HBM/L2 into LDS with coalesced 128-bit loads, double-buffered so the next
// step's loads are in flight while the current step runs on the matrix cores
// (the load / barrier / compute / overlap / write-back lifecycle of page 3,
// "Why GEMM", section 2.2). Partial K tiles are padded with zeros and C
// elements outside M x N are never written (page 4, section 2.4.6.1.3).
//
// gfx950 mapping:
//  * 256 threads = 4 waves of 64 lanes in a 2 x 2 grid; each wave owns a
//    128 x 128 sub-tile held as 4 x 4 blocks of 32 x 32 fp32 accumulators
//    (256 accumulator registers per lane).
//  * Inner product: v_mfma_f32_32x32x16_f16. For a 32x32x16 product each lane
//    supplies 8 consecutive-k binary16 values of one row of each operand
//    (row = lane mod 32, k half = lane / 32), read from LDS as one 128-bit
//    word. The B fragment is passed as the instruction's first operand and
//    the A fragment as its second, so the 32 x 32 result block is C
//    transposed: lane l holds C row (l mod 32), and its accumulator registers
//    4q..4q+3 hold four consecutive C columns 8q + 4*(l/32) + 0..3. The
//    epilogue therefore writes 64-bit runs of four binary16 values.
//  * LDS: both operands are kept K-contiguous, [row][64 halves], as 16-byte
//    chunks; chunk c of row r lives at slot c ^ ((r & 7) ^ ((r >> 3) & 1)).
//    Eight consecutive rows, and sixteen consecutive rows split by parity,
//    map one logical chunk to distinct 16-byte bank groups, so the 128-bit
//    fragment reads (32 rows x one chunk per half-wave) and the 128-bit
//    staging writes are free of bank conflicts (page 3, sections 3.1 and
//    5.3; page 5, "Why swizzle matters").
//  * B stored K x N is transposed in registers while staging: each thread
//    loads an 8 (k) x 8 (n) block with eight 128-bit row loads and writes it
//    as eight 128-bit K-contiguous chunks, so both B layouts share one
//    compute loop.
//  * Workgroup -> tile: die-aware renumbering, then the grouped order of
//    page 1, section "Swizzle" (tile_of in tgemm_plan.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm.h"
#include "tgemm_plan.h"

namespace tg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float acc16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunks = BK / 8;                 // 16-byte chunks per LDS row
constexpr int kTileChunks = 256 * kChunks;      // chunks per staged operand block
static_assert(BM == 256 && BN == 256 && BK == 64 && NTHREADS == 256,
              "the staging maps below assume a 256 x 256 x 64 tile and 256 threads");

struct Args {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int grid_m, grid_n, W, group_m, num_xcd;
};

__device__ __forceinline__ int lds_slot(int row, int chunk) {
    return row * kChunks + (chunk ^ ((row & 7) ^ ((row >> 3) & 1)));
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
    for (int p = 0; p < 8; ++p) s[lds_slot((tid >> 3) + 32 * p, c)] = r[p];
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
        s[lds_slot(nb * 8 + (sidx ^ odd), kb)] = v;
    }
}

// One BK step of the wave's 128 x 128 sub-tile: 4 k16 slices x 4 x 4 MFMAs.
__device__ __forceinline__ void mma_step(acc16 (&acc)[4][4], const u32x4* __restrict__ sA,
                                         const u32x4* __restrict__ sB, int wm, int wn, int lane) {
    const int r32 = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        half8 af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = __builtin_bit_cast(half8, sA[lds_slot(wm * 128 + i * 32 + r32, kk * 2 + khalf)]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bf[j] = __builtin_bit_cast(half8, sB[lds_slot(wn * 128 + j * 32 + r32, kk * 2 + khalf)]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
}

__device__ __forceinline__ unsigned pack_half2(float a, float b) {
    // fp32 -> binary16, round to nearest even (page 1, section 6: the fp32
    // accumulator is converted to C's type when it is stored)
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (unsigned)__builtin_bit_cast(uint16_t, ha) | ((unsigned)__builtin_bit_cast(uint16_t, hb) << 16);
}

template <bool VEC_C>
__device__ __forceinline__ void store_c(const acc16 (&acc)[4][4], const Args& a, int m0, int n0, int wm,
                                        int wn, int lane) {
    const int r32 = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + r32;
        if (m >= a.M) continue;
        uint16_t* crow = a.C + (int64_t)m * a.ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 128 + j * 32 + q * 8 + khalf * 4;
                const unsigned w0 = pack_half2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
                const unsigned w1 = pack_half2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                if (VEC_C && n + 4 <= a.N) {
                    *(u32x2*)(crow + n) = u32x2{w0, w1};
                } else {
                    if (n + 0 < a.N) crow[n + 0] = (uint16_t)(w0 & 0xffffu);
                    if (n + 1 < a.N) crow[n + 1] = (uint16_t)(w0 >> 16);
                    if (n + 2 < a.N) crow[n + 2] = (uint16_t)(w1 & 0xffffu);
                    if (n + 3 < a.N) crow[n + 3] = (uint16_t)(w1 >> 16);
                }
            }
        }
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


// ---------------------------------------------------------------------------
// Direct HBM/L2 -> LDS staging, used when both operands are K-contiguous
// (A, and B stored N x K), 16-byte aligned, K a multiple of 8.
//
// buffer_load_dwordx4 ... lds writes lane L of a wave instruction to LDS
// bytes [base + 16L, base + 16L + 16): the destination slot is fixed by the
// lane, so the XOR swizzle is applied on the source side instead.
//
// Zero padding (page 4, section 2.4.6.1.3) comes from the buffer range
// check: a lane whose byte offset (vector + scalar part) reaches the
// resource's record count reads zeros, and the zeros are what it writes into
// its LDS slot. Rows past the operand carry the offset bit kOob; on the last,
// partial K step so do chunks past K; and steps past the end of K use a
// scalar offset of kOob, so they touch no memory at all. The main loop is
// therefore the same for edge and interior tiles, and branch-free.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

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
// to the operand's last element (below 2^31 by the host's stride limit).
struct Rsrc {
    const uint16_t* base;
    int nrec;
};

__device__ __forceinline__ Rsrc operand_rsrc(const uint16_t* X, int64_t ld, int nrows, int ncols, int row0) {
    int64_t span = ((int64_t)(nrows - row0 - 1) * ld + ncols) * 2;
    if (span > (int64_t)kOob - 1) span = (int64_t)kOob - 1;
    return Rsrc{X + (int64_t)row0 * ld, (int)span};
}

// LDS layout of one staged operand block (256 rows x KS halves) as 16-byte
// chunks, CPR = KS / 8 per row, chunk c of row r at slot r*CPR + (c ^ f(r)):
//   KS = 64: f(r) = (r & 7) ^ ((r >> 3) & 1)
//   KS = 32: f(r) = ((r >> 1) ^ (r >> 3)) & 3
// For the 128-bit fragment reads (32 consecutive rows at one chunk per
// half-wave) both keep every 8-lane and every 16-lane group on distinct
// 16-byte bank groups, whether LDS is served 128 or 256 bytes per pass.
template <int KS>
struct Lds {
    static constexpr int kCpr = KS / 8;
    static constexpr int kBlock = 256 * kCpr;          // chunks per operand block
    static constexpr int kStage = 2 * kBlock;          // A block then B block
    __device__ static __forceinline__ int swz(int r) {
        return KS == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : (((r >> 1) ^ (r >> 3)) & 3);
    }
    __device__ static __forceinline__ int slot(int r, int c) { return r * kCpr + (c ^ swz(r)); }
};

template <int KS>
__device__ __forceinline__ void read_frags(half8 (&fa)[4], half8 (&fb)[4], const u32x4* __restrict__ sA,
                                           const u32x4* __restrict__ sB, int wm, int wn, int lane, int kk) {
    const int r32 = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        fa[i] = __builtin_bit_cast(half8, sA[Lds<KS>::slot(wm * 128 + i * 32 + r32, kk * 2 + khalf)]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        fb[j] = __builtin_bit_cast(half8, sB[Lds<KS>::slot(wn * 128 + j * 32 + r32, kk * 2 + khalf)]);
}

// Per-lane source offsets of the 2 * CPR load instructions of a K step (A's
// CPR, then B's). A wave instruction j fills LDS slots (4j + w) * 64 + L.
//  * K-contiguous operand (A; B stored N x K): slot -> row (256 / CPR) * j +
//    tid / CPR, physical chunk tid % CPR, which must hold logical chunk
//    (tid % CPR) ^ f(row); f(row) does not depend on j. The K step advances
//    the scalar offset by KS * 2 bytes.
//  * B stored K x N, kept N-contiguous ([k][n], 32 chunks of 8 n per k row):
//    slot -> k row 8j + (tid >> 5), physical chunk tid & 31, holding logical
//    chunk g^-1 of it (see KnLds). The K step advances the scalar offset by
//    KS * ldb * 2 bytes; k rows past K lie past the buffer and read zeros.
// voff[idx] is the row's byte offset plus the chunk's, with kOob set when the
// row lies past its operand. tail_oob is kOob when this lane's A chunk lies
// past K on the last, partial K step (0 otherwise).
template <int KS>
struct LaneLoads {
    static constexpr int kCpr = KS / 8;
    unsigned voff[2 * kCpr];
    unsigned tail_oob;
    unsigned kchunk;      // k offset (elements) of this lane's K-contiguous chunk inside a K step
};

// B stored K x N in LDS as [k][n]: 16-byte chunk c (n = 8c .. 8c+7) of k row
// k sits at physical chunk c ^ 2(k & 3) ^ 8((c >> 1) & 1). For the
// transposing fragment reads (16 lanes: 4 k rows x 32 contiguous bytes) this
// keeps every 16- and 32-lane group on distinct banks.
struct KnLds {
    __device__ static __forceinline__ int phys(int c, int k) { return c ^ (2 * (k & 3)) ^ (8 * ((c >> 1) & 1)); }
    __device__ static __forceinline__ int logical(int p, int k) {
        return p ^ (2 * (k & 3)) ^ (8 * (((p >> 1) & 1) ^ (k & 1)));
    }
};

template <int KS, int NXK>
__device__ __forceinline__ LaneLoads<KS> lane_loads(const Args& a, int m0, int n0, int tid) {
    constexpr int kCpr = KS / 8;
    LaneLoads<KS> p;
    const int r = tid / kCpr;
    const unsigned chunk = (unsigned)((tid % kCpr) ^ Lds<KS>::swz(r));
#pragma unroll
    for (int j = 0; j < kCpr; ++j) {
        const int row = r + (256 / kCpr) * j;
        p.voff[j] = ((unsigned)row * (unsigned)a.lda * 2u + chunk * 16u) | (m0 + row < a.M ? 0u : kOob);
        if (NXK) {
            p.voff[kCpr + j] = ((unsigned)row * (unsigned)a.ldb * 2u + chunk * 16u) | (n0 + row < a.N ? 0u : kOob);
        } else {
            const int krow = 8 * j + (tid >> 5);
            const unsigned c = (unsigned)KnLds::logical(tid & 31, krow);
            p.voff[kCpr + j] = (unsigned)krow * (unsigned)a.ldb * 2u + c * 16u;
        }
    }
    const int krem = a.K % KS;             // valid k of the last step (0: the last step is full)
    p.tail_oob = (krem != 0 && (int)chunk * 8 >= krem) ? kOob : 0u;
    p.kchunk = chunk * 8u;
    return p;
}

// Load instruction `idx` (0 .. 2*CPR-1) of a K step into `stage`, with the
// step's scalar offsets (soa for A, sob for B) and this lane's extra
// out-of-range bit `oob` for its K-contiguous chunks.
template <int KS, int NXK>
__device__ __forceinline__ void issue_load(const Rsrc& ra, const Rsrc& rb, const LaneLoads<KS>& p, int idx,
                                           unsigned soa, unsigned sob, unsigned oob, u32x4* __restrict__ stage,
                                           int wave) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass cannot instantiate these target builtins
    constexpr int kCpr = KS / 8;
    const bool isb = idx >= kCpr;
    const int j = isb ? idx - kCpr : idx;
    const Rsrc& rs = isb ? rb : ra;
    // word 3 = 0x00020000: raw (untyped) access, 32-bit data format
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)rs.base, 0, rs.nrec, 0x00020000);
    u32x4* dst = stage + (isb ? Lds<KS>::kBlock : 0) + (j * 4 + wave) * 64;
    // chunks past K: A, and B when it is K-contiguous (a K x N B's rows past K lie past its buffer)
    const unsigned v = (isb && !NXK) ? p.voff[idx] : (p.voff[idx] | oob);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, v, isb ? sob : soa, 0, 0);
#endif
}

// Eight binary16 values, p[e] for e < nv and zero past nv, as one 16-byte
// LDS chunk.
__device__ __forceinline__ u32x4 chunk_from(const uint16_t* __restrict__ p, int nv) {
    unsigned w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const unsigned lo = (2 * q < nv) ? (unsigned)p[2 * q] : 0u;
        const unsigned hi = (2 * q + 1 < nv) ? (unsigned)p[2 * q + 1] : 0u;
        w[q] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Last K step (k0 = its first k): the 16-byte chunks that straddle the end
// of valid data. A chunk straddling K (A, and B stored N x K) was loaded
// whole, so past K it holds the next row's elements; and in an operand's
// final row the range check zeroes a straddling access entirely. Each lane
// rebuilds such chunks of its own slots from element loads - the valid part,
// zeros after it - once its loads have landed and before the barrier that
// publishes the stage. B stored K x N straddles only at column N, and only
// its final row K - 1 loses data (other rows read the next row past N,
// which lands in output columns that are never stored).
template <int KS, int NXK>
__device__ __forceinline__ void fix_last_step(u32x4* __restrict__ stage, const LaneLoads<KS>& p, const Args& a,
                                              int m0, int n0, int k0, int tid, int wave, int lane) {
    constexpr int kCpr = KS / 8;
    const int r = tid / kCpr;
    const int kc = k0 + (int)p.kchunk;
    const int nv = a.K - kc;                          // valid elements of this lane's K chunk
    if (nv > 0 && nv < 8) {
#pragma unroll
        for (int j = 0; j < kCpr; ++j) {
            const int row = r + (256 / kCpr) * j;
            const int slot = (j * 4 + wave) * 64 + lane;
            if (m0 + row < a.M) stage[slot] = chunk_from(a.A + (int64_t)(m0 + row) * a.lda + kc, nv);
            if (NXK && n0 + row < a.N)
                stage[Lds<KS>::kBlock + slot] = chunk_from(a.B + (int64_t)(n0 + row) * a.ldb + kc, nv);
        }
    }
    if (!NXK) {
#pragma unroll
        for (int j = 0; j < kCpr; ++j) {
            const int krow = 8 * j + (tid >> 5);
            const int c = KnLds::logical(tid & 31, krow);
            const int nc = n0 + 8 * c;
            const int nvn = a.N - nc;
            if (k0 + krow == a.K - 1 && nvn > 0 && nvn < 8)
                stage[Lds<KS>::kBlock + (j * 4 + wave) * 64 + lane] =
                    chunk_from(a.B + (int64_t)(a.K - 1) * a.ldb + nc, nvn);
        }
    }
    TG_COMPILER_FENCE();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_waitcnt(0);                    // element loads returned and written
    TG_COMPILER_FENCE();
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four k values (k0 .. k0+3, from 4 k rows) of one n column of B stored
// [k][n] in LDS, by the transposing read: in each 16-lane group, lane i
// points at k row k0 + i/4, columns n0 + 4(i % 4) .. +3, and lane j receives
// column n0 + j.
__device__ __forceinline__ s16x4 read_tr(const u32x4* __restrict__ sB, int krow, int ncol) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int c = ncol >> 3;
    const int byte = krow * 512 + KnLds::phys(c, krow) * 16 + (ncol & 7) * 2;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) char*)(sB) + byte));
#else
    return s16x4{};
#endif
}

// One k16 slice: 16 MFMAs on the current fragments, with the next slice's
// fragment reads and (when LOADS) kHalf = CPR load instructions placed
// between them, reads first, in the order the next slice consumes them:
// A0, B0..B3, A1..A3. A K-contiguous B fragment is one 128-bit read; a
// [k][n] B fragment is two transposing 64-bit reads (k +0..3, k +4..7), so
// that layout has 12 reads per slice and CPR must be 4. The newest read is
// at least four MFMAs old when the slice ends. With one wave per SIMD every
// other instruction competes with MFMA issue, so the order is pinned at both
// the IR and the machine level.
template <int KS, int NXK, bool LOADS>
__device__ __forceinline__ void slice(acc16 (&acc)[4][4], const half8 (&fa)[4], const half8 (&fb)[4],
                                      half8 (&na)[4], half8 (&nb)[4], const u32x4* __restrict__ rA,
                                      const u32x4* __restrict__ rB, int wm, int wn, int lane, int next_kk,
                                      const Rsrc& ra, const Rsrc& rb, const LaneLoads<KS>& p, int ld_first,
                                      unsigned soa, unsigned sob, unsigned oob, u32x4* __restrict__ ld_stage,
                                      int wave) {
    constexpr int kHalf = KS / 8;
    constexpr int kReads = NXK ? 8 : 12;
    static_assert(kReads + kHalf <= 16, "reads and loads must fit the 16 MFMA slots");
    const int r32 = lane & 31, khalf = lane >> 5;
    s16x4 lo[4];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = q >> 2, j = q & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        if (q < kReads) {
            // read slot q -> fragment: NxK: A0,B0,B1,B2,B3,A1,A2,A3; KxN: A0,B0h0,B0h1,...,B3h1,A1,A2,A3
            const int nbr = NXK ? 4 : 8;
            if (q >= 1 && q <= nbr) {
                if (NXK) {
                    nb[q - 1] = __builtin_bit_cast(
                        half8, rB[Lds<KS>::slot(wn * 128 + (q - 1) * 32 + r32, next_kk * 2 + khalf)]);
                } else {
                    const int fbi = (q - 1) >> 1, h = (q - 1) & 1;
                    const int g = lane >> 4, jl = lane & 15;
                    const int ncol = wn * 128 + fbi * 32 + 16 * (g & 1) + 4 * (jl & 3);
                    const int krow = next_kk * 16 + 8 * (g >> 1) + 4 * h + (jl >> 2);
                    const s16x4 v = read_tr(rB, krow, ncol);
                    if (h == 0) {
                        lo[fbi] = v;
                    } else {
                        nb[fbi] = __builtin_bit_cast(half8, __builtin_shufflevector(lo[fbi], v, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                }
            } else {
                const int ai = q == 0 ? 0 : q - nbr;
                na[ai] = __builtin_bit_cast(half8, rA[Lds<KS>::slot(wm * 128 + ai * 32 + r32, next_kk * 2 + khalf)]);
            }
        } else if (LOADS && q - kReads < kHalf) {
            issue_load<KS, NXK>(ra, rb, p, ld_first + (q - kReads), soa, sob, oob, ld_stage, wave);
        }
        TG_COMPILER_FENCE();
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Tile kernel with both operands streamed straight into an S-stage LDS
// ring of KS-deep K steps: A K-contiguous, B either K-contiguous (stored
// N x K, NXK = 1) or kept [k][n] and transposed on read (stored K x N).
// Step t's loads go into stage t mod S in two halves: the first right after
// the barrier that ends every wave's reads of that stage (during the last
// k16 slice of step t - S), the second during the first slice of step
// t - S + 1. Each step's loads thus have about S - 1 steps of compute to
// land. The barrier sits before the last slice of a step: the next step's
// first fragment reads overlap that slice's MFMAs. Every step issues the
// same number of loads (steps past K read nothing and write zeros into
// stages that are never read), so all wait counts are constants.
template <int NXK, bool VEC_C, int KS, int S>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(1, 1)))
tgemm_f16_dma_kernel(Args a) {
    using L = Lds<KS>;
    static_assert(KS == 64 || KS == 32, "K step");
    static_assert(NXK || KS == 32, "B stored K x N streams 32-deep K steps");
    static_assert(S >= 2 && S <= 5 && S * L::kStage * 16 <= 160 * 1024, "LDS ring must fit 160 KiB");
    constexpr int kSlices = KS / 16;                 // k16 slices per step (even)
    constexpr int kCpr = KS / 8;
    constexpr int kLps = 2 * kCpr;                   // load instructions per step per wave
    __shared__ u32x4 smem[S * L::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_of((int)blockIdx.x, a.W, a.grid_m, a.grid_n, a.group_m, a.num_xcd, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (a.K + KS - 1) / KS;

    acc16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = acc16{};

    if (nk > 0) {
        const Rsrc ra = operand_rsrc(a.A, a.lda, a.M, a.K, m0);
        // B: N x K rows n0.. ; K x N columns n0.. of all K rows
        const Rsrc rb = NXK ? operand_rsrc(a.B, a.ldb, a.N, a.K, n0) : operand_rsrc(a.B + n0, a.ldb, a.K, a.N - n0, 0);
        const LaneLoads<KS> p = lane_loads<KS, NXK>(a, m0, n0, tid);
        const unsigned bstep = NXK ? (unsigned)(KS * 2) : (unsigned)KS * (unsigned)a.ldb * 2u;
        // scalar offsets and A's extra out-of-range bits of K step t
#define TG_SOA(t) ((t) < nk ? (unsigned)(t) * (unsigned)(KS * 2) : kOob)
#define TG_SOB(t) ((t) < nk ? (unsigned)(t) * bstep : kOob)
#define TG_OOB(t) ((t) == nk - 1 ? p.tail_oob : 0u)

        // prologue: steps 0 .. S-2 and the first half of step S-1
        for (int t = 0; t < S; ++t) {
            u32x4* stage = smem + t * L::kStage;
            const int n = (t + 1 < S) ? kLps : kCpr;
            for (int idx = 0; idx < n; ++idx)
                issue_load<KS, NXK>(ra, rb, p, idx, TG_SOA(t), TG_SOB(t), TG_OOB(t), stage, wave);
        }
        // the last step has chunks straddling the end of valid data
        const bool straddle = (a.K % 8) != 0 || (!NXK && (a.N % 8) != 0);
        const int klast = (nk - 1) * KS;
        wait_vmcnt<(S - 2) * kLps + kCpr>();          // step 0 landed
        if (straddle && nk == 1) fix_last_step<KS, NXK>(smem, p, a, m0, n0, klast, tid, wave, lane);
        block_barrier();

        half8 fa[2][4], fb[2][4];
        read_frags<KS>(fa[0], fb[0], smem, smem + L::kBlock, wm, wn, lane, 0);
        if (!NXK) {
            const int g = lane >> 4, jl = lane & 15;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int ncol = wn * 128 + f * 32 + 16 * (g & 1) + 4 * (jl & 3);
                const int krow = 8 * (g >> 1) + (jl >> 2);
                const s16x4 v0 = read_tr(smem + L::kBlock, krow, ncol);
                const s16x4 v1 = read_tr(smem + L::kBlock, krow + 4, ncol);
                fb[0][f] = __builtin_bit_cast(half8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
        int st = 0;                                   // stage of step t
        for (int t = 0; t < nk; ++t) {
            const u32x4* sA = smem + st * L::kStage;
            const u32x4* sB = sA + L::kBlock;
            const int pst = (st == 0) ? S - 1 : st - 1;   // stage of step t + S - 1
            const int nst = (st + 1 == S) ? 0 : st + 1;
            // slice 0 carries the second half of step t + S - 1's loads
            slice<KS, NXK, true>(acc, fa[0], fb[0], fa[1], fb[1], sA, sB, wm, wn, lane, 1, ra, rb, p, kCpr,
                                 TG_SOA(t + S - 1), TG_SOB(t + S - 1), TG_OOB(t + S - 1), smem + pst * L::kStage,
                                 wave);
#pragma unroll
            for (int kk = 1; kk + 1 < kSlices; ++kk)
                slice<KS, NXK, false>(acc, fa[kk & 1], fb[kk & 1], fa[(kk + 1) & 1], fb[(kk + 1) & 1], sA, sB, wm,
                                      wn, lane, kk + 1, ra, rb, p, 0, 0u, 0u, 0u, smem, wave);
            TG_COMPILER_FENCE();
            wait_lgkmcnt0();                          // this wave's reads of stage st returned
            wait_vmcnt<(S - 2) * kLps>();             // step t + 1 landed
            if (straddle && t + 2 == nk)
                fix_last_step<KS, NXK>(smem + nst * L::kStage, p, a, m0, n0, klast, tid, wave, lane);
            block_barrier();
            // the first half of step t + S's loads goes into the stage just released
            const u32x4* nA = smem + nst * L::kStage;
            slice<KS, NXK, true>(acc, fa[(kSlices - 1) & 1], fb[(kSlices - 1) & 1], fa[0], fb[0], nA,
                                 nA + L::kBlock, wm, wn, lane, 0, ra, rb, p, 0, TG_SOA(t + S), TG_SOB(t + S),
                                 TG_OOB(t + S), smem + st * L::kStage, wave);
            st = nst;
        }
        // no load may still be writing this workgroup's LDS when it exits
        wait_vmcnt<0>();
#undef TG_SOA
#undef TG_SOB
#undef TG_OOB
    }
    store_c<VEC_C>(acc, a, m0, n0, wm, wn, lane);
}

template <int NXK, bool VEC, bool VEC_C>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(1, 1)))
tgemm_f16_kernel(Args a) {
    __shared__ u32x4 smem[2][2][kTileChunks];   // [stage][A | B], 128 KiB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_of((int)blockIdx.x, a.W, a.grid_m, a.grid_n, a.group_m, a.num_xcd, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool interior = (m0 + BM <= a.M) && (n0 + BN <= a.N);
    const int nk = (a.K + BK - 1) / BK;

    acc16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = acc16{};

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
        mma_step(acc, smem[cur][0], smem[cur][1], wm, wn, lane);
        if (more) store_stage<NXK>(smem[cur ^ 1][0], smem[cur ^ 1][1], ra, rb, tid);
        __syncthreads();
    }
    store_c<VEC_C>(acc, a, m0, n0, wm, wn, lane);
}

template <int NXK, bool VEC, bool VEC_C>
static const void* kernel_ptr() {
    return reinterpret_cast<const void*>(&tgemm_f16_kernel<NXK, VEC, VEC_C>);
}

template <bool VEC_C>
static const void* dma_kernel_ptr(int nxk, int k_step, int stages) {
    if (!nxk) {
        switch (stages) {
            case 2: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<0, VEC_C, 32, 2>);
            case 3: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<0, VEC_C, 32, 3>);
            case 4: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<0, VEC_C, 32, 4>);
            default: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<0, VEC_C, 32, 5>);
        }
    }
    if (k_step == 64) return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<1, VEC_C, 64, 2>);
    switch (stages) {
        case 2: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<1, VEC_C, 32, 2>);
        case 3: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<1, VEC_C, 32, 3>);
        case 4: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<1, VEC_C, 32, 4>);
        default: return reinterpret_cast<const void*>(&tgemm_f16_dma_kernel<1, VEC_C, 32, 5>);
    }
}

static const void* pick_kernel(const Plan& pl) {
    const int variant = pl.variant;
    if (variant & kDma)
        return (variant & kVecC) ? dma_kernel_ptr<true>(pl.layout, pl.k_step, pl.stages)
                                 : dma_kernel_ptr<false>(pl.layout, pl.k_step, pl.stages);
    switch (variant & 7) {
        case 0: return kernel_ptr<0, false, false>();
        case 1: return kernel_ptr<0, true, false>();
        case 2: return kernel_ptr<0, false, true>();
        case 3: return kernel_ptr<0, true, true>();
        case 4: return kernel_ptr<1, false, false>();
        case 5: return kernel_ptr<1, true, false>();
        case 6: return kernel_ptr<1, false, true>();
        default: return kernel_ptr<1, true, true>();
    }
}

static thread_local int g_last_hip_error = 0;

}  // namespace tg

extern "C" int tgemm_f16_config(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, int b_layout, void* C, int64_t ldc,
                                void* stream, int force_generic, int group_m, int num_xcd, int k_step,
                                int stages) {
    tg::Plan pl;
    const int rc = tg::make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, force_generic, group_m,
                                 num_xcd, k_step, stages, &pl);
    if (rc != TGEMM_OK) return rc;
    if (pl.M == 0 || pl.N == 0) return TGEMM_OK;
    tg::Args args;
    args.A = static_cast<const uint16_t*>(A);
    args.B = static_cast<const uint16_t*>(B);
    args.C = static_cast<uint16_t*>(C);
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
    const void* fn = tg::pick_kernel(pl);
    if (!fn) return TGEMM_ERR_UNSUPPORTED;
    void* kargs[] = {&args};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)pl.W),
                                         dim3(tg::NTHREADS), kargs, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        tg::g_last_hip_error = (int)e;
        return TGEMM_ERR_HIP;
    }
    return TGEMM_OK;
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

extern "C" int tgemm_plan_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, int b_layout, void* C, int64_t ldc, int force_generic,
                              int group_m, int num_xcd, int k_step, int stages, int64_t* info) {
    if (!info) return TGEMM_ERR_INVALID;
    tg::Plan pl;
    const int rc = tg::make_plan(M, N, K, A, lda, B, ldb, b_layout, C, ldc, force_generic, group_m,
                                 num_xcd, k_step, stages, &pl);
    if (rc != TGEMM_OK) return rc;
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
    return TGEMM_OK;
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
