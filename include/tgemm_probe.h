/*
 * tgemm_probe: measurement aids for the tgemm library on MI355X (gfx950).
 * Not part of the product operation: a library of its own
 * (libtgemm_probe.so), used by the benchmark and by tests that check what
 * the GEMM's design assumes about the hardware. C ABI, plain pointers and
 * sizes; status codes are those of tgemm.h.
 */
#ifndef TGEMM_PROBE_H_
#define TGEMM_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Matrix-core ceiling probe: launches `workgroups` workgroups of 256 threads
 * that run the GEMM kernel's instruction stream without its
 * synchronization, tile changes or C stores: per wave, `iters` rounds of two
 * slices of 64 independent 16x16x32 fp16 MFMAs, with 16 128-bit LDS fragment
 * reads and 8 direct-to-LDS 16-byte loads per slice (operands drawn from
 * `data`). MI355X is power-limited under MFMA load and the operands'
 * switching activity sets the clock, so with the benchmark's inputs as
 * `data` its TFLOP/s is the ceiling the GEMM's instruction mix reaches on
 * this board.
 *   data:   device memory, 16-byte aligned, data_bytes a power of two in
 *           [1 MiB, 1 GiB]; only read.
 *   out:    device memory for workgroups * 256 floats (sums, written so that
 *           the work is not optimized away).
 *   clocks: NULL, or device memory for 2 * workgroups uint64 values: per
 *           workgroup, the shader-clock cycles (s_memtime) and the 100 MHz
 *           reference ticks (s_memrealtime) that its first wave spent in the
 *           MFMA rounds. Their ratio times 100 MHz is that workgroup's average
 *           clock.
 * Returns TGEMM_OK, TGEMM_ERR_INVALID (bad sizes or pointers, nothing
 * enqueued) or TGEMM_ERR_HIP. Asynchronous on `stream`.
 */
int tgemm_mfma_issue_probe(int64_t workgroups, int iters, const void* data, int64_t data_bytes,
                           float* out, uint64_t* clocks, void* stream);

/*
 * Instruction-stream probes: the GEMM's steady-state instruction stream
 * taken apart, to measure what each part costs the matrix cores (issue
 * slots) and the power-limited clock. Every kind runs, per workgroup and
 * round, the matrix work of one 64-deep step of a 256 x 256 tile (2^23
 * flops; TGEMM_STREAM_F32_GEMM 2^22, two 16-deep binary32 steps), on operands
 * drawn from `data`; loads read 4 KiB windows (8 KiB with 512 threads) that
 * four workgroups of one die share per round. Kinds (256 threads, one wave
 * per SIMD, 8 x 8 blocks of 16x16x32 fp16 per wave, unless stated):
 *   TGEMM_STREAM_F16_MFMA              matrix instructions only
 *   TGEMM_STREAM_F16_READS             + 16 128-bit LDS fragment reads per
 *                                      32-deep slice
 *   TGEMM_STREAM_F16_GEMM              + 16 direct-to-LDS 16-byte loads per
 *                                      round in its second slice; before that
 *                                      slice vmcnt(0), lgkmcnt(0) and a
 *                                      workgroup barrier (the GEMM's stream)
 *   TGEMM_STREAM_F16_GEMM_NO_BARRIER   the same without lgkmcnt(0) and barrier
 *   TGEMM_STREAM_F16_HALF_LOADS        TGEMM_STREAM_F16_GEMM with 8 loads
 *   TGEMM_STREAM_F16_VGPR_LOADS        reads + 16 loads into registers per
 *                                      round, no LDS writes, no waits beyond
 *                                      the use of each a round later
 *   TGEMM_STREAM_F16_LDS_WRITES        reads + 16 ds_write_b128 per round, no
 *                                      global loads
 *   TGEMM_STREAM_F16_32X32             32x32x16 fp16, 4 x 4 blocks: matrix
 *                                      instructions only
 *   TGEMM_STREAM_F16_32X32_GEMM        the same with the reads, loads, waits
 *                                      and barrier of TGEMM_STREAM_F16_GEMM
 *   TGEMM_STREAM_F16_8W_MFMA           512 threads (two waves per SIMD), 4 x
 *                                      8 blocks per wave: matrix instructions
 *   TGEMM_STREAM_F16_8W_GEMM           the same with 12 reads per slice, 8
 *                                      loads per wave per round, waits and
 *                                      barrier
 *   TGEMM_STREAM_F32_GEMM              16x16x4 binary32, each block's four
 *                                      instructions back to back, 16 reads
 *                                      per 16-deep slice (the binary32
 *                                      GEMM's stream without its loads)
 * Arguments, `out` (workgroups * 256 floats, * 512 for the 512-thread kinds)
 * and `clocks` as for tgemm_mfma_issue_probe. Returns TGEMM_OK,
 * TGEMM_ERR_INVALID (unknown kind, bad sizes or pointers; nothing
 * enqueued) or TGEMM_ERR_HIP.
 */
enum {
    TGEMM_STREAM_F16_MFMA = 0,
    TGEMM_STREAM_F16_READS = 1,
    TGEMM_STREAM_F16_GEMM = 2,
    TGEMM_STREAM_F16_GEMM_NO_BARRIER = 3,
    TGEMM_STREAM_F16_HALF_LOADS = 4,
    TGEMM_STREAM_F16_VGPR_LOADS = 5,
    TGEMM_STREAM_F16_LDS_WRITES = 6,
    TGEMM_STREAM_F16_32X32 = 7,
    TGEMM_STREAM_F16_32X32_GEMM = 8,
    TGEMM_STREAM_F16_8W_MFMA = 9,
    TGEMM_STREAM_F16_8W_GEMM = 10,
    TGEMM_STREAM_F32_GEMM = 11
};
int tgemm_mfma_stream_probe(int kind, int64_t workgroups, int iters, const void* data, int64_t data_bytes,
                            float* out, uint64_t* clocks, void* stream);

/*
 * Die probe: launches `workgroups` workgroups of 64 threads; workgroup w
 * writes to out[w] the number (0-15) of the accelerator die (XCD) it ran on,
 * read from the XCC_ID hardware register. The GEMM's die-aware renumbering
 * assumes that the workgroups sharing a die are those with equal w mod
 * num_xcd (page 1, "Using NVIDIA CUDA Tile to write a high-performance
 * matrix multiply", section "Swizzle", gives the grouped order this
 * renumbering feeds). `out`: device memory for `workgroups` ints. Returns
 * TGEMM_OK, TGEMM_ERR_INVALID (workgroups outside [1, 2^20] or a null
 * `out`) or TGEMM_ERR_HIP.
 */
int tgemm_xcd_probe(int64_t workgroups, int* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_PROBE_H_ */
