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
