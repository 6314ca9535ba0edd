/*
 * tgemm: dense tiled matrix product C = A * B on AMD Instinct MI355X
 * (gfx950), binary16 in and out (tgemm_f16), with bfloat16 or binary32
 * inputs, bfloat16 or fp32 output and a scale / bias / activation epilogue
 * (tgemm_gemm).
 * C ABI: plain pointers and sizes, no HIP or framework types.
 *
 * The operation (page 1, "Using NVIDIA CUDA Tile to write a high-performance
 * matrix multiply", section "What is matrix multiplication?"): for A of M x K
 * and B of K x N, C[i][j] = sum over k of A[i][k] * B[k][j].
 * Numerics follow the pages' tile kernels (page 1, sections 4-6; page 4,
 * CUDA programming guide 13.4.2, chapter "Writing tile kernels", section
 * 2.4.9.1 "Matrix multiplication"): binary16 inputs, fp32 accumulation,
 * conversion to binary16 (round to nearest even) only when C is stored,
 * partial K tiles padded with zeros, out-of-range C elements never written.
 * Each workgroup owns one output tile and walks K tile by tile.
 *
 * Storage (all row-major, element strides in units of 16-bit elements):
 *   A: M x K,  element (i, k) at A[i*lda + k]
 *   B: b_layout TGEMM_B_KxN: K x N, element (k, j) at B[k*ldb + j]
 *      b_layout TGEMM_B_NxK: N x K, element (k, j) at B[j*ldb + k]
 *         (C = A * B^T when B is viewed as the N x K array it is stored as)
 *   C: M x N,  element (i, j) at C[i*ldc + j]
 * A, B, C point to device memory holding IEEE 754 binary16 bit patterns.
 *
 * Ownership: the caller owns all three buffers. The library allocates no
 * device memory and keeps no pointer after a call returns.
 *
 * Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL means the
 * default stream) and the call returns without waiting. C is valid once the
 * stream has been synchronized. A and B are only read.
 *
 * Errors: nothing is printed and nothing is thrown across the ABI. A call
 * that returns TGEMM_ERR_INVALID or TGEMM_ERR_UNSUPPORTED has enqueued no
 * work. TGEMM_ERR_HIP means the HIP runtime refused the launch; its
 * hipError_t value is available from tgemm_last_hip_error() on the calling
 * thread.
 */
#ifndef TGEMM_H_
#define TGEMM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TGEMM_B_KxN = 0, TGEMM_B_NxK = 1 } tgemm_b_layout;

/* Element types: IEEE 754 binary16, bfloat16 (the upper 16 bits of a
 * binary32), IEEE 754 binary32. */
typedef enum { TGEMM_F16 = 0, TGEMM_BF16 = 1, TGEMM_F32 = 2 } tgemm_dtype;

/* Activation applied by the epilogue of tgemm_gemm. */
typedef enum { TGEMM_ACT_NONE = 0, TGEMM_ACT_RELU = 1 } tgemm_act;

enum {
    TGEMM_OK = 0,
    TGEMM_ERR_INVALID = -1,     /* argument check failed; nothing enqueued */
    TGEMM_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels cover  */
    TGEMM_ERR_HIP = -3          /* the HIP runtime reported an error       */
};

/*
 * C = A * B (binary16 in, fp32 accumulate, binary16 out) on `stream`.
 *
 * Argument checks (TGEMM_ERR_INVALID, nothing enqueued) - the call fails if:
 *   M, N or K is negative or above 2^31 - 1;
 *   lda < max(1, K); ldb < max(1, N) for KxN or < max(1, K) for NxK;
 *   ldc < max(1, N); b_layout is neither TGEMM_B_KxN nor TGEMM_B_NxK;
 *   a pointer is NULL while its operand holds at least one element;
 *   a pointer is not 2-byte aligned;
 *   the memory spanned by C overlaps the memory spanned by A or B.
 * Degenerate shapes: M == 0 or N == 0 is a successful no-op. K == 0 writes
 * zeros to the M x N region of C (the accumulator starts at zero and the K
 * walk runs zero times).
 * Alignment: any 2-byte-aligned operand works. When K > 0 and both operand
 * row strides are at least 8 elements and small enough for 32-bit offsets,
 * A and B stream into LDS by 16-byte loads at any 2-byte alignment (rows that
 * start 16-byte aligned run faster, and rows that start 128-byte aligned,
 * a stride that is a multiple of 64 elements, fastest); otherwise they are
 * staged through registers with 128-bit or element loads. C is written with
 * 16-byte stores at any 2-byte alignment (element stores at its right edge;
 * 8-byte or element stores when a byte offset within 128 rows of C would
 * exceed 2^31), streamed past the caches where C's base and row pitch are
 * multiples of 128 bytes and through the L2 otherwise.
 * C must not alias A or B (page 4, section 2.4.12.1: restrict-qualified
 * operands must not overlap).
 */
int tgemm_f16(int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda,
              const void* B, int64_t ldb, int b_layout,
              void* C, int64_t ldc,
              void* stream);

/*
 * Same as tgemm_f16 with explicit launch choices, for tests and tuning.
 *   force_generic: 1 = use element-wise operand loads even where 128-bit
 *                  loads are possible (same results); 0 = automatic.
 *   group_m:       tile-rows per raster group (page 1, section "Swizzle",
 *                  GROUP_SIZE_M, counted in its 128-row tiles); 0 = default
 *                  (4 of these 256-row tiles: the same 1024 rows as the
 *                  page's 8); 1..1024 otherwise.
 *   num_xcd:       number of dies the workgroups are spread over for the
 *                  die-aware renumbering; 0 = default (the device's compute
 *                  units / 32, from 1 to 8: 8 on a whole MI355X, fewer on
 *                  a partitioned one); 1 disables the renumbering; 1..64
 *                  otherwise.
 *   k_step:        K depth of one LDS stage of the direct-to-LDS path
 *                  (used whenever K > 0 and both row strides are at least
 *                  8 elements and small enough for 32-bit offsets):
 *                  0 = default (64, or 32 when stages > 2 or K <= 64),
 *                  32 or 64 (64 needs K > 64).
 *   stages:        LDS ring depth of that path: 0 = default (2 at k_step 64,
 *                  4 at k_step 32, 3 for the smaller tiles), 2..5 (k_step
 *                  64 allows only 2; the smaller tiles 2..3, producer/
 *                  consumer workgroups 3..6). Other paths ignore k_step and
 *                  stages. With every launch choice 0 and no tuned choice
 *                  recorded, 16-bit operands with B stored K x N, K > 64
 *                  not a multiple of 64 and at most one tile per compute
 *                  unit run at k_step 32 (default depth).
 *   tile_m:        output tile rows of that path (page 2, section 7.4 tunes
 *                  the tile shape): 0 = automatic, 256, 128 or 64. Tiles of
 *                  128 or 64 rows (x 256 columns) run two workgroups per
 *                  compute unit with 32-deep steps. Automatic (with every
 *                  other launch choice 0 and no tuned choice): 256 rows,
 *                  except where a grid of 256-row tiles would fill at most
 *                  half of the compute units (128 rows) or at most a
 *                  quarter (64 rows); binary32 operands follow their own
 *                  rule (tgemm_gemm). Other paths accept only 0 and 256
 *                  (else TGEMM_ERR_UNSUPPORTED).
 *   producers:     0, or 4: producer/consumer workgroups (page 5, Croqtile
 *                  tutorial "dense GEMM fp16 from naive", section "Kernel 3:
 *                  warp specialization"): 8 waves, 4 of which only load
 *                  operands into LDS and 4 only compute, on 128 x 256 tiles
 *                  with 32-deep steps (tile_m 0 or 128).
 * Out-of-range choices return TGEMM_ERR_INVALID. Every choice computes the
 * same C bit for bit (each output's k order is fixed by its tile position).
 */
int tgemm_f16_config(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb, int b_layout,
                     void* C, int64_t ldc,
                     void* stream,
                     int force_generic, int group_m, int num_xcd,
                     int k_step, int stages, int tile_m, int producers);

/*
 * C = act(alpha * A * B + bias) with a choice of element types, on `stream`.
 *
 * The pages' tile kernels take their element types as parameters: inputs
 * of two bytes (binary16 or bfloat16) share one tile configuration and
 * binary32 inputs get another (page 1, section "Step 2: set the tile size"),
 * and the guide's example accumulates
 * binary16 products in fp32 and stores an fp32 C (page 4, section 2.4.9.1);
 * production GEMMs fuse work on the output into the store (page 5, Croqtile
 * tutorial "dense GEMM fp16 from naive", section "SOTA comparison": epilogue
 * fusion).
 * For every output element, in fp32 after the fp32 accumulation:
 *   v = alpha * sum_k A[i][k] * B[k][j] + bias[j]   (one fused multiply-add)
 *   v = max(v, 0) if act == TGEMM_ACT_RELU (a NaN stays NaN)
 * then v is converted to c_type with round to nearest even (an fp32 C gets
 * v itself). alpha == 1, bias == NULL and act == TGEMM_ACT_NONE store the
 * sums exactly as tgemm_f16 does (for binary16 in and out: the same bits).
 *
 *   ab_type: TGEMM_F16, TGEMM_BF16 or TGEMM_F32, the type of both A and B
 *            (lda and ldb count elements of that type; binary32 operands
 *            must be 4-byte aligned). Binary32 operands run on
 *            v_mfma_f32_16x16x4_f32 with fp32 accumulation in 16-deep K
 *            steps. With K > 0 and row strides of 4 to 2,000,000 floats
 *            they take the direct-to-LDS kernel of the 16-bit types on their
 *            bytes (both B layouts): tiles
 *            of 256, 128 or 64 rows, an LDS ring of 2 (default), 3 or 4
 *            stages at 256 rows and 3 for the smaller tiles; automatic
 *            launches take 64-row tiles unless 256-row tiles fill at least
 *            7/8 of their rounds over the compute units. Otherwise a general
 *            kernel staged through registers (256 x 256 tiles, 2 stages). The
 *            k_step choice of tgemm_gemm_config does not apply to binary32
 *            operands (a plan reports 16).
 *   c_type:  TGEMM_F16, TGEMM_BF16 or TGEMM_F32; ldc counts elements of
 *            that type (C[i*ldc + j]).
 *   bias:    NULL, or N fp32 values in device memory (4-byte aligned),
 *            added to every row; only read.
 * Storage, ownership, asynchrony and the remaining argument checks are those
 * of tgemm_f16, with these in addition (TGEMM_ERR_INVALID, nothing enqueued):
 * ab_type or c_type or act out of range; A, B or C not aligned to its
 * element size;
 * bias not 4-byte aligned; the bias overlapping C.
 * K == 0 stores act(bias[j]) (zero sums, scaled, plus the bias).
 */
int tgemm_gemm(int64_t M, int64_t N, int64_t K,
               int ab_type, const void* A, int64_t lda,
               const void* B, int64_t ldb, int b_layout,
               int c_type, void* C, int64_t ldc,
               float alpha, const float* bias, int act,
               void* stream);

/*
 * tgemm_gemm with the launch choices of tgemm_f16_config (same meaning and
 * ranges). The binary16-in, binary16-out product without epilogue is built
 * for every K step, ring depth and tile choice listed there (producer/
 * consumer workgroups with 3 or 5 stages); every other 16-bit combination
 * for the default ring depth of each K step (2 stages at 64, 4 at 32) and of
 * the 128- and 64-row tiles (3), without producer/consumer workgroups;
 * binary32 operands as listed under tgemm_gemm. Other choices return
 * TGEMM_ERR_UNSUPPORTED for the combination, with nothing enqueued.
 */
int tgemm_gemm_config(int64_t M, int64_t N, int64_t K,
                      int ab_type, const void* A, int64_t lda,
                      const void* B, int64_t ldb, int b_layout,
                      int c_type, void* C, int64_t ldc,
                      float alpha, const float* bias, int act,
                      void* stream,
                      int force_generic, int group_m, int num_xcd,
                      int k_step, int stages, int tile_m, int producers);

/*
 * Runtime tuning, per problem shape (page 2, "CUDA 13.1 new feature: the Tile
 * programming model", section 7.4 "Autotuning": several tile configurations
 * are tried, the fastest is kept per problem shape, and later calls reuse it
 * at no cost).
 *
 * tgemm_tune_gemm takes the arguments of tgemm_gemm and runs the problem on
 * the caller's buffers under each launch choice that leaves the result
 * unchanged bit for bit: the tile rows, K step, LDS ring depth and
 * producer/consumer choice of the direct-to-LDS pipeline (those built for
 * the types) and a raster group height of 4, 8 or 16 tile rows. Each choice runs once; then the untuned launch runs for about
 * 100 ms of GPU time (at most 4096 launches) so that the power-limited clock
 * settles; then every choice runs `rounds` times (1..100), interleaved with the
 * others (round r starts at a different choice), timed with HIP events on
 * `stream`. The choice with the smallest median time is recorded for the
 * problem's key on the current device, unless it is less than 1% faster than
 * the untuned launch, which is then recorded instead. The key is everything that selects a kernel: M, N, K, the
 * three strides, b_layout, both types, whether an epilogue is requested, and
 * the alignment classes of A, B and C. From then on, tgemm_gemm, tgemm_f16,
 * the *_config calls with all five launch choices 0, and the plan queries use
 * the recorded choice for that key.
 *
 * Synchronizes `stream` (not for use under graph capture). C holds the
 * product on return, as after tgemm_gemm (every choice computes the same
 * bits). Creates and destroys HIP events; allocates no device memory.
 * info: NULL or 8 values: the chosen k_step, stages, group_m, num_xcd, its
 * median launch time in ns, the number of choices tried, and the chosen
 * tile rows and producer waves.
 * Returns the argument errors of tgemm_gemm (nothing run), TGEMM_ERR_INVALID
 * for rounds outside 1..100, or TGEMM_ERR_HIP. M == 0 or N == 0: nothing is
 * run or recorded (info all 0). The table is shared by all threads.
 */
int tgemm_tune_gemm(int64_t M, int64_t N, int64_t K,
                    int ab_type, const void* A, int64_t lda,
                    const void* B, int64_t ldb, int b_layout,
                    int c_type, void* C, int64_t ldc,
                    float alpha, const float* bias, int act,
                    void* stream, int rounds, int64_t* info);

/* Number of problem keys with a recorded choice (all devices). */
int tgemm_tuning_entries(void);

/* Forget every recorded choice; later calls use the default launch choices. */
void tgemm_tuning_clear(void);

/* Human-readable text of a TGEMM_* status code (static storage). */
const char* tgemm_status_string(int status);

/* hipError_t of the most recent TGEMM_ERR_HIP on the calling thread (0 if none). */
int tgemm_last_hip_error(void);

/*
 * Planning query: the launch tgemm_f16_config would make for these
 * arguments on a device with `compute_units` compute units (256 on MI355X).
 * The plan depends on that count in three places: a launch of 64-deep steps
 * with more tiles than compute units runs one workgroup per compute unit,
 * the automatic tile rows depend on how much of the device a 256-row grid
 * fills, and the automatic 32-deep rule for B stored K x N applies to grids
 * of at most one tile per compute unit.
 *   compute_units: 1..65536, or 0 for the current device's count, read with
 *                  one HIP attribute query once the arguments have passed
 *                  (TGEMM_ERR_HIP when there is no device). With a count
 *                  given, the query makes no HIP call at all (unless a
 *                  tuned choice is recorded, whose key names the current
 *                  device).
 * Returns TGEMM_OK and fills info[0..9]:
 *   info[0] variant bits: bit0 128-bit A/B loads, bit1 vector C stores
 *           (64-bit runs of a 16-bit C, 128-bit runs of an fp32 C), bit2 B
 *           layout is NxK, bit3 the pipelined kernel (operands streamed
 *           directly into LDS)
 *   info[1] tile rows        info[2] tile columns      info[3] K step
 *   info[4] workgroups launched (the tile count ceil(M/BM) * ceil(N/BN), or
 *           compute_units when each workgroup walks several tiles; 0 when
 *           M or N is 0)
 *   info[5] group_m  info[6] num_xcd
 *   info[7] threads per workgroup  info[8] LDS stages  info[9] LDS bytes
 * or the same error tgemm_f16_config would return. `info` must hold 10 values.
 */
int tgemm_plan_f16(int64_t M, int64_t N, int64_t K,
                   const void* A, int64_t lda,
                   const void* B, int64_t ldb, int b_layout,
                   void* C, int64_t ldc,
                   int force_generic, int group_m, int num_xcd,
                   int k_step, int stages, int tile_m, int producers,
                   int compute_units, int64_t* info);

/*
 * Planning query for tgemm_gemm_config: the same compute_units and
 * info[0..9] as tgemm_plan_f16, or the error tgemm_gemm_config would return
 * (including TGEMM_ERR_UNSUPPORTED for a ring depth that is not built for
 * the types).
 */
int tgemm_plan_gemm(int64_t M, int64_t N, int64_t K,
                    int ab_type, const void* A, int64_t lda,
                    const void* B, int64_t ldb, int b_layout,
                    int c_type, void* C, int64_t ldc,
                    float alpha, const float* bias, int act,
                    int force_generic, int group_m, int num_xcd,
                    int k_step, int stages, int tile_m, int producers,
                    int compute_units, int64_t* info);

/*
 * Host-only: the output tile that workgroup `wid` of a grid_m x grid_n tile
 * grid computes, exactly as the kernels compute it (die-aware renumbering,
 * then the grouped order of page 1, section "Swizzle"). Returns TGEMM_OK, or
 * TGEMM_ERR_INVALID for non-positive sizes or wid outside the grid.
 */
int tgemm_tile_of(int64_t grid_m, int64_t grid_n, int group_m, int num_xcd,
                  int64_t wid, int64_t* tile_m, int64_t* tile_n);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H_ */
