/*
 * pgemm.h -- C ABI of a tiled GEMM whose K loop is software-pipelined over a
 * ring of LDS stages, for AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Double Buffering: Software Pipelining the K-Loop",
 * section "The Kernel": row-major A, B, C and the fused alpha/beta
 * read-modify-write of C) is
 *
 *     C[i*ldc + j] = alpha * sum_k A[i*lda + k] * B[k*ldb + j] + beta * C[i*ldc + j]
 *
 * for 0 <= i < M, 0 <= j < N.  The K loop runs as a prologue, a steady state
 * and an epilogue over `stages` LDS buffers (page "Software pipelines and
 * asynchronous copies", sections "Prologue, steady state, and epilogue" and
 * "Producer-consumer synchronization"): one readiness barrier per K tile, the
 * loads of tile t+stages-1 in flight while tile t is multiplied.
 *
 * Conventions shared by every entry point:
 *   - Layout: row-major A[M][K], B[K][N], C[M][N] with lda >= K, ldb >= N,
 *     ldc >= N (elements, not bytes).
 *   - dtype: PGEMM_F32 (A, B, C fp32), PGEMM_F16 and PGEMM_BF16 (A, B 16-bit,
 *     C fp32, fp32 accumulation), PGEMM_I8 (A, B int8, C int32, int32
 *     accumulation and int32 two's-complement epilogue; alpha and beta must be
 *     integers in int32 range; sums, products and the result wrap modulo 2^32,
 *     with no saturation, so C is the exact result reduced to int32).
 *   - Pointers A, B, C are device pointers owned by the caller.  The library
 *     allocates nothing and keeps no state besides constant tables.
 *   - beta == 0: C is written without being read (NaN/Inf in C do not
 *     propagate).  K == 0: C = beta*C.  M == 0 or N == 0: nothing happens.
 *   - C must not overlap A or B.
 *   - stream: a hipStream_t (NULL = the default stream).  The call only
 *     enqueues work and returns; completion is observed through the stream.
 *   - Misaligned pointers or leading dimensions are not an error: rows may
 *     start at any element (the copies take element-aligned addresses), and
 *     an operand whose rows are not whole 16-byte chunks is completed by
 *     element loads (A's K tail) or goes through registers (B; slower, same
 *     results) (pgemm_producer).
 *   - 32-bit tile addressing: M, N, K <= 2^31 - 256, lda * elem * 256, ldb *
 *     elem * 128 and ldc * 4 * 256 below 2^31 bytes; otherwise
 *     PGEMM_ERR_TOO_LARGE.
 *   - Return value: PGEMM_OK (0) or a negative pgemm_status.  Argument errors
 *     are detected on the host before anything is enqueued.
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pgemm_dtype {
    PGEMM_F32 = 0,
    PGEMM_F16 = 1,
    PGEMM_BF16 = 2,
    PGEMM_I8 = 3
};

/* Status codes.  Each error is detected on the host before anything is
 * enqueued, except PGEMM_ERR_HIP.  Their sources:
 *   INVALID_ARG, TOO_LARGE -- the indexing of page "Double Buffering:
 *     Software Pipelining the K-Loop", section "The Kernel" (row-major A, B,
 *     C addressed by row * leading dimension + column), generalised to
 *     leading dimensions of at least the row length and bounded by the
 *     kernels' 32-bit tile offsets;
 *   UNSUPPORTED_DTYPE -- the data types of page "GPU-Kernel pipelinen",
 *     section "Eingaben" (FP16, FP32, INT8), with bf16 beside fp16;
 *   BAD_STAGES, INFEASIBLE_PLAN -- the stage counts and tile shapes of page
 *     "Software pipelines and asynchronous copies", section "Selecting the
 *     number of stages" (a ring depth, and a tile, that the LDS and the
 *     compiled variants can hold);
 *   NONINTEGRAL_SCALAR -- the int32 epilogue of an int8 GEMM: alpha and beta
 *     must be integers so that int8 results stay exact (page "GPU-Kernel
 *     pipelinen", step 5: pipelining changes no arithmetic);
 *   HIP -- a launch the runtime rejected (page "Software pipelines and
 *     asynchronous copies", section "Common errors": issuing work is not
 *     completing it, so only the launch itself can fail here). */
enum pgemm_status {
    PGEMM_OK = 0,
    PGEMM_ERR_INVALID_ARG = -1,        /* negative size, ld too small, null pointer with work to do */
    PGEMM_ERR_UNSUPPORTED_DTYPE = -2,  /* dtype not one of pgemm_dtype */
    PGEMM_ERR_BAD_STAGES = -3,         /* stages outside 0..4 */
    PGEMM_ERR_INFEASIBLE_PLAN = -4,    /* no compiled variant satisfies the forced options */
    PGEMM_ERR_NONINTEGRAL_SCALAR = -5, /* int8 with alpha or beta not an int32 integer */
    PGEMM_ERR_HIP = -6,                /* the HIP runtime rejected the launch (its error string is
                                          printed to stderr) */
    PGEMM_ERR_TOO_LARGE = -7           /* a dimension or byte offset exceeds the 32-bit tile addressing */
};

/* Producer of a K tile (page "Double Buffering...", section "Two Stages, One
 * Barrier"; page "GPU-Kernel pipelinen", step 2):
 *   DIRECT   -- buffer_load ... lds: global memory straight into the LDS stage
 *               with no register involvement (the cp.async analogue).  When
 *               A's rows are not whole 16-byte chunks, the chunk of each row
 *               that straddles the end of K is loaded element by element
 *               (zero past K) and written to the stage, in the K tile that
 *               holds the end of K.
 *   REGISTER -- global memory into VGPRs at the top of the iteration, written
 *               to the LDS stage after the iteration's MFMA work.
 *   GENERIC  -- as REGISTER, for any element-aligned layout: 16-byte loads;
 *               in the last K tile the elements past K are zeroed in
 *               registers and the chunk at the very end of a matrix is loaded
 *               element by element.  Elements read past N reach only output
 *               columns that are never stored.
 *   STAGED_A -- one producer per operand, as the first page's kernel 11 does
 *   STAGED_B    (one operand copied asynchronously, the other staged through
 *               registers): STAGED_A moves A as GENERIC and B by LDS-DMA,
 *               STAGED_B moves A by LDS-DMA and B as GENERIC.  The operand
 *               that meets the chunk rule keeps the direct copy while the
 *               other one goes through registers.  Two LDS stages.
 *
 * The chunk rule, per operand (K == 0 meets both): A: K * elem is a multiple
 * of 16 bytes; B: N * elem is a multiple of 16 bytes (each row is whole
 * 16-byte chunks).  Pointers and leading dimensions need only element
 * alignment.  DIRECT needs B's rule, REGISTER both, STAGED_A B's, STAGED_B
 * A's, GENERIC neither.  The planner (stages = 0, producer AUTO) picks DIRECT
 * when B's rule holds and otherwise the fastest admissible variant by its
 * measured efficiencies. */
enum pgemm_producer {
    PGEMM_PRODUCER_AUTO = 0,
    PGEMM_PRODUCER_DIRECT = 1,
    PGEMM_PRODUCER_REGISTER = 2,
    PGEMM_PRODUCER_GENERIC = 3,
    PGEMM_PRODUCER_STAGED_A = 4,
    PGEMM_PRODUCER_STAGED_B = 5
};

/* Which operands meet the chunk rule above (pgemm_plan's `aligned`). */
enum pgemm_aligned {
    PGEMM_ALIGNED_NONE = 0,
    PGEMM_ALIGNED_BOTH = 1,
    PGEMM_ALIGNED_A = 2,  /* A only */
    PGEMM_ALIGNED_B = 3   /* B only */
};

/* Optional overrides for pgemm_gemm_ex / pgemm_plan.  Zero-initialise and set
 * only what you want to force. */
typedef struct pgemm_opts {
    int producer;  /* pgemm_producer; AUTO lets the planner choose */
    int tile_m;    /* 0 = planner's choice; else force BM (with tile_n, tile_k) */
    int tile_n;
    int tile_k;
    int skew;      /* stress test, 0..64 (0 = off): in every K tile one wave of
                      each workgroup (rotating) sleeps skew x 8128 cycles after
                      the ready barrier.  Results are unchanged; only timing is. */
    int workgroups; /* 0 = planner's choice; else launch this many persistent
                       workgroups (rounded up to a multiple of 8, at most one per
                       output tile), each looping over its share of the tiles
                       with one K-tile ring running across tile boundaries. */
    int waves;     /* 0 = planner's choice; else force the workgroup's wave count
                      (with tile_m/n/k this selects one compiled variant) */
    int reserved[1]; /* must be 0 */
} pgemm_opts;

/* What the planner chose (pgemm_plan output). */
typedef struct pgemm_plan_info {
    int tile_m, tile_n, tile_k;  /* BM, BN, BK */
    int stages;                  /* requested ring depth after auto selection */
    int stages_eff;              /* min(stages, max(nK, 1)): buffers actually filled */
    int num_k_tiles;             /* nK = ceil(K / BK) */
    int producer;                /* pgemm_producer actually used */
    int threads;                 /* workgroup size */
    int waves_m, waves_n;        /* wave grid inside the workgroup */
    int lds_bytes;               /* stages * (BM*BK + BK*BN) * element size */
    int wg_per_cu;               /* resident workgroups per CU (LDS and VGPR limit) */
    int grid;                    /* number of workgroups launched */
    int variant;                 /* index into the library's compiled-variant table */
    double est_uncovered_cycles; /* latency left exposed per K tile by the stage-count model */
} pgemm_plan_info;

/* C = alpha*A*B + beta*C with the planner's choices (stages = 0: auto, 1..4:
 * ring depth).  The operation is the one defined at the top of this file
 * (page "Double Buffering: Software Pipelining the K-Loop", section "The
 * Kernel").  Asynchronous on `stream`: the call returns once the kernel is
 * enqueued, and C is complete only when the stream has reached that point
 * (page "Software pipelines and asynchronous copies", section "Common
 * errors": an issued operation is not a completed one; synchronise on the
 * stream or record an event before reading C).  A, B and C are device
 * memory owned by the caller; the library keeps no pointer after the call
 * returns.  Returns PGEMM_OK or a pgemm_status error; on error nothing has
 * been enqueued unless the status is PGEMM_ERR_HIP. */
int pgemm_gemm(int64_t M, int64_t N, int64_t K, double alpha,
               const void* A, int64_t lda, const void* B, int64_t ldb,
               double beta, void* C, int64_t ldc,
               int dtype, int stages, void* stream);

/* As pgemm_gemm, with producer, tile, wave-layout and persistent-launch
 * overrides (opts may be NULL; see pgemm_opts).  The producer choice is the
 * one of page "Double Buffering: Software Pipelining the K-Loop", section
 * "Two Stages, One Barrier" (an operand copied straight into shared memory
 * asynchronously, or staged through registers) and page "GPU-Kernel
 * pipelinen", step 2 (the LDG-register and asynchronous-copy variants).
 * Asynchronous exactly as pgemm_gemm.  An override no compiled variant
 * satisfies returns PGEMM_ERR_INFEASIBLE_PLAN before anything is enqueued. */
int pgemm_gemm_ex(int64_t M, int64_t N, int64_t K, double alpha,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  double beta, void* C, int64_t ldc,
                  int dtype, int stages, const pgemm_opts* opts, void* stream);

/* Host-only: the plan pgemm_gemm_ex would use for these sizes (page
 * "Software pipelines and asynchronous copies", sections "Selecting the
 * number of stages" and "Worked example: Choosing between two and four
 * stages": the ring depth balances the latency one K tile's arithmetic
 * covers against shared-memory use and resident workgroups, and is clipped
 * to the number of K tiles).  `aligned` (a pgemm_aligned value) says which
 * operands meet the chunk rule of pgemm_producer; any other value returns
 * PGEMM_ERR_INVALID_ARG.  Writes *out and touches no GPU state.
 * Returns PGEMM_OK or the error pgemm_gemm_ex would return for the same
 * sizes and options. */
int pgemm_plan(int64_t M, int64_t N, int64_t K, int dtype, int stages,
               int aligned, const pgemm_opts* opts, pgemm_plan_info* out);

/* Static description of a pgemm_status value (the sources of each code are
 * listed at enum pgemm_status); "unknown status" for any other value.  The
 * string is owned by the library and never freed. */
const char* pgemm_strerror(int status);

/* Number of compiled kernel variants and their static description
 * (host-only; for sweeps and tests): the instantiation table the re-run tile
 * and depth search of page "Double Buffering: Software Pipelining the
 * K-Loop", section "What Could Be Improved", walks.  pgemm_variant_info
 * returns PGEMM_ERR_INVALID_ARG for an index outside 0..num-1. */
int pgemm_num_variants(void);
int pgemm_variant_info(int index, pgemm_plan_info* out, int* dtype);

/* Planner models (host-only, exposed for tests and reports).
 *
 * pgemm_model_uncovered_cycles: load latency left exposed per K tile with a
 * ring of `stages` buffers when one tile's arithmetic takes compute_per_tile
 * cycles: max(0, latency - (stages-1)*compute_per_tile), and the whole latency
 * for a single buffer.  Page "Software pipelines and asynchronous copies",
 * section "Worked example: Choosing between two and four stages" (two stages:
 * max(0, 500 - 220) = 280 cycles).
 *
 * pgemm_model_lds_bytes: bytes of a ring of `stages` A (BM x BK) and B
 * (BK x BN) tiles, with `a_pad_elems_per_k` extra elements per A row of K
 * (page "Double Buffering: Software Pipelining the K-Loop", section "The
 * Kernel": As[2][BK*A_STRIDE] and Bs[2][BK*BN]).
 *
 * pgemm_model_global_loads_per_output: global loads per output element of a
 * BM x BN tile over K, K/BN + K/BM (same page, section "What The Overlap
 * Cost": 96 at 128 x 64 and K = 4096, unchanged by pipelining).
 *
 * pgemm_model_compute_load_ratio: flops of one K tile over the bytes loaded
 * for it, 2*BM*BN*BK / ((BM*BK + BK*BN) * elem_bytes) (page "GPU-Kernel
 * pipelinen", step 2).  A reported diagnostic only: the page's thresholds for
 * choosing a producer by it were measured on another GPU, and the planner
 * chooses by measured sweeps instead.  Returns 0 for non-positive sizes. */
double pgemm_model_uncovered_cycles(double latency, double compute_per_tile, int stages);
int64_t pgemm_model_lds_bytes(int bm, int bn, int bk, int stages, int elem_bytes, int a_pad_elems_per_k);
double pgemm_model_global_loads_per_output(int bm, int bn, int64_t K);
double pgemm_model_compute_load_ratio(int bm, int bn, int bk, int elem_bytes);

/* Consume-before-reuse hazard demonstrator (page "Software pipelines and
 * asynchronous copies", sections "Producer-consumer synchronization" and
 * "Practice").  Not a GEMM: a two-stage tiled copy-and-reduce that computes
 *
 *     row_sums[r] = sum_c X[r*ldx + c]    for 0 <= r < rows, 0 <= c < cols
 *
 * in int32 (two's-complement wrap; exact and order-independent, so any
 * difference from the plain sum is a protocol failure, not rounding).
 * Each workgroup owns 16 rows and walks the columns in tiles of 16 x 256
 * through two LDS stages: the loads of tile t+2 are in flight in registers
 * while the four waves reduce tile t (four rows each) from stage t%2; then
 * stage t%2 is rewritten with tile t+2.
 *
 *   reuse_wait = 1: the correct protocol, two workgroup barriers per tile:
 *       the reuse barrier (every wave has finished reading stage t%2) before
 *       the rewrite, the readiness barrier (the rewrite is visible) after it.
 *   reuse_wait = 0: the same kernel with only the reuse barrier removed.  A
 *       wave that finishes early may overwrite stage t%2 with tile t+2 while
 *       another wave still reads tile t from it: the sums of that wave's rows
 *       come out wrong, intermittently without a delay.  Every remaining
 *       barrier is still executed by all waves and every address is the same
 *       as in the correct protocol, so the variant cannot hang or fault.
 *
 *   delay_wave (-1 = none, else 0..3) sleeps about delay_cycles shader
 *   clocks (0..10 000 000, in steps of 64) before reading each tile: the
 *   artificial consumer delay.
 *
 *   trace (optional, NULL = off): for workgroup trace_wg, lane 0 of each wave
 *   w records six shader-clock stamps per tile t at trace[(w*nT + t)*6 + e]:
 *   e = 0 top of the iteration (loads of tile t+2 issued), 1 start of the
 *   reads of stage t%2, 2 reads complete, 3 past the reuse barrier (same as 2
 *   without it), 4 stage t%2 rewritten, 5 past the readiness barrier;
 *   nT = cols / 256, trace_len >= 24 * nT.
 *
 * Layout: X row-major int32 with leading dimension ldx (elements), device
 * pointer, 16-byte aligned; rows a multiple of 16, cols a positive multiple
 * of 256, ldx >= cols and a multiple of 4.  row_sums: device int32[rows].
 * All buffers belong to the caller; nothing is allocated.  Argument errors
 * (PGEMM_ERR_INVALID_ARG) are detected before anything is enqueued; a
 * rejected launch returns PGEMM_ERR_HIP.  Asynchronous on `stream`. */
int pgemm_hazard_copy_reduce(const int32_t* X, int64_t rows, int64_t cols, int64_t ldx,
                             int32_t* row_sums, int reuse_wait, int delay_wave, int delay_cycles,
                             int64_t* trace, int64_t trace_len, int trace_wg, void* stream);

/* Diagnostics that bound the GEMM from above (page "Software pipelines and
 * asynchronous copies", section "Worked example: Choosing between two and
 * four stages", last point: a timing difference alone does not show the
 * cause).  Neither is part of the GEMM path.
 *
 * pgemm_diag_mfma_ceiling: the matrix cores alone.  `grid` workgroups
 * (one per CU) of waves_per_simd (1 or 2) waves per SIMD each run `iters`
 * rounds of independent MFMA blocks of the dtype: block = 16 gives sixteen
 * 16x16 blocks per round, the GEMM's own (bf16/fp16 16x16x32, int8 16x16x64,
 * fp32 four 16x16x4); block = 32 gives eight 32x32 blocks of the same flops
 * (bf16/fp16 32x32x16, int8 32x32x32; not for fp32).  Operands come from a
 * hash of `seed` and the lane (random values in [-1, 1), or any int8), or
 * are zeros when zero_operands = 1.  No memory traffic besides one float per
 * wave written to out[grid * 4 * waves_per_simd] (device memory owned by
 * the caller, 4-byte aligned), which keeps the accumulators live.  *flops
 * (optional) receives the flops of the launch.  `clock` (optional, device
 * memory, 8-byte aligned, grid * 4 entries) receives per workgroup the
 * shader clock and the constant 100 MHz clock (s_memtime, s_memrealtime) of
 * wave 0 at its start, then both at its end: the shader clock's rate under
 * this load.  Asynchronous on `stream`.  Errors: UNSUPPORTED_DTYPE;
 * INVALID_ARG for waves_per_simd not 1 or 2, block not 16 or 32 (or 32 for
 * fp32), iters outside 0..2^24, grid outside 1..65536 or a bad `out` or
 * `clock`; HIP for a rejected launch.
 *
 * pgemm_diag_lds_stream: the producer alone.  For the compiled stream of tile
 * class (tile_m, tile_n, tile_k) at ring depth `stages` it issues exactly the
 * LDS-DMA pieces the GEMM's DIRECT producer would for C = A*B with these
 * operands (same workgroup raster, 1-KiB blocks, one ready barrier per K
 * tile, stages - 1 K tiles in flight) and does no arithmetic.  A and B follow
 * the GEMM's layout rules, with both operands 16-byte aligned and lda, ldb,
 * K and N whole 16-byte chunks (the aligned case); they are only read.  *lds_bytes (optional) receives the
 * LDS bytes the launch fills.  Asynchronous on `stream`.  Errors:
 * UNSUPPORTED_DTYPE; INVALID_ARG (sizes, leading dimensions, alignment);
 * TOO_LARGE (32-bit tile addressing); INFEASIBLE_PLAN when no stream of that
 * class and depth is compiled (bf16 256x256x64 S2 and 256x256x32 S2..4,
 * fp16 256x256x64 S2, int8 256x256x128 S2, fp32 128x64x16 S2 and
 * 256x256x32 S2); HIP for a rejected launch. */
/* pgemm_diag_wait_profile: C = A*B (alpha = 1, beta = 0, same layout rules
 * and results as pgemm_gemm) with a wait-profile build of the DIRECT variant
 * of tile class (tile_m, tile_n, tile_k) at ring depth `stages`: the same
 * kernel with shader-clock stamps around the two waits of every ready edge.
 * For each wave w of each workgroup b that has a tile, out[(b*W + w)*8 + i]
 * (W = waves per workgroup) receives: in shader clocks, i = 0 the time in
 * the vmcnt wait (the K tile's loads landing), 1 the time from there through
 * the workgroup barrier (every other wave arriving; for one stage also the
 * reuse barrier), 2 the number of ready edges, 3 the whole K loop; and on the
 * GPU's constant 100 MHz clock (s_memrealtime), the wave's timeline: 4 its
 * start, 7 the first ready edge passed (end of the prologue), 5 the end of
 * the K loop, 6 its C stores complete.  `out` is device memory owned by the
 * caller, 8-byte aligned, out_len >= grid * W * 8 entries with
 * grid = ceil(tiles / 8) * 8.  Both operands must be 16-byte aligned with
 * lda, ldb, K and N whole 16-byte chunks (the aligned case).  Asynchronous on `stream`.  Errors:
 * UNSUPPORTED_DTYPE; INVALID_ARG; TOO_LARGE; INFEASIBLE_PLAN when no profile
 * build of that class and depth is compiled (bf16 256x256x64 S1/S2,
 * 256x256x32 S1..S4, 128x128x64 S2/S3; fp16 256x256x64 S1/S2; int8
 * 256x256x128 S1/S2; fp32 128x64x16 S1/S2, 256x256x32 S1/S2); HIP for a rejected launch. */
int pgemm_diag_wait_profile(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            const void* B, int64_t ldb, void* C, int64_t ldc, int dtype,
                            int tile_m, int tile_n, int tile_k, int stages, int64_t* out,
                            int64_t out_len, void* stream);
int pgemm_diag_mfma_ceiling(int dtype, int zero_operands, int waves_per_simd, int block, int iters,
                            int grid, uint32_t seed, float* out, int64_t* flops, int64_t* clock,
                            void* stream);
int pgemm_diag_lds_stream(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                          const void* B, int64_t ldb, int dtype, int tile_m, int tile_n,
                          int tile_k, int stages, int64_t* lds_bytes, void* stream);

/* pgemm_diag_parts: the parts ladder (page "Software pipelines and
 * asynchronous copies", section "Worked example: Choosing between two and
 * four stages", last point, as above).  The GEMM kernel of the DIRECT
 * variant of tile class (tile_m, tile_n, tile_k) at ring depth `stages`,
 * built with only the steady-state parts in `parts` (a set of pgemm_part
 * bits; PGEMM_PART_ALL is the GEMM itself):
 *   PGEMM_PART_DMA      the LDS-DMA pieces of the K tiles after the prologue;
 *                       without them the two stages keep the prologue's K
 *                       tiles, so the matrix cores still multiply operand
 *                       data;
 *   PGEMM_PART_BARRIER  the workgroup barrier of each ready edge (its waits
 *                       stay); the prologue keeps its barrier;
 *   PGEMM_PART_AREADS   the A fragment reads from LDS;
 *   PGEMM_PART_BREADS   the B fragment (transposing) reads from LDS; a
 *                       left-out read leaves the previous fragment in place
 *                       (both fragment register sets start from operand
 *                       data: K steps 0 and 1 of the first K tile).
 * The MFMAs and the C store always run.  C receives A*B only for
 * PGEMM_PART_ALL; otherwise C receives values of no meaning.  Wave 0 of each
 * workgroup b with a tile writes clock[b*4 + i]: i = 0 the shader clock
 * (s_memtime) and 1 the 100 MHz clock (s_memrealtime) at its start, 2 and 3
 * the same after its last store; dividing the shader-clock span by the
 * 100 MHz span gives the clock the launch ran at.  Layout and alignment
 * rules as for pgemm_diag_wait_profile; `clock` is device memory owned by
 * the caller, 8-byte aligned, clock_len >= grid * 4 with
 * grid = ceil(tiles / 8) * 8.  Asynchronous on `stream`.  Errors:
 * UNSUPPORTED_DTYPE; INVALID_ARG (including `parts` outside 0..15);
 * TOO_LARGE; INFEASIBLE_PLAN unless the class is bf16 or fp16 256x256x64
 * S2, int8 256x256x128 S2 or fp32 128x64x16 S2 and `parts` is one of 0,
 * AREADS, BREADS, AREADS|BREADS, AREADS|BREADS|BARRIER, ALL; HIP for a
 * rejected launch. */
enum pgemm_part {
    PGEMM_PART_DMA = 1,
    PGEMM_PART_BARRIER = 2,
    PGEMM_PART_AREADS = 4,
    PGEMM_PART_BREADS = 8,
    PGEMM_PART_ALL = 15
};
int pgemm_diag_parts(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, int dtype, int tile_m, int tile_n,
                     int tile_k, int stages, int parts, int64_t* clock, int64_t clock_len,
                     void* stream);

/* ABI version: major*10000 + minor*100 + patch (a library convention, not
 * from the pages). */
int pgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
