/*
 * sgemm_f32.h -- C ABI of the MI355X (gfx950) FP32 matrix multiply C = A x B.
 *
 * Operation (every entry point that computes):
 *     C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[k*ldb + j]      for 0 <= i < M, 0 <= j < N
 * The product is the one every page builds on: each output is the dot product of a row of
 * A with a column of B ("SGEMM: Shared Memory Tiling Visualizer", "Why Tiling Works (The
 * Math)"; "Shared Memory Tiling", "The naive kernel"). A is M x K, B is K x N, C is M x N,
 * all row-major FP32; the pages use packed rows (lda = K, ldb = N, ldc = N) and this ABI
 * adds leading dimensions (in elements) so the operands may be sub-matrices. C is
 * overwritten, never accumulated into (alpha = 1, beta = 0), as in every kernel the pages
 * print. Arithmetic is FP32 with FP32 accumulation; the order of the K-sum is not fixed.
 *
 * Ownership: A, B and C are device pointers owned by the caller. The library keeps no
 * mutable state between calls apart from a per-device cache of the compute-unit count,
 * and is safe to call from several host threads.
 *
 * Errors: every argument is validated before any HIP runtime call, so the validation
 * paths work (and are tested) on a host without a GPU. A negative return value is an
 * sgemm_status; the library never aborts. Launches are asynchronous on `stream` (a
 * hipStream_t; NULL is the default stream); a launch failure is reported as
 * SGEMM_ELAUNCH, and faults during execution surface at the caller's next synchronisation.
 *
 * Validation rules (checked in this order):
 *   M, N, K >= 0                                   else SGEMM_EINVAL_DIM
 *   lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N)   else SGEMM_EINVAL_LD
 *   a pointer whose region is non-empty is non-NULL and 4-byte aligned   else SGEMM_EINVAL_PTR
 *   C's region does not overlap A's or B's region  else SGEMM_EALIAS
 * Regions: A spans (M-1)*lda + K elements from A (empty if M or K is 0); B spans
 * (K-1)*ldb + N (empty if K or N is 0); C spans (M-1)*ldc + N (empty if M or N is 0).
 * Quick returns: M == 0 or N == 0 launches nothing; K == 0 sets C's M x N region to 0
 * (the empty sum) with one small kernel.
 */
#ifndef SGEMM_F32_H
#define SGEMM_F32_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SGEMM_OK = 0,
    SGEMM_EINVAL_DIM = -1,   /* a dimension is negative                                  */
    SGEMM_EINVAL_LD = -2,    /* a leading dimension is smaller than its row length       */
    SGEMM_EINVAL_PTR = -3,   /* a needed pointer is NULL or not 4-byte aligned           */
    SGEMM_EALIAS = -4,       /* C overlaps A or B                                        */
    SGEMM_ELAUNCH = -5,      /* the HIP runtime refused a launch or device query         */
    SGEMM_EINVAL_ARG = -6,   /* an option argument (tile, pad, variant, buffer) is invalid */
    SGEMM_ETOO_LARGE = -7,   /* the shape exceeds what the chosen kernel can address     */
    SGEMM_ESCRATCH = -8      /* sgemm_f32_streamk_noalloc: the plan's partial tiles exceed
                                the library's static scratch                             */
} sgemm_status;

/*
 * The hot path: the LDS-tiled, register-tiled matrix-core kernel ("SGEMM: 2D Register
 * Tiling Visualizer", "Why 2D Register Tiling Dominates", carried onto the FP32 MFMA
 * instructions), with tiles zero-filled past the edges of ragged shapes. The tile shape
 * is chosen per (M, N, K) and compute-unit count; when N leaves one to four columns past
 * the last whole tile column (or M as many rows past the last tile row), the tiles may also
 * compute them, on the vector ALUs beside their MFMAs, instead of a nearly empty column (or
 * row) of tiles. Any 4-byte aligned
 * pointers and any leading dimensions work. Leading dimensions so large that 256 rows of A or C (or 32
 * rows of B) exceed 2^31 bytes return SGEMM_ETOO_LARGE.
 */
int sgemm_f32(int M, int N, int K,
              const float *A, int lda,
              const float *B, int ldb,
              float *C, int ldc,
              void *stream);

/*
 * Split-K for shapes whose M x N gives too few tiles to fill the GPU (small M * N, large
 * K). The pages fill the GPU by the choice of tile size alone ("Shared Memory Tiling",
 * "Choosing a tile size"; "Visual walkthrough - Memory hierarchy", Step 7); when even the
 * smallest tile leaves compute units idle, this entry point also cuts each tile's K-sum.
 * K is cut into `splits` ranges of whole K-panels; the hot kernel computes each
 * (tile, range) item into its own M x N slice of `workspace` (packed rows of N floats),
 * and a second kernel sums the slices in ascending range order into C, so repeated calls
 * give identical bits. splits = 0 lets the library choose: the count whose estimated time
 * (the busiest compute unit's items, plus the reduce's pass over the slices) is lowest,
 * with ranges of at least four 64-deep panels; it may be 1, which runs sgemm_f32's plan.
 * splits = 1 is sgemm_f32. At most 32.
 * workspace is a caller-owned device buffer of at least splits * M * N * 4 bytes
 * (sgemm_f32_splitk_workspace_size) that must not overlap A, B or C (SGEMM_EINVAL_PTR if
 * NULL or misaligned, SGEMM_EINVAL_ARG if too small, SGEMM_EALIAS on overlap; checked
 * before any HIP call when splits >= 2); its contents on return are unspecified. Both
 * kernels run on `stream`.
 */
int sgemm_f32_splitk(int M, int N, int K,
                     const float *A, int lda,
                     const float *B, int ldb,
                     float *C, int ldc,
                     int splits, float *workspace, size_t workspace_bytes,
                     void *stream);

/* Bytes of workspace sgemm_f32_splitk needs for this shape and split count (0 when it
 * needs none: splits of 1, empty shapes, or arguments out of range). splits = 0 asks for
 * the automatic choice and queries the current device. */
size_t sgemm_f32_splitk_workspace_size(int M, int N, int K, int splits);

/*
 * Stream-K for tile grids that do not divide evenly over the GPU (a tile count just past a
 * multiple of the resident workgroups, such as 272 tiles on 256 compute units): the pages
 * size tiles against the parallelism they leave ("Shared Memory Tiling", "Choosing a tile
 * size"; "Visual walkthrough - Memory hierarchy", Step 7), and this entry point goes one
 * step finer. The unit of work is one K-panel of one tile; the last tiles' units are
 * shared out evenly over the resident workgroups (CUs x workgroups per CU), each taking a
 * contiguous range. A range that covers a whole tile writes it to C; a tile shared by
 * several ranges gets their partial sums, which go through `workspace` and are added by a
 * second kernel in ascending K order, so repeated calls give identical bits. Results
 * differ from sgemm_f32's only by the order of the K-sum (exact on small integers).
 * variant < 0: the library prices every tile variant run plainly and as stream-K and
 * takes the cheapest; when that is a plain grid this is sgemm_f32 and the workspace is
 * not touched. variant >= 0 forces stream-K with that tile variant (an index below
 * sgemm_f32_variant_count() whose name ends in "_dl", else SGEMM_EINVAL_ARG); a grid that
 * divides evenly still runs plainly.
 * workspace: caller-owned device memory of sgemm_f32_streamk_workspace_size bytes (2 x
 * the workgroup count x one tile of floats), 16-byte aligned, not overlapping A, B or C
 * (SGEMM_EINVAL_PTR, SGEMM_EALIAS; checked before any HIP call whenever workspace_bytes
 * > 0); too small for the plan is SGEMM_EINVAL_ARG. It needs no initialisation, and
 * its contents on return are unspecified. Calls that share a workspace must not overlap
 * in time (same stream, or synchronised). Both kernels run on `stream`.
 */
int sgemm_f32_streamk(int M, int N, int K,
                      const float *A, int lda,
                      const float *B, int ldb,
                      float *C, int ldc,
                      int variant, float *workspace, size_t workspace_bytes,
                      void *stream);

/* Bytes of workspace sgemm_f32_streamk needs for these arguments on the current device:
 * the same shape, leading dimensions and variant the call will get (the plan depends on
 * them). 0 when the plan shares no tile, for empty shapes, for dimensions or leading
 * dimensions that sgemm_f32_streamk would reject, or on a bad variant. */
size_t sgemm_f32_streamk_workspace_size(int M, int N, int K, int lda, int ldb, int ldc,
                                        int variant);

/*
 * sgemm_f32_streamk for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, and harnesses that forbid allocation. It takes no
 * workspace. The partial tiles go to a static scratch array that the library holds on
 * each GPU it runs on until the process ends. Its size is
 * sgemm_f32_streamk_noalloc_scratch_bytes(), 64 MiB. The function calls no allocator: no
 * hipMalloc, no hipFree, no allocating library routine.
 *
 * Arguments, plan, kernels and results are those of sgemm_f32_streamk with the same
 * variant, so the two give identical bits. A plan whose partial tiles need more scratch
 * than that returns SGEMM_ESCRATCH before any launch. That needs 2 x the workgroup count
 * x one tile of floats above 64 MiB: 256 x 256 tiles, or 128 x 256 tiles at two per CU.
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's partial
 * tiles. Nothing in it needs to start at zero: each slot is written before it is read.
 * Calls that overlap in time on one GPU race on it: different streams, or host threads
 * that are not synchronised. Such calls give wrong results. Calls on one stream are
 * ordered and safe.
 */
int sgemm_f32_streamk_noalloc(int M, int N, int K,
                              const float *A, int lda,
                              const float *B, int ldb,
                              float *C, int ldc,
                              int variant,
                              void *stream);

/* Bytes of the static scratch behind sgemm_f32_streamk_noalloc (per GPU). */
size_t sgemm_f32_streamk_noalloc_scratch_bytes(void);

/*
 * Writes a one-line JSON description of sgemm_f32_streamk's plan for packed operands of
 * this shape into buf: variant and tile, whether it shares tiles, the workgroup count G,
 * the plain and shared tile counts, K-panels per tile, the shared units, how many tiles
 * are shared and by at most how many workgroups, segments per workgroup, workspace bytes,
 * "partition_ok": the result of walking every range with the kernels' own partition
 * functions (every unit in exactly one range, every partial slot the fixup reads written
 * once for that tile), for a plain plan the columns its last tile column computes as a
 * strip ("strip_cols"; the tile count then leaves them out), and the two prices the choice
 * compares, in microseconds at the cost model's unit rate: the cheapest plain plan
 * ("plain_cost_us") and this variant as stream-K ("streamk_cost_us", 0 when it shares no
 * tile). num_cus > 0 plans for that many compute units (no GPU needed); num_cus <= 0
 * queries the current device. M, N and K must be positive (else
 * SGEMM_EINVAL_DIM). Returns the variant index, or a negative sgemm_status.
 */
int sgemm_f32_streamk_describe(int M, int N, int K, int variant, int num_cus,
                               char *buf, int buflen);

/*
 * The reference kernel: one thread per element of C, a length-K dot product read
 * straight from global memory ("Shared Memory Tiling", "The naive kernel"), with bounds
 * checks so any shape works. Slow on purpose; the pages' 2*M*N*K read count applies.
 */
int sgemm_f32_naive(int M, int N, int K,
                    const float *A, int lda,
                    const float *B, int ldb,
                    float *C, int ldc,
                    void *stream);

/*
 * The scalar shared-memory tiled kernel ("SGEMM: Shared Memory Tiling Visualizer", code
 * panel; "Shared Memory Tiling", "The tiled kernel"): TILE x TILE threads per block, one
 * output each, tiles of A and B staged in LDS and zero-filled at the edges, ceil(K/TILE)
 * steps. tile is 16 or 32; pad is 0 (unpadded rows) or 1 (rows of TILE + 1 words, the
 * padded layout of "Shared Memory Tiling", "Conflict-free layout"). Anything else is
 * SGEMM_EINVAL_ARG. Kept as a measurable rung between the naive and the hot kernel.
 */
int sgemm_f32_tiled(int M, int N, int K,
                    const float *A, int lda,
                    const float *B, int ldb,
                    float *C, int ldc,
                    int tile, int pad,
                    void *stream);

/*
 * Scalar register tiling ("SGEMM: 2D Register Tiling Visualizer", code panel and "Why 2D
 * Register Tiling Dominates"): each thread keeps a tm x tn block of C in registers and,
 * per k, loads tm values of A and tn values of B from LDS for tm*tn FMAs. (tm, tn) is
 * (4, 1) (the page's 1-D strip), (4, 4) or (8, 8); anything else is SGEMM_EINVAL_ARG.
 * A measurable rung of the pages' ladder, on the vector ALUs rather than the matrix cores.
 * Shapes with more than 65535 row tiles (64 rows, 128 for 8 x 8) return SGEMM_ETOO_LARGE.
 */
int sgemm_f32_regtiled(int M, int N, int K,
                       const float *A, int lda,
                       const float *B, int ldb,
                       float *C, int ldc,
                       int tm, int tn,
                       void *stream);

/*
 * LDS bank-geometry microbenchmark: out[j*ldo + i] = in[i*ldi + j] for i < rows, j < cols,
 * through a tile x tile LDS tile written by rows and read by columns, with rows padded by
 * `pad` words ("Visual walkthrough - Memory hierarchy", Step 6; "Shared Memory Tiling",
 * "Conflict-free layout"). tile is 32 or 64, pad 0 or 1. in and out are device pointers
 * (rows x cols and cols x rows, row-major); validation mirrors the GEMM entry points
 * (ldi >= max(1, cols), ldo >= max(1, rows), out must not overlap in). More than 65535
 * row tiles returns SGEMM_ETOO_LARGE.
 */
int sgemm_f32_lds_transpose(int rows, int cols,
                            const float *in, int ldi,
                            float *out, int ldo,
                            int tile, int pad,
                            void *stream);

/*
 * The hot kernel with a fixed tile variant instead of the automatic choice (for tests
 * and tuning). variant < 0 is the automatic choice (same as sgemm_f32); otherwise an
 * index below sgemm_f32_variant_count(), else SGEMM_EINVAL_ARG. Every variant computes
 * the same product for every shape; they differ in tile shape, waves and how panels reach
 * LDS (names ending in "_dl" load straight from global memory into LDS, the others stage
 * through registers; "_rp" is the one-wave-per-SIMD kernel that holds a whole K-panel's
 * operands in registers; "_ps" is the persistent kernel, one workgroup per CU walking
 * 128 x 256 tiles and writing each tile among the next one's MFMAs), and some are never
 * chosen automatically (kept for comparison). "_ps" computes only whole tiles of a product
 * with more than 32 values of K: the rest of C (the strips past the last whole tile row and
 * column), or the whole product when it has no whole tile or K <= 32, is computed by the
 * automatic choice, on the same stream. A variant whose 31-bit buffer offsets cannot span
 * one workgroup's rows of A or C or one K-panel of B returns SGEMM_ETOO_LARGE.
 */
int sgemm_f32_variant(int variant, int M, int N, int K,
                      const float *A, int lda,
                      const float *B, int ldb,
                      float *C, int ldc,
                      void *stream);

/* Number of hot-kernel tile variants, and the name of one (NULL when out of range). */
int sgemm_f32_variant_count(void);
const char *sgemm_f32_variant_name(int variant);

/*
 * Writes a one-line JSON description of tile variant `variant` into buf (at most buflen
 * bytes including the NUL): name, tile (BM, BN, BK), waves along M and N, K-groups,
 * threads, the MFMA instruction shape ("32x32x2" or "16x16x4"), resident workgroups per
 * CU, direct loads, whether the automatic plan may pick it, whether it has a stream-K
 * form, the plan's cost-model parameters (rate, overhead, solo, and the launch's latency in
 * microseconds, "latency_us") for it, the kernel family
 * ("mfma": the LDS-double-buffered template; "regpanel": the one-wave-per-SIMD kernel;
 * "persist": the persistent kernel), whether split-K may use it, whether it runs one
 * workgroup per CU over the tiles ("persistent"), whether it only takes whole tiles
 * ("whole_tiles"), whether its tiles can also compute columns of N past the last whole
 * tile column, on the vector ALUs ("strip"), and how many at most ("strip_cols_max": 1, 2
 * or 4; more than one only spread over the tiles of each row), the LDS stages per K-group of the
 * template kernel ("lds_stages": 2, or 3 where each panel's loads are issued two panels
 * ahead; "Shared Memory Tiling", "What tiling does not fix"). Host-only, no GPU needed. Returns SGEMM_OK, or
 * SGEMM_EINVAL_ARG for a bad index or a buffer too small.
 */
int sgemm_f32_variant_info(int variant, char *buf, int buflen);

/* A static, NUL-terminated description of a status code. */
const char *sgemm_f32_status_string(int status);

/*
 * Writes a one-line JSON description of the plan sgemm_f32 would run for these
 * arguments into buf (at most buflen bytes including the NUL): variant, tile shape,
 * waves, grid, workgroups resident per CU, whether panels load straight into LDS, the
 * operand bytes the tiles request, and the column strip: "strip_cols" (the columns past
 * the last whole tile column that the tiles also compute, 0 to 4), "row_strip" and
 * "row_strip_cols" (the rows past the last whole tile row that the tiles of each tile
 * column compute instead, 0 to 4, and the columns each tile takes of them), "strip_rows" (the
 * strip rows each tile of a row computes when they are spread over the row's tiles; 0
 * when the last tile column computes them all), "strip_tiles" (how many tiles compute
 * some) and "edge_launches" (0-2: the right and bottom edges a whole-tile variant leaves to
 * kernels of their own). The plan is the pages' tile-size trade-off: reuse
 * per staged element against the parallelism left ("Shared Memory Tiling", "Choosing a
 * tile size"). Dimensions and leading dimensions are validated as in sgemm_f32
 * (SGEMM_EINVAL_DIM, SGEMM_EINVAL_LD); pointers are used for their alignment only and
 * are never dereferenced. num_cus > 0 plans for that many compute units; num_cus <= 0
 * queries the current device (SGEMM_ELAUNCH if none). Returns the variant index (>= 0),
 * or a negative sgemm_status (buffer too small: SGEMM_EINVAL_ARG).
 */
int sgemm_f32_plan_describe(int M, int N, int K,
                            const float *A, int lda,
                            const float *B, int ldb,
                            const float *C, int ldc,
                            int num_cus, char *buf, int buflen);

/*
 * The same description for a tile variant forced as sgemm_f32_variant runs it (variant
 * < 0: the plan's choice, as sgemm_f32_plan_describe), with the leading dimensions given:
 * which variant, its grid and whether its tiles compute a column strip and how. Host-only,
 * no pointers. Returns the variant index, SGEMM_EINVAL_ARG for an unknown variant or a
 * buffer too small, SGEMM_EINVAL_DIM / SGEMM_EINVAL_LD as sgemm_f32, SGEMM_ETOO_LARGE if
 * the variant's buffer offsets cannot reach the operands, SGEMM_ELAUNCH if num_cus <= 0
 * and no device answers. The tile-size trade-off it reports is that of "Shared Memory
 * Tiling", "Choosing a tile size".
 */
int sgemm_f32_variant_describe(int variant, int M, int N, int K, int lda, int ldb, int ldc,
                               int num_cus, char *buf, int buflen);

/* Version of this ABI (incremented on any incompatible change). */
int sgemm_f32_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_H */
