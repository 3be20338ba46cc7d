/*
 * gemmf32 -- FP32 GEMM C = A.B for AMD MI355X (gfx950), tiled over LDS with a
 * single-buffered and a double-buffered (two-slot, one barrier per K step) K-loop.
 *
 * Operation (all entry points that launch):
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]      0 <= i < M, 0 <= j < N
 * with row-major A (M x K, row stride lda), B (K x N, row stride ldb) and C (M x N, row
 * stride ldc), all FP32, products and sums in FP32 on the matrix cores.  C is overwritten
 * and never read (no alpha/beta); there are no transposed modes.  The K-loop walks tiles
 * of A and B through on-chip shared memory ("Double Buffering", opening paragraph and code
 * figure; "Case Study: The Double-Buffered GEMM", code figure).
 *
 * Memory and ownership: A, B and C are caller-owned DEVICE pointers (for instance the
 * data pointers of GPU tensors).  Each must be 4-byte aligned; any leading dimension is
 * accepted (rows that are not 16-byte aligned, and row strides so large that one tile of
 * A or B spans 4 GiB or more, take an element-wise copy path).  The library allocates
 * nothing, keeps no per-call state and only borrows `stream` (a hipStream_t; NULL = the
 * legacy default stream).  C must not overlap A or B.
 *
 * Asynchrony: a launching call only enqueues one kernel on `stream` and returns; the
 * caller synchronizes.  Calls are re-entrant: the only shared state is a constant table.
 *
 * Errors: every entry point returns GEMMF32_OK (0) or a negative GEMMF32_ERR_* code.
 * Arguments are validated before any HIP call, so a rejected call launches nothing and
 * touches no memory.  GEMMF32_ERR_HIP means the launch itself failed; the HIP error code
 * is then available from gemm_f32_last_hip_error() (per thread).
 *
 * Degenerate shapes: M == 0 or N == 0 is a no-op that returns 0 (pointers may be NULL);
 * K == 0 writes zeros to the M x N block of C (A and B may be NULL).
 */
#ifndef GEMMF32_H
#define GEMMF32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GEMMF32_OK = 0,
    GEMMF32_ERR_NEGATIVE_DIM = -1,  /* M, N or K < 0                                    */
    GEMMF32_ERR_BAD_LD = -2,        /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
    GEMMF32_ERR_NULL_PTR = -3,      /* NULL pointer for a non-empty operand              */
    GEMMF32_ERR_MISALIGNED = -4,    /* A, B or C not 4-byte aligned                      */
    GEMMF32_ERR_ALIAS = -5,         /* the byte range of C overlaps that of A or B       */
    GEMMF32_ERR_TOO_LARGE = -6,     /* M, N or K beyond 2^31 - 1025; a leading dimension
                                       beyond 64 times that (about 2^37); an operand or
                                       workspace whose byte extent ((rows-1)*ld + cols)*4
                                       passes 2^61 or wraps the address space; or a grid
                                       that does not fit one launch                     */
    GEMMF32_ERR_BAD_CONFIG = -7,    /* unknown variant or tile configuration id          */
    GEMMF32_ERR_HIP = -8,           /* the HIP launch failed                             */
    GEMMF32_ERR_SCRATCH_LIMIT = -9  /* gemm_f32_splitk_noalloc: the split needs more than
                                       GEMMF32_SCRATCH_FLOATS floats of scratch         */
};

/* Floats of the static device scratch array behind gemm_f32_splitk_noalloc (32 MiB). */
#define GEMMF32_SCRATCH_FLOATS (8 * 1024 * 1024)

/* Variants of the K-loop. */
enum {
    GEMMF32_VARIANT_AUTO = 0,  /* per-shape choice: dispatch table, else its cost model */
    GEMMF32_VARIANT_SB = 1,    /* one LDS slot: load -> barrier -> compute -> barrier,
                                  two barriers per K step ("Case Study: The
                                  Double-Buffered GEMM", second paragraph: the sibling) */
    GEMMF32_VARIANT_DB = 2,    /* two LDS slots: prologue loads tile 0 into slot 0; each
                                  K step has one barrier, prefetches tile l+1 into the
                                  idle slot and computes on the current one ("Double
                                  Buffering", code figure; "Case Study", code figure)   */
    GEMMF32_VARIANT_MS = 3,    /* S >= 2 LDS stages filled by asynchronous direct-to-LDS
                                  copies, tiles l+1 .. l+S-1 in flight, one barrier per
                                  K step: the multi-stage asynchronous-copy pipeline the
                                  glossary page names as the CUDA analogue ("Double
                                  Buffering", second paragraph)                         */
    GEMMF32_VARIANT_SB3 = 4,   /* measurement baseline: single-buffered with the A and B
                                  copies published by separate barriers, copy A ->
                                  barrier -> copy B -> barrier -> compute -> barrier,
                                  three barriers per K step (the pre-coalescing fence
                                  placement of "Dependence-aware group synchronization on
                                  M1 Max", section "Transformation and safety boundary");
                                  only through gemm_f32_ex, never dispatched; its tile
                                  configuration defaults to the single-buffered column  */
    GEMMF32_VARIANT_KS = 5     /* K split inside a workgroup: four one-wave groups each
                                  run the double-buffered loop over a quarter of the K
                                  tiles and add their sums through LDS in a fixed order;
                                  for few rows against a long K (the skinny regime of
                                  "Case Study", paragraph on the three regimes).  Only
                                  configurations that have it (gemm_f32_config_variants) */
};

/* C = A.B with the variant and tile configuration chosen per shape: the measured pick
 * for a shape in the dispatch table, otherwise the pick of the table's cost model, which
 * weighs each pair's fixed cost against its time per K tile and round of workgroups over
 * the 256 compute units.  The GEMMF32_VARIANT environment variable ("sb", "db", "ms" or
 * "ks") forces the variant, for measurement; GEMMF32_RASTER=<group_m>[,noxcd] changes the
 * order in which workgroups walk the output tiles, for every launching entry point, also
 * for measurement only.  The pages' lesson that the faster variant depends on the shape is
 * the reason for the table ("Double Buffering", last two paragraphs). */
int gemm_f32(int64_t M, int64_t N, int64_t K,
             const float *A, int64_t lda,
             const float *B, int64_t ldb,
             float *C, int64_t ldc,
             void *stream);

/* C = A.B with the single-buffered K-loop (two barriers per K step); tile configuration
 * from the dispatch table's single-buffered column for this shape (the cost model's best
 * single-buffered configuration for a shape not in the table). */
int gemm_f32_sb(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream);

/* C = A.B with the double-buffered K-loop (one barrier per K step); tile configuration
 * from the dispatch table's double-buffered column for this shape (the cost model's best
 * double-buffered configuration for a shape not in the table). */
int gemm_f32_db(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream);

/* C = A.B with the multi-stage direct-to-LDS K-loop; tile configuration from the
 * dispatch table's multi-stage column for this shape (the cost model's pick for a shape
 * not in the table).  Edge, misaligned and K-ragged
 * tiles of the launch run the guarded double-buffered loop instead. */
int gemm_f32_ms(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                void *stream);

/* C = A.B with an explicit variant (GEMMF32_VARIANT_SB, _DB, _MS, _SB3 or _KS; _AUTO =
 * dispatch table) and tile configuration id (0 .. gemm_f32_num_configs()-1; -1 = dispatch
 * table).  For measurement and tests: every (variant, configuration) pair computes the
 * same product.  A configuration without a kernel for the variant
 * (gemm_f32_config_variants) gives GEMMF32_ERR_BAD_CONFIG; with _AUTO and a forced
 * configuration that lacks the picked variant, the double-buffered kernel runs. */
int gemm_f32_ex(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                int variant, int cfg_id,
                void *stream);

/* C = A.B with the K range split into chunks (whole multiples of 64, so at most the
 * requested number are used), for shapes whose M x N tiles cannot fill the GPU, such as
 * the skinny decode-like regime the case study mentions ("Case Study: The Double-Buffered
 * GEMM", paragraph on the three regimes), or leave the last round of workgroups partly
 * empty.
 *   splits = s in 1 .. 64: every tile is split into s chunks; chunk y's partial product
 *            is an M x N plane (rows of N floats) at workspace + y * M * N.
 *   splits = -s, s in 2 .. 64 (tail split): the tiles that fill whole rounds of
 *            workgroups run over the whole K range into C; only the tiles of the last,
 *            partly filled round are split, their chunks packed as tile-sized blocks of
 *            the workspace.  A product with no full round of tiles splits every tile.
 *   splits = 0: the modelled choice of gemm_f32_splitk_select.
 * A second kernel then sums each element's partials into C in the fixed chunk order, so
 * the result is deterministic (it differs in rounding, within the accuracy of one
 * product, from the unsplit one).  The `workspace` is device memory of at least
 * gemm_f32_splitk_workspace(M, N, K, splits) floats, 4-byte aligned, overlapping none of
 * A, B, C; it is owned by the caller and overwritten, and it may be NULL when fewer than
 * two chunks result.  Both kernels go on `stream`.  Errors as for gemm_f32, plus
 * GEMMF32_ERR_BAD_CONFIG for `splits` outside -64 .. 64 or equal to -1,
 * GEMMF32_ERR_BAD_LD for a workspace that is too small, GEMMF32_ERR_NULL_PTR /
 * _MISALIGNED / _ALIAS for a bad workspace pointer. */
int gemm_f32_splitk(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    float *C, int64_t ldc,
                    int splits, float *workspace, int64_t workspace_floats,
                    void *stream);

/* For callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same product, split and launches as
 * gemm_f32_splitk, but the partial products go to a scratch array the library holds in
 * device memory (a file-scope __device__ array of GEMMF32_SCRATCH_FLOATS floats, 32 MiB,
 * one copy per device, held from the library's first use on that device until the
 * process ends), so the call itself allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine.  The caller still passes A, B and C.
 *   splits: as for gemm_f32_splitk (0 = the modelled choice of gemm_f32_splitk_select).
 *   The device is the one `stream` belongs to (the current device for NULL).  Its first
 *   call on a device looks up the array's device address (hipGetSymbolAddress, with that
 *   device current) and keeps it.
 * The array is shared by every call on its device and keeps the last call's partials; each
 * call overwrites every partial it reads before reading it, so nothing needs clearing.
 * Calls on one device whose kernels can run at the same time (different streams without
 * ordering between them) race on the array and give wrong results; calls ordered on one
 * stream are safe.
 * Errors: as for gemm_f32_splitk, with GEMMF32_ERR_SCRATCH_LIMIT when the split needs more
 * than GEMMF32_SCRATCH_FLOATS floats (gemm_f32_splitk_workspace gives the need; pick
 * fewer splits or use gemm_f32_splitk with a workspace of the caller's), and
 * GEMMF32_ERR_HIP when the device or the array's address cannot be found. */
int gemm_f32_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            float *C, int64_t ldc,
                            int splits, void *stream);

/* Workspace floats gemm_f32_splitk needs for this shape and split count (0 = the modelled
 * choice; the result is 0 when it will not split), or a negative error code
 * (GEMMF32_ERR_TOO_LARGE for sizes beyond the limits of gemm_f32 or a workspace of more
 * than 2^61 bytes). */
int64_t gemm_f32_splitk_workspace(int64_t M, int64_t N, int64_t K, int splits);

/* The split count for a shape with the least modelled time among 1 (do not split), the
 * full splits 2, 4, 8, 16 and the tail splits -2, -4, -8, -16: the dispatch table's cost
 * model of the GEMM part plus the split overhead fitted to the measured split study; host
 * code only.  Negative sizes give GEMMF32_ERR_NEGATIVE_DIM. */
int gemm_f32_splitk_select(int64_t M, int64_t N, int64_t K);

/* The launches a gemm_f32_splitk call with this shape and split count (0 = the modelled
 * choice) would make, without launching: *variant and *cfg_id receive the GEMM kernel and
 * tile configuration, *chunks the number of K chunks of each split tile (1: no split, the
 * call is the plain gemm_f32 product), *split_from the number of tiles, in launch order,
 * that run whole over K (0 for a full split; all tiles when *chunks is 1).  Output
 * pointers may be NULL.  Pure host code.  Returns 0, GEMMF32_ERR_NEGATIVE_DIM, or
 * GEMMF32_ERR_BAD_CONFIG for a split count gemm_f32_splitk rejects. */
int gemm_f32_splitk_plan(int64_t M, int64_t N, int64_t K, int splits, int *variant,
                         int *cfg_id, int *chunks, int64_t *split_from);

/* The dispatch decision for a shape, without launching: *variant receives
 * GEMMF32_VARIANT_SB, _DB, _MS or _KS and *cfg_id the tile configuration id that gemm_f32
 * would launch for it.  The choice is made per shape because the pages measure the
 * double-buffered loop winning at one size, losing at another and tying at a third, and
 * conclude that no one kernel is fastest everywhere ("Double Buffering", last two
 * paragraphs; "Case Study: The Double-Buffered GEMM", paragraph on the three regimes).
 * Either output pointer may be NULL.  Pure host code (no GPU needed).  Returns
 * GEMMF32_ERR_NEGATIVE_DIM for negative sizes. */
int gemm_f32_select(int64_t M, int64_t N, int64_t K, int *variant, int *cfg_id);

/* Tile configuration id for an explicit variant (SB, DB or MS) and shape, as used by
 * gemm_f32_sb / gemm_f32_db / gemm_f32_ms.  Returns the id (>= 0) or a negative error
 * code. */
int gemm_f32_select_cfg(int64_t M, int64_t N, int64_t K, int variant);

/* Number of compiled tile configurations. */
int gemm_f32_num_configs(void);

/* Describe tile configuration cfg_id: output tile BM x BN, K tile BK, threads per
 * workgroup, and the LDS bytes one workgroup uses with one slot (single-buffered) and
 * with two slots (double-buffered).  Output pointers may be NULL.  Returns 0 or
 * GEMMF32_ERR_BAD_CONFIG. */
int gemm_f32_config_info(int cfg_id, int *BM, int *BN, int *BK, int *threads,
                         int *lds_bytes_sb, int *lds_bytes_db);

/* Multi-stage figures of tile configuration cfg_id: number of LDS stages and LDS bytes per
 * workgroup of the multi-stage kernel (0 and 0 for a configuration without one).  Output
 * pointers may be NULL.  Returns 0 or GEMMF32_ERR_BAD_CONFIG. */
int gemm_f32_config_ms(int cfg_id, int *stages, int *lds_bytes);

/* Variants tile configuration cfg_id has a kernel for: bit v set for GEMMF32_VARIANT_v
 * (the multi-stage kernel needs B tiles at least 64 wide; the K-split kernel exists for
 * one-wave configurations).  Returns the mask or GEMMF32_ERR_BAD_CONFIG. */
int gemm_f32_config_variants(int cfg_id);

/* Wave groups of the K-split kernel of tile configuration cfg_id (1: it has none), or
 * GEMMF32_ERR_BAD_CONFIG. */
int gemm_f32_config_ks(int cfg_id);

/* The HIP error code of this thread's last failed launch (0 if none). */
int gemm_f32_last_hip_error(void);

/* Static description of an error code (never NULL). */
const char *gemm_f32_strerror(int code);

/* Library version string, e.g. "gemmf32 0.1.0 gfx950". */
const char *gemm_f32_version(void);

/* Measurement aid, not a GEMM: the FP32 matrix-core ceiling at the clock the device runs
 * at.  The pages price their kernels against nothing but time; this call gives the
 * attainable matrix-instruction rate of this device, against which a GEMM's TFLOP/s can
 * be read besides the 2.4 GHz specification peak.
 *
 * Enqueues one kernel on `stream`: `blocks` workgroups of 4 waves (256 lanes), each wave
 * issuing 16 * iters v_mfma_f32_32x32x2_f32 instructions (4096 FLOP each) on register
 * operands and nothing else in its loop.  FLOP per launch = blocks * 4 * 16 * iters * 4096.
 *   out  device buffer of blocks * 256 floats (one per lane, written; keeps the work live)
 *   rec  device buffer of blocks * 8 uint64 (written): for wave w = 4 * block + wave-in-
 *        block, rec[2w] = shader-clock cycles of its loop (s_memtime) and rec[2w+1] =
 *        100 MHz wall-clock ticks of the same interval (s_memrealtime); their ratio
 *        times 0.1 GHz is the shader clock.
 * Errors: GEMMF32_ERR_TOO_LARGE if blocks is outside 1..65536 or iters outside 0..2^20;
 * GEMMF32_ERR_NULL_PTR / GEMMF32_ERR_MISALIGNED for out (4-byte) or rec (8-byte);
 * GEMMF32_ERR_HIP if the launch fails.  Validation precedes any HIP call. */
int gemm_f32_peak_probe(int blocks, int iters, float *out, uint64_t *rec, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMMF32_H */
