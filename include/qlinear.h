/*
 * qlinear.h -- C ABI of libqlinear.so, the MI355X (gfx950) quantized
 * linear-layer GEMM.
 *
 * The operation (restated from "Building a High-Performance and Portable vLLM
 * Linear Backend with Helion", section "Helion Linear Backend / Scope"):
 *
 *   FP8_Dynamic   Y[m,n] = bf16( sA[m] * sB[n] * sum_k A[m,k] * B[n,k] )
 *                 A, B in OCP e4m3fn; one fp32 scale per activation token m
 *                 and per weight output channel n.
 *   W8A8_INT8     the same with int8 A, B (exact int32 accumulation).
 *   Block_FP8     Y[m,n] = bf16( sum_g sA[m,g] * sB[n/128,g]
 *                                   * sum_{k in group g} A[m,k] * B[n,k] )
 *                 e4m3 A, B; one activation scale per 1x128 K group, one
 *                 weight scale per 128x128 block (groups start at k = 0 and
 *                 blocks at n = 0).
 *
 * Layouts: A is [M rows][lda bytes], B is [N rows][ldb bytes], both
 * K-contiguous (B is the weight in its [out_features, in_features] form, so
 * Y = A * B^T).  Y is [M rows][ldy elements] of bfloat16 bit patterns.
 * Scales are fp32: sA [M] and sB [N] (token/channel), or row-major
 * sA [M][K/128] and sB [N/128][K/128] (block).
 *
 * The same post's "Kernel Implementation" section describes the algorithm
 * variants exposed here as configuration: Standard, Split-K (K partitioned
 * across workgroups; here reduced through a workspace in a fixed order, so
 * results are run-to-run reproducible) and Swap-AB (computing the transposed
 * product so the small token dimension sits on the matrix core's N side).
 * The techfeed.io summary of the post gives the tunable domains: split_k is
 * a power of two from 1 to 256, swap_ab is a boolean.  The kernel, variant,
 * tiles and split_k are looked up per (format, M, N, K) in a table written
 * by an offline sweep on the MI355X itself.
 *
 * Conventions
 *  - Ownership: the caller owns every buffer (A, B, scales, Y, workspace);
 *    all are device pointers.  The library never allocates, frees or
 *    synchronises on the call path; its only state is the host-side config
 *    table.
 *  - Asynchrony: calls enqueue kernels on `stream` (a hipStream_t; NULL is
 *    the default stream) and return at once.  No host synchronisation, no
 *    allocation and no memset is issued, so calls may be captured into a
 *    HIP graph.
 *  - Errors: argument checks run on the host before any HIP call; a failed
 *    check returns its status and launches nothing.  A launch failure
 *    returns QLIN_ERR_HIP.  Device faults surface at the caller's next
 *    stream synchronisation.
 *  - Shapes: M >= 0 and N >= 0 (M == 0 or N == 0 returns QLIN_OK with no
 *    launch); K > 0 and K % 16 == 0; lda, ldb >= K and % 16 == 0; ldy >= N.
 *    Block_FP8 also needs K % 128 == 0 and N % 128 == 0.  Any M and, for
 *    token/channel scaling, any N are handled (tails are masked).
 *  - Alignment: A, B, Y and the workspace 16-byte aligned; scales 4-byte.
 *  - Workspace: split_k > 1 needs `workspace_bytes >= qlin_workspace_size(..)`
 *    for the selected config (0 when split_k == 1).  Layout: the first
 *    128 KiB hold one int32 counter per output tile for the last-arriver
 *    reduction, then the fp32/int32 split partials [split_k][M][N].  The
 *    counter region must hold zeros before the first call (allocate the
 *    workspace zeroed); every completed call leaves it zeroed again, and no
 *    call writes partials into it, so one workspace serves every config.
 *    Calls that may overlap in time (different streams) need distinct
 *    workspaces.
 *  - Threading: concurrent calls are safe, qlin_load_config_table included:
 *    a call that overlaps a table replacement uses either the old or the new
 *    table (replaced tables stay in host memory until the process ends).
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLINEAR_ABI_VERSION 1

typedef enum qlin_status {
    QLIN_OK = 0,
    QLIN_ERR_NULL_POINTER = 1,  /* a required pointer is NULL */
    QLIN_ERR_BAD_SHAPE = 2,     /* M/N/K out of range or not a required multiple */
    QLIN_ERR_BAD_STRIDE = 3,    /* lda/ldb/ldy too small or not a required multiple */
    QLIN_ERR_MISALIGNED = 4,    /* a pointer violates the alignment rules */
    QLIN_ERR_WORKSPACE = 5,     /* workspace missing or smaller than required */
    QLIN_ERR_BAD_CONFIG = 6,    /* explicit config not valid / not built for this shape */
    QLIN_ERR_CONFIG_FILE = 7,   /* config table file unreadable or malformed */
    QLIN_ERR_HIP = 8,           /* a HIP call or kernel launch failed */
    QLIN_ERR_BAD_ARGUMENT = 9   /* unknown enum value */
} qlin_status;

typedef enum qlin_dtype {
    QLIN_E4M3 = 0,              /* OCP e4m3fn bytes */
    QLIN_INT8 = 1               /* two's-complement int8 bytes */
} qlin_dtype;

typedef enum qlin_scaling {
    QLIN_TOKEN_CHANNEL = 0,     /* sA [M], sB [N] */
    QLIN_BLOCK128 = 1           /* sA [M][K/128], sB [N/128][K/128]; e4m3 only */
} qlin_scaling;

typedef enum qlin_kernel {
    QLIN_KERNEL_STREAM = 0,     /* weights streamed HBM -> registers; small M */
    QLIN_KERNEL_TILE = 1,       /* A and B tiles staged through a double-buffered LDS ring; large M */
    QLIN_KERNEL_STREAM_LDS = 2, /* weights and tokens copied HBM -> LDS in 1 KB row segments
                                   through a multi-stage ring; small M; K % 256 == 0 */
    QLIN_KERNEL_GEMV = 3,       /* one wave per weight row, dot products on the vector ALUs;
                                   1-8 tokens (token/channel scaling) or 1-2 tokens
                                   (block scaling); split_k = 1 */
    QLIN_KERNEL_STREAM_TOK = 4  /* one persistent workgroup per CU: the token rows of its K
                                   range copied into LDS once, weight rows streamed through an
                                   LDS ring; token/channel scaling, Swap-AB, 8-32 tokens per
                                   token tile; K % 256 == 0, a split's K range at most
                                   81920 / tile_m bytes, split_k > 1 with the two-pass
                                   reduction; not for grouped calls */
} qlin_kernel;

typedef enum qlin_variant {
    QLIN_STANDARD = 0,          /* matrix-core rows = tokens, columns = weights */
    QLIN_SWAP_AB = 1            /* computes Y^T = B A^T: rows = weights, columns = tokens */
} qlin_variant;

typedef enum qlin_reduce {
    QLIN_REDUCE_TWO_PASS = 0,   /* split partials summed by a second kernel */
    QLIN_REDUCE_LAST_ARRIVER = 1 /* summed in-kernel by the last split to finish */
} qlin_reduce;

/* One launch configuration.  For the STREAM kernel: tile_m = tokens per
 * workgroup (16 or 32), tile_n = weight rows per workgroup, tile_k = K bytes
 * each wave loads per pipeline step (multiple of 128), waves_n x waves_k
 * waves split the tile's rows and the split's K range.  For STREAM_LDS:
 * tile_m / tile_n as for STREAM, tile_k = bytes per row per LDS chunk (512
 * or 1024), waves_k waves share each chunk's K steps, stages = ring depth;
 * tile_k = 256 is the wide-row form (Swap-AB only, tile_n = 128 or 256 rows,
 * each of the waves_k waves owning whole 16-row blocks for every K step),
 * waves_n = 1 for workgroups of tile_n weight rows each, or 2 for spread
 * placement: N in 8-row units shared evenly over a grid that is a multiple
 * of the device's compute units per (token tile, split), at most tile_n
 * rows per workgroup.  For STREAM_TOK: tile_m = token rows per token tile,
 * tile_n = 16 * waves_k weight rows per ring stage, tile_k = chunk bytes,
 * waves_k = waves (one 16-row block each), stages = ring depth.
 * For the TILE kernel:
 * tile_m x tile_n output tile, waves_n x waves_k is the wave grid over the
 * tile (rows x columns), stages = depth of the LDS ring; tile_k = 128 is the
 * ring of whole 128-byte K steps (all three formats), tile_k = 64 the ring of
 * 64-byte half-steps with fragments prefetched into registers (token/channel
 * scaling only).  split_k is 1..256, a power of two; each split covers a
 * contiguous, 128-aligned K range. */
typedef struct qlin_config {
    int32_t kernel;     /* qlin_kernel */
    int32_t variant;    /* qlin_variant */
    int32_t tile_m;
    int32_t tile_n;
    int32_t tile_k;
    int32_t waves_n;
    int32_t waves_k;
    int32_t stages;
    int32_t split_k;
    int32_t reduce;     /* qlin_reduce */
} qlin_config;

/* FP8_Dynamic (dt = QLIN_E4M3) and W8A8_INT8 (dt = QLIN_INT8) with per-token
 * a_scale[M] and per-channel b_scale[N].  Config from the table. */
qlin_status qlin_scaled_mm(qlin_dtype dt, int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda, const float *a_scale,
                           const void *B, int64_t ldb, const float *b_scale,
                           void *Y, int64_t ldy,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Block_FP8: e4m3 A and B, a_scale [M][K/128], b_scale [N/128][K/128]. */
qlin_status qlin_block_scaled_mm(int64_t M, int64_t N, int64_t K,
                                 const void *A, int64_t lda, const float *a_scale,
                                 const void *B, int64_t ldb, const float *b_scale,
                                 void *Y, int64_t ldy,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* The same two operations with an explicit configuration (tuning, tests).
 * cfg must name a built kernel instance; otherwise QLIN_ERR_BAD_CONFIG. */
qlin_status qlin_scaled_mm_cfg(qlin_dtype dt, int64_t M, int64_t N, int64_t K,
                               const void *A, int64_t lda, const float *a_scale,
                               const void *B, int64_t ldb, const float *b_scale,
                               void *Y, int64_t ldy,
                               void *workspace, size_t workspace_bytes, void *stream,
                               const qlin_config *cfg);
qlin_status qlin_block_scaled_mm_cfg(int64_t M, int64_t N, int64_t K,
                                     const void *A, int64_t lda, const float *a_scale,
                                     const void *B, int64_t ldb, const float *b_scale,
                                     void *Y, int64_t ldy,
                                     void *workspace, size_t workspace_bytes, void *stream,
                                     const qlin_config *cfg);

/* Grouped GEMM for mixture-of-experts layers: `groups` independent
 * scaled_mm / block_scaled_mm problems sharing N and K, in one launch.  The
 * ai-radar commentary "Helion in vLLM: il tuning dei GEMM diventa ricerca…",
 * section "Oltre Hopper: Blackwell, AMD, TPU e il perimetro del fork", names
 * MoE as the next target: many experts with few tokens each, where the
 * Split-K / Swap-AB choice matters more.  Reading: group g (an expert) owns
 * the rows group_offsets[g] .. group_offsets[g+1]-1 of A, a_scale and Y
 * (tokens sorted by expert) and its own weights B_g = B + g * b_group_stride
 * bytes with scales b_scale + g * b_scale_group_stride floats; each group's
 * result is exactly that of the single call on its slice.
 *
 * group_offsets: groups + 1 nondecreasing int32 values in DEVICE memory,
 * group_offsets[0] = 0 (the call reads them on the GPU, so routing computed
 * on the device needs no host round trip).  max_rows: a bound on any
 * group's row count (host value): the grid covers max_rows rows per group,
 * and rows of a group beyond max_rows are not computed.  A, a_scale and Y
 * must hold group_offsets[groups] rows.  Per-group layouts and scales as in
 * qlin_scaled_mm (token/channel) or qlin_block_scaled_mm (b_scale of a
 * group [N/128][K/128]).  b_group_stride % 16 == 0, both strides >= 0.
 * groups <= 65535 (0 is a no-op).  The config (NULL: the grouped choice,
 * qlin_select_grouped_config) runs with split_k = 1: the groups fill the
 * machine, grid.z carries the group, and no workspace is used; a config
 * with split_k > 1 is rejected.  Empty groups cost one early-exiting
 * workgroup per tile.  Asynchronous on `stream`; allocates nothing; errors
 * as for qlin_scaled_mm (the offsets are not checked on the host). */
qlin_status qlin_grouped_scaled_mm(qlin_dtype dt, int64_t groups, const int32_t *group_offsets,
                                   int64_t max_rows, int64_t N, int64_t K, const void *A,
                                   int64_t lda, const float *a_scale, const void *B, int64_t ldb,
                                   int64_t b_group_stride, const float *b_scale,
                                   int64_t b_scale_group_stride, void *Y, int64_t ldy, void *stream,
                                   const qlin_config *cfg);
/* The config a grouped call uses when given none (split_k = 1): the table's
 * grouped entry for (format, N, K) with the smallest rows-per-group bound
 * >= max_rows (else the largest bound), tuned on 128-expert layers; for
 * shapes without grouped entries, a kernel chosen by max_rows. */
qlin_status qlin_select_grouped_config(qlin_scaling sc, qlin_dtype dt, int64_t max_rows,
                                       int64_t N, int64_t K, qlin_config *out);
qlin_status qlin_grouped_block_scaled_mm(int64_t groups, const int32_t *group_offsets,
                                         int64_t max_rows, int64_t N, int64_t K, const void *A,
                                         int64_t lda, const float *a_scale, const void *B,
                                         int64_t ldb, int64_t b_group_stride, const float *b_scale,
                                         int64_t b_scale_group_stride, void *Y, int64_t ldy,
                                         void *stream, const qlin_config *cfg);

/* Test hook: the raw int32 dot products acc[M][ldacc] = A * B^T of W8A8_INT8
 * with the given config (NULL: the table's), no scaling, no rounding. */
qlin_status qlin_int8_accumulate(int64_t M, int64_t N, int64_t K,
                                 const void *A, int64_t lda, const void *B, int64_t ldb,
                                 int32_t *acc, int64_t ldacc,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 const qlin_config *cfg);

/* Activation quantization, the producer of A: dynamic per-token FP8 and
 * per-token-group FP8 quantization, items 1 and 5 of the kernel list in
 * "HelionがvLLMに統合 ..." (24-ai.news), section "vLLMに統合されたカーネル".
 *
 * X [M][ldx] bf16 bit patterns (row-major, K used per row) -> Q [M][ldq]
 * codes (e4m3 or int8 bytes) and fp32 scales, such that X ~= Q * scale.
 * Scale of a row (per token) or of a 1x128 group: amax / 448 (e4m3) or
 * amax / 127 (int8), one correctly rounded fp32 division, 1 when amax = 0.
 * Code: x / scale in fp32 (correctly rounded), clamped to +-448 and rounded
 * to the nearest e4m3 value, ties to even (int8: nearest integer, ties to
 * even, clamped to +-127).  The outputs feed qlin_scaled_mm /
 * qlin_block_scaled_mm as A and a_scale.
 *
 * Shapes: M >= 0 (0 is a no-op), 0 < K <= 2^20, K % 16 == 0 (per group:
 * K % 128 == 0).  ldx >= K with ldx % 8 == 0 (elements), ldq >= K with
 * ldq % 16 == 0 (bytes); X and Q 16-byte aligned, scale 4-byte aligned.
 * scale: [M] per token; [M][K/128] row-major per group.  The caller owns
 * every buffer; the call is asynchronous on `stream` (a hipStream_t) and
 * allocates nothing.  Errors as for qlin_scaled_mm. */
qlin_status qlin_quant_per_token(qlin_dtype dt, int64_t M, int64_t K,
                                 const uint16_t *X, int64_t ldx, void *Q, int64_t ldq,
                                 float *scale, void *stream);
qlin_status qlin_quant_per_group128(int64_t M, int64_t K, const uint16_t *X, int64_t ldx,
                                    void *Q, int64_t ldq, float *scale, void *stream);

/* Fused producers of A: RMS norm or SiLU-and-mul followed by the quantizer
 * above, in one pass; items 2, 3, 6 and 7 of the kernel list in
 * "HelionがvLLMに統合 ..." (24-ai.news), section "vLLMに統合されたカーネル"
 * (rms_norm_dynamic_per_token_quant, silu_and_mul_dynamic_per_token_quant,
 * rms_norm_per_block_quant, silu_and_mul_per_block_quant).  The pages give
 * names only.  Each call returns exactly what the quantizer returns on the
 * producer's bf16 output, where that output is the real-number value
 * rounded once to nearest-even bf16:
 *   RMS norm of a row of K:  h = x, or h = bf16(x + residual) when residual
 *     is not NULL (the residual row is then overwritten with h);
 *     y_k = bf16(h_k * weight_k / sqrt(sum_j(h_j^2) / K + eps)).
 *   SiLU-and-mul of a row of 2K values (gate in columns 0..K-1, up in
 *     K..2K-1):  y_k = bf16(gate_k / (1 + exp(-gate_k)) * up_k).
 * Per token: scale [M], dt e4m3 or int8.  Per block: 1x128 groups, e4m3,
 * scale [M][K/128] row-major, K % 128 == 0.
 *
 * Shapes: M >= 0 (0 is a no-op), 0 < K <= 2^20, K % 16 == 0.  X [M][ldx]
 * bf16 bits with ldx >= K (RMS norm) or >= 2K (SiLU-and-mul), ldx % 8 == 0;
 * residual [M][ldr], ldr >= K, ldr % 8 == 0; weight [K] bf16; eps finite
 * and > 0.  Q [M][ldq] codes, ldq >= K, ldq % 16 == 0.  X, residual,
 * weight and Q 16-byte aligned, scale 4-byte aligned.  The caller owns every
 * buffer; the call is asynchronous on `stream` (a hipStream_t) and allocates
 * nothing.  Errors as for qlin_scaled_mm (bad eps: QLIN_ERR_BAD_ARGUMENT). */
qlin_status qlin_rms_norm_dynamic_per_token_quant(qlin_dtype dt, int64_t M, int64_t K,
                                                  const uint16_t *X, int64_t ldx,
                                                  uint16_t *residual, int64_t ldr,
                                                  const uint16_t *weight, float eps, void *Q,
                                                  int64_t ldq, float *scale, void *stream);
qlin_status qlin_rms_norm_per_block_quant(int64_t M, int64_t K, const uint16_t *X, int64_t ldx,
                                          uint16_t *residual, int64_t ldr,
                                          const uint16_t *weight, float eps, void *Q,
                                          int64_t ldq, float *scale, void *stream);
qlin_status qlin_silu_and_mul_dynamic_per_token_quant(qlin_dtype dt, int64_t M, int64_t K,
                                                      const uint16_t *X, int64_t ldx, void *Q,
                                                      int64_t ldq, float *scale, void *stream);
qlin_status qlin_silu_and_mul_per_block_quant(int64_t M, int64_t K, const uint16_t *X,
                                              int64_t ldx, void *Q, int64_t ldq, float *scale,
                                              void *stream);

/* The config the table selects for a problem: the entry for (scaling, dt,
 * N, K) at the smallest tuned M >= M (else the largest tuned M); shapes not
 * in the table get the format's default for that M range. */
qlin_status qlin_select_config(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N,
                               int64_t K, qlin_config *out);

/* Workspace bytes needed by a config (NULL: the table's choice) for a
 * problem; 0 when split_k == 1. */
size_t qlin_workspace_size(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N, int64_t K,
                           const qlin_config *cfg);

/* Validate a config for a problem without launching (QLIN_OK if it would run). */
qlin_status qlin_check_config(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N,
                              int64_t K, const qlin_config *cfg);

/* Enumerate the built kernel instances: fills *out with instance i (split_k
 * and reduce set to 1 and 0) and returns QLIN_OK, or QLIN_ERR_BAD_ARGUMENT
 * past the end.  *fmt_mask gets bit0 = e4m3 token/channel, bit1 = int8,
 * bit2 = block. */
qlin_status qlin_kernel_instance(int32_t i, qlin_config *out, int32_t *fmt_mask);

/* Replace the config table with the text file at `path` (NULL or "" restores
 * the compiled-in table).  Format: one entry per line,
 *   <fmt> <N> <K> <M> <kernel> <variant> <tile_m> <tile_n> <tile_k>
 *   <waves_n> <waves_k> <stages> <split_k> <reduce>
 * with <fmt> one of fp8, int8, block_fp8; '#' starts a comment.  A line
 * starting with the word `grouped` (then the same fields, M being the bound
 * on rows per expert and split_k 1) configures grouped calls.  On error the
 * previous table is kept. */
qlin_status qlin_load_config_table(const char *path);

/* Number of entries in the active table. */
int32_t qlin_config_table_size(void);

const char *qlin_status_string(qlin_status s);
int32_t qlin_abi_version(void);

/* scaled_mm / block_scaled_mm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same validation, config selection, kernels and results as
 * qlin_scaled_mm (scaling QLIN_TOKEN_CHANNEL, dtype e4m3 or int8) and
 * qlin_block_scaled_mm (scaling QLIN_BLOCK128, dtype e4m3), with the split-K
 * workspace taken from a 32 MiB device array inside the library instead of
 * a caller's buffer.  Arguments as in those calls; the caller owns A, the
 * scales, B and Y.
 *  - The array is one per GPU, set up by the first call that needs it on that
 *    GPU (its device address looked up once; its counter region cleared by a
 *    small kernel on the caller's stream, recorded into the graph when that
 *    first call is being captured) and held until the process ends.
 *  - Nothing is allocated or freed, on the host or the device, on any call.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's partials: calls that may overlap in time on one GPU (different
 *    streams, or graphs replayed concurrently) race on it and must not be
 *    issued; calls ordered on one stream are safe.
 *  - QLIN_ERR_WORKSPACE when the selected config needs more than the array
 *    holds (32 MiB less 128 KiB of counters for the split partials
 *    split_k * M * N * 4 bytes: never at M <= 256 on the tuned shapes); no
 *    launch then.  QLIN_ERR_HIP when the device address cannot be obtained.
 *    Other errors as in qlin_scaled_mm. */
qlin_status qlin_scaled_mm_noalloc(qlin_scaling scaling, qlin_dtype dtype, int64_t M, int64_t N,
                                   int64_t K, const void *A, int64_t lda, const float *a_scale,
                                   const void *B, int64_t ldb, const float *b_scale, void *Y,
                                   int64_t ldy, void *stream);

/* Stream-capture state of `stream` (a hipStream_t; NULL is the null stream),
 * for callers that keep one split-K workspace per HIP graph: returns 1 and
 * sets *capture_id to the id of the capture in progress (unique per capture
 * within the process), 0 (and *capture_id = 0) when the stream is not
 * capturing, or -1 when the query fails or capture_id is NULL.  Launches
 * nothing and does not synchronise. */
int32_t qlin_stream_capture_id(void *stream, unsigned long long *capture_id);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
