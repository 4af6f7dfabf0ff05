// Internal declarations shared by the translation units of libqlinear.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qlinear.h"

namespace qlin {

enum Fmt { FMT_E4M3 = 0, FMT_INT8 = 1 };
enum Scal { SC_TC = 0, SC_BLOCK = 1 };

// Which of the three formats a kernel instance serves (bit mask).
enum FmtBit { FB_FP8 = 1, FB_INT8 = 2, FB_BLOCK = 4 };

// Kernel arguments, passed by value.  All sizes fit 32 bits for the
// supported problem range (checked by the host); row offsets are formed in
// 64 bits inside the kernels.
struct KArgs {
    const uint8_t *A;
    const uint8_t *B;
    const float *sA;
    const float *sB;
    uint16_t *Y;         // bf16 output, or NULL in raw-accumulator mode
    int32_t *acc_out;    // raw int32 accumulators (INT8 test hook), or NULL
    void *part;          // split-K partials [split_k][M][N] (4-byte elements)
    int32_t *counters;   // last-arriver counters, one per output tile
    int M, N, K;
    int lda, ldb, ldy, ldacc;
    int G;               // K / 128 (block scale columns)
    int split_k;
    int steps_per_split; // 128-byte K steps per split
    int reduce;          // qlin_reduce
    int nspread;         // STREAM_LDS spread placement: 8-row units (ceil(N/8)) shared
                         // evenly over grid.x; 0 = tiles of tile_n rows
    // Grouped GEMM (mixture of experts): grid.z is the group; group g owns
    // rows group_off[g] .. group_off[g+1]-1 of A, sA and Y (at most M of
    // them) and the weights B + g * b_gstride bytes, sB + g * sb_gstride.
    // NULL for an ordinary call.
    const int32_t *group_off;
    int64_t b_gstride;
    int64_t sb_gstride;
};

// Host-side description of a problem.
struct Problem {
    int fmt;             // Fmt
    int scal;            // Scal
    int64_t M, N, K;
    const void *A;
    int64_t lda;
    const float *sA;
    const void *B;
    int64_t ldb;
    const float *sB;
    void *Y;
    int64_t ldy;
    int32_t *acc_out;    // non-NULL selects the raw int32 output
    int64_t ldacc;
    void *ws;
    size_t ws_bytes;
    hipStream_t stream;
    // grouped GEMM: groups > 0 and the device row offsets of the groups;
    // M is then the bound on rows per group
    int64_t groups;
    const int32_t *group_off;
    int64_t b_gstride;   // bytes
    int64_t sb_gstride;  // floats
};

typedef hipError_t (*LaunchFn)(const KArgs &a, dim3 grid, hipStream_t s);

struct Instance {
    qlin_config cfg;     // split_k = 1, reduce = 0 in the registry
    int fmt_mask;        // FmtBit
    int fmt, scal;       // the (format, scaling) the function was built for
    LaunchFn fn;
};

// Registries of built kernel instances, one per translation unit.
const Instance *stream_instances_fp8(int *count);
const Instance *stream_instances_int8(int *count);
const Instance *stream_instances_block(int *count);
const Instance *tile_instances_fp8(int *count);
const Instance *tile_instances_int8(int *count);
const Instance *tile_instances_block(int *count);
const Instance *stream_lds_instances_fp8(int *count);
const Instance *stream_lds_instances_int8(int *count);
const Instance *stream_lds_instances_block(int *count);
const Instance *gemv_instances(int *count);
const Instance *stream_tok_instances_fp8(int *count);
const Instance *stream_tok_instances_int8(int *count);
const Instance *stream_own_instances(int *count);
const Instance *tile_h_instances_fp8(int *count);
const Instance *tile_h_instances_int8(int *count);

// Split-K two-pass reduction + epilogue.
hipError_t launch_reduce(int fmt, int scal, const KArgs &a, hipStream_t s);

// The host dispatcher (qlin_api.cpp), for entry points in other units:
// validate, select (or check) the config and launch; validate only; build a Problem; the
// workspace bytes the selected config needs; the size of the counter region
// at the start of every workspace.
qlin_status run_problem(const Problem &pb, const qlin_config *cfg);
qlin_status check_problem(const Problem &pb);   // argument checks only, no HIP call
Problem problem(int fmt, int scal, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                const float *sA, const void *B, int64_t ldb, const float *sB, void *Y,
                int64_t ldy, void *ws, size_t ws_bytes, void *stream);
size_t selected_workspace_bytes(int fmt, int scal, int64_t M, int64_t N, int64_t K);
size_t counter_bytes();

}  // namespace qlin
