// The STREAM kernel family: small token counts (decode), where the GEMM is
// bound by reading the weight matrix B once from HBM.
//
// Each workgroup owns tile_n = 16*RB*WN weight rows and tile_m = 16*TB
// tokens of one K split.  Its WN x WK waves split the rows (WN) and the
// split's K range (WK).  Every weight byte is used by exactly one matrix-core
// instruction, so B goes straight from HBM into registers with 16-byte
// non-temporal loads in the matrix-core operand layout, double-buffered U
// steps deep so 2*U*RB steps of loads stay in flight per wave.  Within a
// 128-byte K step, lane group g = lane/16 feeds the matrix core the bytes
// [16g, 16g+16) as its first 16-byte piece and [64+16g, 64+16g+16) as its
// second, so each load instruction reads 64 contiguous bytes of each of its
// 16 rows (A uses the same assignment, so every K slot pairs the same k).  Staging B through LDS would add traffic and
// a barrier per step without any reuse to pay for it.  The small activation
// tile A (tokens) is re-read from L1/L2 by each wave.
//
// SWAP selects the variant ("Kernel Implementation" section of "Building a
// High-Performance and Portable vLLM Linear Backend with Helion"):
//   SWAP = false (Standard): matrix-core rows = tokens, columns = weights.
//   SWAP = true  (Swap-AB):  computes Y^T = B A^T, rows = weights and the
//                            token dimension on the matrix core's N side;
//                            each lane then owns 4 consecutive output
//                            columns n of one token, stored as 8 bytes.
// Split-K (same section) is grid.z: each split sums a contiguous 128-aligned
// K range; partials go to the workspace and are summed in split order,
// either by the last split to arrive (counter per tile) or by a second
// kernel.
//
// Block_FP8 (the post's "Helion Linear Backend / Scope" section): a 128-byte
// K step is exactly one 1x128 activation group and one column of 128x128
// weight blocks, so each step's product goes into a zeroed accumulator and
// is added to the running sum times sA[t][g] * sB[n/128][g] in fp32.
#pragma once

#include "qlin_device.h"

namespace qlin {

template <int FMT, int SCAL, int TB, int RB, int U>
struct StreamFrag {
    v4i b[U][RB][2];
    v4i a[U][TB][2];
    float sb[SCAL == SC_BLOCK ? U : 1][RB];
    float sa[SCAL == SC_BLOCK ? U : 1][TB][4];
};

template <int FMT, int SCAL, bool SWAP, int TB, int RB, int WN, int WK, int U>
__global__ void __launch_bounds__(64 * WN * WK)
k_stream(KArgs p_)
{
    KArgs p = p_;
    if (p.group_off && !enter_group<SCAL>(p))
        return;
    typedef typename AccT<FMT>::v4 A4;
    typedef typename AccT<FMT>::scalar AS;
    typedef StreamFrag<FMT, SCAL, TB, RB, U> Frag;
    constexpr int ROWS_W = 16 * RB;
    constexpr int TILE_N = ROWS_W * WN;
    constexpr int TILE_M = 16 * TB;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % WN;
    const int wk = wave / WN;
    const int r16 = lane & 15;
    const int g = lane >> 4;

    const int nw0 = blockIdx.x * TILE_N + wn * ROWS_W;
    const int m0 = blockIdx.y * TILE_M;
    const int split = split_index(p);
    if (m0 >= p.M)
        return;                 // a group with fewer rows than the grid covers

    const int KS = (p.K + 127) >> 7;
    const int s_beg = min(KS, split * p.steps_per_split);
    const int s_end = min(KS, s_beg + p.steps_per_split);
    const int per_w = (s_end - s_beg + WK - 1) / WK;
    const int w_beg = min(s_end, s_beg + wk * per_w);
    const int w_end = min(s_end, w_beg + per_w);

    const uint8_t *brow[RB];
    bool bok[RB];
    int nb[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int n = nw0 + rb * 16 + r16;
        bok[rb] = n < p.N;
        brow[rb] = p.B + (int64_t)(bok[rb] ? n : 0) * p.ldb + g * 16;
        nb[rb] = (nw0 + rb * 16) >> 7;
    }
    const uint8_t *arow[TB];
    bool aok[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = m0 + tb * 16 + r16;
        aok[tb] = t < p.M;
        arow[tb] = p.A + (int64_t)(aok[tb] ? t : 0) * p.lda + g * 16;
    }

    A4 acc[RB][TB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            acc[rb][tb] = A4{0, 0, 0, 0};

    auto load = [&](Frag &f, int s) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = s + u;
            const bool sv = st < w_end;
            const int kb = st * 128;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool ok = sv && bok[rb] && (kb + h * 64 + g * 16 < p.K);
                    f.b[u][rb][h] = ok ? ld_nt(brow[rb] + kb + h * 64) : zero4i();
                }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool ok = sv && aok[tb] && (kb + h * 64 + g * 16 < p.K);
                    f.a[u][tb][h] = ok ? ld16(arow[tb] + kb + h * 64) : zero4i();
                }
            if constexpr (SCAL == SC_BLOCK) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const bool ok = sv && (nw0 + rb * 16 < p.N);
                    f.sb[SCAL == SC_BLOCK ? u : 0][rb] = ok ? p.sB[(int64_t)nb[rb] * p.G + st] : 0.f;
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    if constexpr (SWAP) {
                        const int t = m0 + tb * 16 + r16;
                        const bool ok = sv && t < p.M;
                        f.sa[SCAL == SC_BLOCK ? u : 0][tb][0] = ok ? p.sA[(int64_t)t * p.G + st] : 0.f;
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int t = m0 + tb * 16 + 4 * g + v;
                            const bool ok = sv && t < p.M;
                            f.sa[SCAL == SC_BLOCK ? u : 0][tb][v] = ok ? p.sA[(int64_t)t * p.G + st] : 0.f;
                        }
                    }
                }
            }
        }
    };

    auto compute = [&](const Frag &f) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const v4i *bf = f.b[u][rb];
                    const v4i *af = f.a[u][tb];
                    if constexpr (SCAL == SC_BLOCK) {
                        A4 z = A4{0, 0, 0, 0};
                        A4 pz = SWAP ? mma16<FMT>(bf[0], bf[1], af[0], af[1], z)
                                     : mma16<FMT>(af[0], af[1], bf[0], bf[1], z);
                        const int uu = SCAL == SC_BLOCK ? u : 0;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float s = (SWAP ? f.sa[uu][tb][0] : f.sa[uu][tb][v]) * f.sb[uu][rb];
                            acc[rb][tb][v] = __builtin_fmaf((float)pz[v], s, (float)acc[rb][tb][v]);
                        }
                    } else {
                        acc[rb][tb] = SWAP ? mma16<FMT>(bf[0], bf[1], af[0], af[1], acc[rb][tb])
                                           : mma16<FMT>(af[0], af[1], bf[0], bf[1], acc[rb][tb]);
                    }
                }
    };

    // Register double buffer: the loads of step group i+1 are in flight
    // while group i runs on the matrix cores.
    {
        Frag f0, f1;
        int s = w_beg;
        if (s < w_end)
            load(f0, s);
        while (s < w_end) {
            if (s + U < w_end)
                load(f1, s + U);
            compute(f0);
            s += U;
            if (s >= w_end)
                break;
            if (s + U < w_end)
                load(f0, s + U);
            compute(f1);
            s += U;
        }
    }

    // Combine the WK waves of a row group in fixed order (wave 0 first).
    if (WK > 1) {
        __shared__ AS red[WK > 1 ? WK - 1 : 1][WN][RB * TB * 4][64];
        if (wk > 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[wk - 1][wn][(rb * TB + tb) * 4 + v][lane] = acc[rb][tb][v];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int j = 0; j < WK - 1; ++j)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[rb][tb][v] += red[j][wn][(rb * TB + tb) * 4 + v][lane];
        }
    }

    // Output positions of this lane's accumulators.
    //   SWAP:     n = nw0 + 16*rb + 4*g + v,  t = m0 + 16*tb + r16
    //   standard: n = nw0 + 16*rb + r16,      t = m0 + 16*tb + 4*g + v
    auto emit = [&](const A4 (&val)[RB][TB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                if (SWAP) {
                    const int t = m0 + tb * 16 + r16;
                    const int n = nw0 + rb * 16 + 4 * g;
                    if (t >= p.M)
                        continue;
                    if (n + 3 < p.N) {
                        store_final4<FMT, SCAL>(p, t, n, val[rb][tb]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (n + v < p.N)
                                store_final<FMT, SCAL>(p, t, n + v, val[rb][tb][v]);
                    }
                } else {
                    const int n = nw0 + rb * 16 + r16;
                    if (n >= p.N)
                        continue;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = m0 + tb * 16 + 4 * g + v;
                        if (t < p.M)
                            store_final<FMT, SCAL>(p, t, n, val[rb][tb][v]);
                    }
                }
            }
    };

    if (p.split_k == 1) {
        if (wk == 0)
            emit(acc);
        return;
    }

    // Split-K: write this split's partial sums.  For the two-pass reduction
    // plain stores suffice (the kernel boundary orders them before the
    // second pass); the last-arriver exchange uses device-coherent stores.
    const bool la = p.reduce == QLIN_REDUCE_LAST_ARRIVER;
    if (wk == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = SWAP ? m0 + tb * 16 + r16 : m0 + tb * 16 + 4 * g + v;
                    const int n = SWAP ? nw0 + rb * 16 + 4 * g + v : nw0 + rb * 16 + r16;
                    if (t < p.M && n < p.N) {
                        AS *d = part_ptr<FMT>(p, split, t, n);
                        if (la)
                            st_dev(d, (AS)acc[rb][tb][v]);
                        else
                            *d = acc[rb][tb][v];
                    }
                }
            }
    }
    if (!la)
        return;

    // Last arriver: the final split to finish sums all partials of the tile
    // in split order 0..split_k-1 and applies the epilogue.
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    if (!arrive_last(p.counters + tile, p.split_k))
        return;
    if (wk == 0) {
        A4 sum[RB][TB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                sum[rb][tb] = A4{0, 0, 0, 0};
                for (int s = 0; s < p.split_k; ++s) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = SWAP ? m0 + tb * 16 + r16 : m0 + tb * 16 + 4 * g + v;
                        const int n = SWAP ? nw0 + rb * 16 + 4 * g + v : nw0 + rb * 16 + r16;
                        if (t < p.M && n < p.N)
                            sum[rb][tb][v] += ld_dev(part_ptr<FMT>(p, s, t, n));
                    }
                }
            }
        emit(sum);
    }
    rearm(p.counters + tile);
}

template <int FMT, int SCAL, bool SWAP, int TB, int RB, int WN, int WK, int U>
hipError_t launch_stream(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_stream<FMT, SCAL, SWAP, TB, RB, WN, WK, U>), grid,
                       dim3(64 * WN * WK), 0, s, a);
    return hipGetLastError();
}

#define QLIN_STREAM_INSTANCE(FMT, SCAL, BIT, SW, TB, RB, WN, WK, U)                         \
    {{QLIN_KERNEL_STREAM, SW, 16 * (TB), 16 * (RB) * (WN), 128 * (U), WN, WK, 2, 1, 0},      \
     BIT, FMT, SCAL, &launch_stream<FMT, SCAL, (SW) != 0, TB, RB, WN, WK, U>}

// The shape list shared by the three formats: (RB, WN, WK, U).
#define QLIN_STREAM_SHAPES(X, FMT, SCAL, BIT, SW, TB) \
    X(FMT, SCAL, BIT, SW, TB, 1, 1, 4, 4),            \
    X(FMT, SCAL, BIT, SW, TB, 1, 1, 4, 8),            \
    X(FMT, SCAL, BIT, SW, TB, 1, 1, 8, 2),            \
    X(FMT, SCAL, BIT, SW, TB, 1, 1, 8, 4),            \
    X(FMT, SCAL, BIT, SW, TB, 2, 1, 8, 2),            \
    X(FMT, SCAL, BIT, SW, TB, 1, 2, 2, 4),            \
    X(FMT, SCAL, BIT, SW, TB, 1, 4, 1, 4),            \
    X(FMT, SCAL, BIT, SW, TB, 2, 1, 4, 2),            \
    X(FMT, SCAL, BIT, SW, TB, 2, 2, 2, 2),            \
    X(FMT, SCAL, BIT, SW, TB, 2, 4, 1, 2),            \
    X(FMT, SCAL, BIT, SW, TB, 4, 1, 4, 1),            \
    X(FMT, SCAL, BIT, SW, TB, 4, 2, 2, 1)

// 16 waves (1024 threads) leave 128 registers per lane: one token block only.
#define QLIN_STREAM_SHAPES_TB1(X, FMT, SCAL, BIT, SW) \
    X(FMT, SCAL, BIT, SW, 1, 1, 1, 16, 2)

#define QLIN_STREAM_ALL(FMT, SCAL, BIT)                                   \
    QLIN_STREAM_SHAPES_TB1(QLIN_STREAM_INSTANCE, FMT, SCAL, BIT, 0),      \
    QLIN_STREAM_SHAPES_TB1(QLIN_STREAM_INSTANCE, FMT, SCAL, BIT, 1),      \
    QLIN_STREAM_SHAPES(QLIN_STREAM_INSTANCE, FMT, SCAL, BIT, 0, 1),       \
    QLIN_STREAM_SHAPES(QLIN_STREAM_INSTANCE, FMT, SCAL, BIT, 0, 2),       \
    QLIN_STREAM_SHAPES(QLIN_STREAM_INSTANCE, FMT, SCAL, BIT, 1, 1),       \
    QLIN_STREAM_SHAPES(QLIN_STREAM_INSTANCE, FMT, SCAL, BIT, 1, 2)

}  // namespace qlin
