// The TILE kernel family: larger token counts (prefill), where the GEMM is
// bound by the matrix cores and operand reuse through LDS pays.
//
// One workgroup computes a BM (tokens) x BN (weights) output tile of one K
// split with WM x WN waves, each owning a (BM/WM) x (BN/WN) sub-tile of
// 32x32 matrix-core blocks.  Per 128-byte K step both operand tiles are
// copied HBM/L2 -> LDS with global_load_lds_dwordx4 (16 bytes per lane
// written straight into LDS, no register staging), into a two-stage ring:
// the copy of step s+1 is in flight while step s is read from LDS
// (ds_read_b128) into the matrix cores.
//
// LDS layout of a stage: [BM rows of A][BN rows of B], 128 bytes per row.
// The eight 16-byte chunks of row r are stored XOR-swizzled, chunk c at slot
// c ^ f(r) with f(r) = (r & 7) ^ ((r >> 3) & 1), so that the 16 rows a
// quarter-wave reads with one ds_read_b128 hit distinct banks.  Because
// global_load_lds writes lane i's 16 bytes to slot (i % 8) of row (i / 8),
// the swizzle is applied on the global side: lane i fetches chunk
// (i % 8) ^ f(row) of its row.
//
// Tile order is XCD-aware: consecutive workgroup ids land on different XCDs
// (round-robin over 8), so ids are remapped to give every XCD a contiguous
// range of tiles, walked in groups of GM token tiles so that the tiles an
// XCD runs together share A rows and B rows in its own L2.
//
// Variants ("Kernel Implementation" section of "Building a High-Performance
// and Portable vLLM Linear Backend with Helion"): SWAP = false puts tokens
// on the matrix-core rows; SWAP = true computes the Y^T tile (weights on
// rows, tokens on the N side), giving each lane 4 consecutive output
// columns to store.  Split-K is grid.z, as in the stream kernel.
// Block_FP8 promotes each 128-wide K group into the running fp32 sum with
// sA[t][g] * sB[n/128][g] (built with SWAP only, where each lane needs one
// token scale per block and one weight-block scale per wave).
#pragma once

#include "qlin_device.h"

namespace qlin {

__device__ inline int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int FMT, int SCAL, bool SWAP, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
k_tile(KArgs p)
{
    typedef typename AccT<FMT>::v16 A16;
    typedef typename AccT<FMT>::scalar AS;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM;       // tokens per wave
    constexpr int WTN = BN / WN;       // weights per wave
    constexpr int FM = WTM / 32;
    constexpr int FN = WTN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int STAGE = ROWS * 128;
    constexpr int GM = 4;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
    static_assert(ROWS % 8 == 0, "rows");

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    // ---- XCD-aware tile id -> (token tile, weight tile)
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    const int T = tiles_m * tiles_n;
    int b = blockIdx.x;
    const int per = T >> 3;
    if (b < per * 8)
        b = (b & 7) * per + (b >> 3);
    const int group_tiles = GM * tiles_n;
    const int grp = b / group_tiles;
    const int first_m = grp * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int in_grp = b - grp * group_tiles;
    const int tm = first_m + in_grp % gsize;
    const int tn = in_grp / gsize;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // ---- K range of this split (128-byte steps)
    const int KS = p.K >> 7;
    const int split = blockIdx.z;
    const int s_beg = min(KS, split * p.steps_per_split);
    const int s_end = min(KS, s_beg + p.steps_per_split);

    // ---- per-lane global source of the stage copy.  Wave w copies row
    // groups w, w+NW, ...; each group is 8 rows = one 1 KB instruction.
    constexpr int GROUPS = ROWS / 8;
    constexpr int GPW = (GROUPS + NW - 1) / NW;
    const uint8_t *src[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int grp_i = wave + i * NW;
        const int row = grp_i * 8 + (lane >> 3);
        const uint8_t *base;
        int r;
        if (row < BM) {
            r = row;
            const int t = min(m0 + r, p.M - 1);   // rows past M feed only masked outputs
            base = p.A + (int64_t)t * p.lda;
        } else {
            r = row - BM;
            const int n = min(n0 + r, p.N - 1);
            base = p.B + (int64_t)n * p.ldb;
        }
        src[i] = base + 16 * ((lane & 7) ^ lds_swz(r));
    }

    auto issue = [&](int st, int stage) {
        uint8_t *dst0 = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int grp_i = wave + i * NW;
            if (GROUPS % NW == 0 || grp_i < GROUPS)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(src[i] + (int64_t)st * 128),
                    (__attribute__((address_space(3))) void *)(dst0 + grp_i * 1024), 16, 0, 0);
        }
    };

    // Block_FP8 scales of a step, prefetched with the stage copy.
    float sa_next[FM], sb_next[FN];
    auto load_scales = [&](int st) {
        if constexpr (SCAL == SC_BLOCK) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int t = min(m0 + wm * WTM + fm * 32 + (lane & 31), p.M - 1);
                sa_next[fm] = p.sA[(int64_t)t * p.G + st];
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int nbk = min(n0 + wn * WTN + fn * 32, p.N - 1) >> 7;
                sb_next[fn] = p.sB[(int64_t)nbk * p.G + st];
            }
        }
    };

    A16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[fm][fn][v] = 0;

    const int fr = lane & 31;          // fragment row
    const int fh = lane >> 5;          // 64-byte half of the K step

    if (s_beg < s_end) {
        issue(s_beg, 0);
        load_scales(s_beg);
    }
    for (int s = s_beg; s < s_end; ++s) {
        const int stage = (s - s_beg) & 1;
        float sa[FM], sb[FN];
        if constexpr (SCAL == SC_BLOCK) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) sa[fm] = sa_next[fm];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) sb[fn] = sb_next[fn];
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (s + 1 < s_end) {
            issue(s + 1, stage ^ 1);
            load_scales(s + 1);
        }
        const uint8_t *la = lds + stage * STAGE;
        const uint8_t *lb = la + BM * 128;
        v4i bf[FN][4];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int r = wn * WTN + fn * 32 + fr;
            const uint8_t *rowp = lb + r * 128;
            const int sw = lds_swz(r);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[fn][j] = *reinterpret_cast<const v4i *>(rowp + 16 * ((4 * fh + j) ^ sw));
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            v4i af[4];
            const int r = wm * WTM + fm * 32 + fr;
            const uint8_t *rowp = la + r * 128;
            const int sw = lds_swz(r);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                af[j] = *reinterpret_cast<const v4i *>(rowp + 16 * ((4 * fh + j) ^ sw));
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if constexpr (SCAL == SC_BLOCK) {
                    A16 z;
#pragma unroll
                    for (int v = 0; v < 16; ++v) z[v] = 0;
                    A16 pz = SWAP ? mma32<FMT>(bf[fn], af, z) : mma32<FMT>(af, bf[fn], z);
                    const float scale = sa[fm] * sb[fn];
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[fm][fn][v] = __builtin_fmaf((float)pz[v], scale, (float)acc[fm][fn][v]);
                } else {
                    acc[fm][fn] = SWAP ? mma32<FMT>(bf[fn], af, acc[fm][fn])
                                       : mma32<FMT>(af, bf[fn], acc[fm][fn]);
                }
            }
        }
    }

    // Output positions of acc[fm][fn][v] for this lane:
    //   SWAP:     t = tok0 + fr,  n = wgt0 + 8*(v/4) + 4*fh + v%4  (4 consecutive n per v/4)
    //   standard: t = tok0 + 8*(v/4) + 4*fh + v%4,  n = wgt0 + fr
    // with tok0 = m0 + wm*WTM + 32*fm and wgt0 = n0 + wn*WTN + 32*fn.
    auto emit = [&](const A16 (&val)[FM][FN]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int tok0 = m0 + wm * WTM + 32 * fm;
                const int wgt0 = n0 + wn * WTN + 32 * fn;
                if (SWAP) {
                    const int t = tok0 + fr;
                    if (t >= p.M)
                        continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = wgt0 + 8 * q + 4 * fh;
                        typename AccT<FMT>::v4 v4v;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v4v[j] = val[fm][fn][4 * q + j];
                        if (n + 3 < p.N) {
                            store_final4<FMT, SCAL>(p, t, n, v4v);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                if (n + j < p.N)
                                    store_final<FMT, SCAL>(p, t, n + j, v4v[j]);
                        }
                    }
                } else {
                    const int n = wgt0 + fr;
                    if (n >= p.N)
                        continue;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int t = tok0 + 8 * (v >> 2) + 4 * fh + (v & 3);
                        if (t < p.M)
                            store_final<FMT, SCAL>(p, t, n, val[fm][fn][v]);
                    }
                }
            }
    };

    if (p.split_k == 1) {
        emit(acc);
        return;
    }

    // Split-K partials (device-coherent stores for the last-arriver exchange)
    const bool la = p.reduce == QLIN_REDUCE_LAST_ARRIVER;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int tok0 = m0 + wm * WTM + 32 * fm;
            const int wgt0 = n0 + wn * WTN + 32 * fn;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = SWAP ? tok0 + fr : tok0 + 8 * (v >> 2) + 4 * fh + (v & 3);
                const int n = SWAP ? wgt0 + 8 * (v >> 2) + 4 * fh + (v & 3) : wgt0 + fr;
                if (t < p.M && n < p.N) {
                    AS *d = part_ptr<FMT>(p, split, t, n);
                    if (la)
                        st_dev(d, (AS)acc[fm][fn][v]);
                    else
                        *d = acc[fm][fn][v];
                }
            }
        }
    if (!la)
        return;

    const int tile = blockIdx.x;
    if (!arrive_last(p.counters + tile, p.split_k))
        return;
    A16 sum[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int tok0 = m0 + wm * WTM + 32 * fm;
            const int wgt0 = n0 + wn * WTN + 32 * fn;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = SWAP ? tok0 + fr : tok0 + 8 * (v >> 2) + 4 * fh + (v & 3);
                const int n = SWAP ? wgt0 + 8 * (v >> 2) + 4 * fh + (v & 3) : wgt0 + fr;
                AS a = 0;
                if (t < p.M && n < p.N)
                    for (int s = 0; s < p.split_k; ++s)
                        a += ld_dev(part_ptr<FMT>(p, s, t, n));
                sum[fm][fn][v] = a;
            }
        }
    emit(sum);
    rearm(p.counters + tile);
}

template <int FMT, int SCAL, bool SWAP, int BM, int BN, int WM, int WN>
hipError_t launch_tile(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_tile<FMT, SCAL, SWAP, BM, BN, WM, WN>), grid, dim3(64 * WM * WN), 0, s,
                       a);
    return hipGetLastError();
}

#define QLIN_TILE_INSTANCE(FMT, SCAL, BIT, SW, BM, BN, WM, WN)                                \
    {{QLIN_KERNEL_TILE, SW, BM, BN, 128, WM, WN, 2, 1, 0}, BIT, FMT, SCAL,                    \
     &launch_tile<FMT, SCAL, (SW) != 0, BM, BN, WM, WN>}

// (BM, BN, WM, WN) shapes shared by the formats.
#define QLIN_TILE_SHAPES(X, FMT, SCAL, BIT, SW) \
    X(FMT, SCAL, BIT, SW, 64, 128, 1, 4),       \
    X(FMT, SCAL, BIT, SW, 128, 128, 2, 2),      \
    X(FMT, SCAL, BIT, SW, 128, 256, 2, 2),      \
    X(FMT, SCAL, BIT, SW, 256, 128, 2, 2)

}  // namespace qlin
