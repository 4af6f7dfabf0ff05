// The TILE kernel family: larger token counts (prefill), where the GEMM is
// bound by the matrix cores and operand reuse through LDS pays.
//
// One workgroup computes a BM (tokens) x BN (weights) output tile of one K
// split with WM x WN waves, each owning a (BM/WM) x (BN/WN) sub-tile of
// 32x32 matrix-core blocks (accumulators live in the AGPR half of the
// register file).  Per 128-byte K step both operand tiles are copied
// HBM/L2 -> LDS with global_load_lds_dwordx4 (16 bytes per lane written
// straight into LDS, no register staging) into a ring of S stages: while
// step s is read from LDS (ds_read_b128) into the matrix cores, steps
// s+1 .. s+S-1 are in flight.  Every global load inside the loop is one of
// these copies (L per wave per step), so the wait for step s is an exact
// s_waitcnt vmcnt(L * steps issued after s), and one barrier per step both
// publishes step s and frees the stage step s+S-1 is copied into.  Within a
// step the wave loads its B fragments once and the A fragments one 32-row
// block at a time, issuing the MFMA pieces across the independent B blocks
// so consecutive matrix-core instructions do not wait on each other.
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
// token scale per block and one weight-block scale per wave).  A step's
// group scales travel with its stage: global_load_lds_dword copies (4 bytes
// per lane) of sA[m0 .. m0+BM-1][g] and sB[n0/128 .. (n0+BN-1)/128][g] into
// an area after the stage's rows, counted in the same exact waits.
#pragma once

#include "qlin_device.h"

namespace qlin {

__device__ inline int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int N>
__device__ inline void wait_vm_tile()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    if constexpr (N == 0)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(L * min(n, NMAX)) for a run-time n >= 0: wait until at
// most n steps' copies (L per step) are still in flight.
template <int L, int NMAX>
__device__ inline void wait_steps(int n)
{
    if constexpr (NMAX > 0) {
        if (n >= NMAX) {
            wait_vm_tile<L * NMAX>();
            return;
        }
        wait_steps<L, NMAX - 1>(n);
    } else {
        wait_vm_tile<0>();
    }
}

// One MFMA piece of a 128-byte K step on a 32x32 block: int8 has four
// pieces of 16 bytes (v_mfma_i32_32x32x32_i8), e4m3 two pieces of 32 bytes
// (v_mfma_f32_32x32x64_f8f6f4).  Same operand layout as mma32.
template <int FMT> struct Pieces;
template <> struct Pieces<FMT_INT8> { static constexpr int n = 4; };
template <> struct Pieces<FMT_E4M3> { static constexpr int n = 2; };

template <int FMT>
__device__ inline typename AccT<FMT>::v16 mma32_piece(const v4i *a, const v4i *b, int j,
                                                      typename AccT<FMT>::v16 c);
template <>
__device__ inline v16i mma32_piece<FMT_INT8>(const v4i *a, const v4i *b, int j, v16i c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[j], c, 0, 0, 0);
}
template <>
__device__ inline v16f mma32_piece<FMT_E4M3>(const v4i *a, const v4i *b, int j, v16f c)
{
    v8i x = __builtin_shufflevector(a[2 * j], a[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    v8i y = __builtin_shufflevector(b[2 * j], b[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
}

// XCD-aware tile id -> origin (m0, n0) of the workgroup's output tile.
// Consecutive workgroup ids land on different XCDs (round-robin over 8), so
// ids are remapped to give every XCD a contiguous range of tiles, walked in
// groups of GM token tiles so that the tiles an XCD runs together share A
// rows and B rows in its own L2.
template <int BM, int BN>
__device__ inline void tile_origin(const KArgs &p, int &m0, int &n0)
{
    constexpr int GM = 4;
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
    m0 = (first_m + in_grp % gsize) * BM;
    n0 = (in_grp / gsize) * BN;
}

// A grouped call sizes grid.x for the largest group: workgroups past the
// tiles of their own (smaller) group have nothing to do.
template <int BM, int BN>
__device__ inline bool tile_in_group(const KArgs &p)
{
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    return (int)blockIdx.x < tiles;
}

// Epilogue of a tile: the wave's FM x FN accumulator blocks of 32x32 are
// either scaled, rounded and stored (no split), or written as split-K
// partials; with the last-arriver reduction the last workgroup of the tile
// sums the partials in split order and stores the result.
// Always inlined: an out-of-line call (it has two callers per tile shape,
// the kernel's two copy forms) saves the live accumulators to scratch.
template <int FMT, int SCAL, bool SWAP, int BM, int BN, int WM, int WN>
__device__ inline __attribute__((always_inline)) void tile_finish(const KArgs &p,
                                   typename AccT<FMT>::v16 (&acc)[BM / WM / 32][BN / WN / 32],
                                   int m0, int n0, int wm, int wn, int lane, uint8_t *lds)
{
    typedef typename AccT<FMT>::v16 A16;
    typedef typename AccT<FMT>::scalar AS;
    constexpr int WTM = BM / WM;
    constexpr int WTN = BN / WN;
    constexpr int FM = WTM / 32;
    constexpr int FN = WTN / 32;
    const int fr = lane & 31;
    const int fh = lane >> 5;
    const int split = split_index(p);

    // Output positions of acc[fm][fn][v] for this lane:
    //   SWAP:     t = tok0 + fr,  n = wgt0 + 8*(v/4) + 4*fh + v%4  (4 consecutive n per v/4)
    //   standard: t = tok0 + 8*(v/4) + 4*fh + v%4,  n = wgt0 + fr
    // with tok0 = m0 + wm*WTM + 32*fm and wgt0 = n0 + wn*WTN + 32*fn.
    //
    // The scales are gathered into registers before any output store: the
    // compiler must assume Y may alias sA/sB, so loads interleaved with the
    // stores would each wait a full memory latency.
    const bool scaled = SCAL == SC_TC && !(FMT == FMT_INT8 && p.acc_out);
    auto emit = [&](const A16 (&val)[FM][FN]) {
        if (SWAP) {
            float sa_r[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int t = m0 + wm * WTM + 32 * fm + fr;
                sa_r[fm] = scaled && t < p.M ? p.sA[t] : 0.f;
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int wgt0 = n0 + wn * WTN + 32 * fn;
                v4f sb_r[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = wgt0 + 8 * q + 4 * fh;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        sb_r[q][j] = scaled && n + j < p.N ? p.sB[n + j] : 0.f;
                }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int t = m0 + wm * WTM + 32 * fm + fr;
                    if (t >= p.M)
                        continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = wgt0 + 8 * q + 4 * fh;
                        typename AccT<FMT>::v4 v4v;
#pragma unroll
                        for (int j = 0; j < 4; ++j) v4v[j] = val[fm][fn][4 * q + j];
                        if (scaled && n + 3 < p.N) {
                            store_final4_pre<FMT, SCAL>(p, t, n, v4v, sa_r[fm], sb_r[q]);
                        } else if (n + 3 < p.N) {
                            store_final4<FMT, SCAL>(p, t, n, v4v);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                if (n + j < p.N)
                                    store_final<FMT, SCAL>(p, t, n + j, v4v[j]);
                        }
                    }
                }
            }
        } else {
            v4f sa_r[FM][4];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = m0 + wm * WTM + 32 * fm + 8 * q + 4 * fh + j;
                        sa_r[fm][q][j] = scaled && t < p.M ? p.sA[t] : 0.f;
                    }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + wn * WTN + 32 * fn + fr;
                if (n >= p.N)
                    continue;
                const float sb = scaled ? p.sB[n] : 0.f;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int tok0 = m0 + wm * WTM + 32 * fm;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int t = tok0 + 8 * (v >> 2) + 4 * fh + (v & 3);
                        if (t >= p.M)
                            continue;
                        if (scaled)
                            p.Y[(int64_t)t * p.ldy + n] =
                                bf16_bits(((float)val[fm][fn][v] * sa_r[fm][v >> 2][v & 3]) * sb);
                        else
                            store_final<FMT, SCAL>(p, t, n, val[fm][fn][v]);
                    }
                }
            }
        }
    };

    // Staged bf16 store: the workgroup's BM x BN output tile is assembled in
    // LDS (the pipeline ring, free once every wave has left the main loop)
    // and written back as whole 16-byte pieces of contiguous rows, so every
    // store instruction covers full 128-byte lines of Y instead of 32 rows x
    // 16 bytes.  Row stride BN*2 bytes; the CPR 16-byte chunks of a row are
    // permuted by the row index against LDS bank conflicts: XOR-swizzled when
    // CPR is a power of two, else rotated by the row index.
    constexpr int CPR = BN / 8;                       // 16-byte chunks per row
    constexpr bool CPR2 = (CPR & (CPR - 1)) == 0;
    constexpr int NT = 64 * WM * WN;
    auto stage_off = [&](int r, int c) {
        return r * (BN * 2) + 16 * (CPR2 ? (c ^ (r & (CPR - 1))) : (c + r) % CPR);
    };
    auto emit_staged = [&](const A16 (&val)[FM][FN]) {
        __syncthreads();                               // every wave is done with the ring
        if (SWAP) {
            float sa_r[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int t = m0 + wm * WTM + 32 * fm + fr;
                sa_r[fm] = scaled && t < p.M ? p.sA[t] : 1.f;
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int nl0 = wn * WTN + 32 * fn;           // tile-local column of the block
                v4f sb_r[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int n = n0 + nl0 + 8 * q + 4 * fh + j;
                        sb_r[q][j] = scaled && n < p.N ? p.sB[n] : 1.f;
                    }
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int r = wm * WTM + 32 * fm + fr;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint16_t h[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float x = (float)val[fm][fn][4 * q + j];
                            h[j] = bf16_bits(scaled ? (x * sa_r[fm]) * sb_r[q][j] : x);
                        }
                        uint2 w;
                        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                        *reinterpret_cast<uint2 *>(lds + stage_off(r, (nl0 >> 3) + q) + 8 * fh) = w;
                    }
                }
            }
        } else {
            v4f sa_r[FM][4];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int t = m0 + wm * WTM + 32 * fm + 8 * q + 4 * fh + j;
                        sa_r[fm][q][j] = scaled && t < p.M ? p.sA[t] : 1.f;
                    }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int nl = wn * WTN + 32 * fn + fr;
                const float sb = scaled && n0 + nl < p.N ? p.sB[n0 + nl] : 1.f;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int r = wm * WTM + 32 * fm + 8 * (v >> 2) + 4 * fh + (v & 3);
                        const float x = (float)val[fm][fn][v];
                        *reinterpret_cast<uint16_t *>(lds + stage_off(r, nl >> 3) + 2 * (nl & 7)) =
                            bf16_bits(scaled ? (x * sa_r[fm][v >> 2][v & 3]) * sb : x);
                    }
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int k = threadIdx.x; k < BM * CPR; k += NT) {
            const int r = k / CPR;
            const int c = k % CPR;
            const int t = m0 + r;
            const int n = n0 + 8 * c;
            if (t >= p.M || n >= p.N)
                continue;
            const v4i d = *reinterpret_cast<const v4i *>(lds + stage_off(r, c));
            uint16_t *y = p.Y + (int64_t)t * p.ldy + n;
            if (n + 8 <= p.N) {
                *reinterpret_cast<v4i *>(y) = d;
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (n + j < p.N)
                        y[j] = (uint16_t)((uint32_t)d[j >> 1] >> (16 * (j & 1)));
            }
        }
    };

    if (p.split_k > 1) {
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
        if (!arrive_last(p.counters + blockIdx.x, p.split_k, reinterpret_cast<int *>(lds)))
            return;
        // The last arriver sums every split's partial in split order (its
        // own included), overwriting its accumulators.
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
                    acc[fm][fn][v] = a;
                }
            }
        rearm(p.counters + blockIdx.x);
    }
    if (scaled || SCAL == SC_BLOCK) {
        if ((p.ldy & 7) == 0) {
            emit_staged(acc);
            return;
        }
    }
    emit(acc);
}

// NTB: the launch has one token tile (M <= BM: decode), so every weight
// tile is read by one workgroup and its copies use the non-temporal policy;
// with several token tiles the workgroups of a weight tile share it through
// L2 and the copies keep the default policy.  A template parameter, so the
// prefill form of the copy loop carries no extra branch.
template <int FMT, int SCAL, bool SWAP, int BM, int BN, int WM, int WN, int S, bool NTB>
__global__ void __launch_bounds__(64 * WM * WN)
k_tile(KArgs p_)
{
    typedef typename AccT<FMT>::v16 A16;
    typedef typename AccT<FMT>::scalar AS;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM;       // tokens per wave
    constexpr int WTN = BN / WN;       // weights per wave
    constexpr int FM = WTM / 32;
    constexpr int FN = WTN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int ROWB = ROWS * 128;                  // the stage's operand rows
    // Block scaling: the step's scales after the rows, as dwords [BM] of sA
    // then [BN/128] of sB; LSC dword copies per wave.
    constexpr bool BLK = SCAL == SC_BLOCK;
    constexpr int SDW = BLK ? BM + BN / 128 : 0;
    constexpr int LSC = BLK ? (SDW + 64 * NW - 1) / (64 * NW) : 0;
    constexpr int STAGE = ROWB + LSC * NW * 256;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
    static_assert(ROWS % 8 == 0, "rows");
    static_assert(S >= 2 && S <= 6 && S * STAGE <= 160 * 1024, "stages");
    static_assert(!BLK || (SWAP && BN % 128 == 0), "block scaling: Swap-AB, whole weight blocks");

    __shared__ __attribute__((aligned(16))) uint8_t lds[S * STAGE];

    KArgs p = p_;
    if (p.group_off && !(enter_group<SCAL>(p) && tile_in_group<BM, BN>(p)))
        return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    int m0, n0;
    tile_origin<BM, BN>(p, m0, n0);

    // ---- K range of this split (128-byte steps)
    const int KS = p.K >> 7;
    const int split = split_index(p);
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
    // NTB: bit i set when copy i of this wave brings weight rows (a group is
    // all token or all weight rows: BM is a multiple of 8).  Derived from the
    // wave index through readfirstlane: the choice of copy instruction is a
    // scalar branch and every wave issues exactly one copy per i.
    unsigned ntmask = 0;
    if constexpr (NTB) {
#pragma unroll
        for (int i = 0; i < GPW; ++i)
            if ((wave + i * NW) * 8 >= BM)
                ntmask |= 1u << i;
        ntmask = __builtin_amdgcn_readfirstlane(ntmask);
    }

    static_assert(ROWS / 8 % NW == 0, "copies must split evenly over the waves");
    constexpr int L = GPW + LSC;                      // copies per wave per step
    static_assert(L * (S - 2) <= 63, "vmcnt range");

    // Block scaling: source of this lane's scale dword at step 0 (step st adds
    // st); rows past M and weight blocks past N read the last valid one.
    const float *ssrc[LSC > 0 ? LSC : 1];
    if constexpr (BLK) {
#pragma unroll
        for (int i = 0; i < LSC; ++i) {
            const int idx = (wave + i * NW) * 64 + lane;
            if (idx < BM)
                ssrc[i] = p.sA + (int64_t)min(m0 + idx, p.M - 1) * p.G;
            else
                ssrc[i] = p.sB + (int64_t)min((n0 >> 7) + min(idx - BM, BN / 128 - 1),
                                              (p.N >> 7) - 1) * p.G;
        }
    }

    auto issue = [&](int st, int stage) {
        uint8_t *dst0 = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < GPW; ++i) {
            const int grp_i = wave + i * NW;
            if (GROUPS % NW == 0 || grp_i < GROUPS) {
                if (NTB && ((ntmask >> i) & 1u))
                    lds_dma16_nt(src[i] + (int64_t)st * 128, dst0 + grp_i * 1024);
                else
                    lds_dma16(src[i] + (int64_t)st * 128, dst0 + grp_i * 1024);
            }
        }
        if constexpr (BLK) {
#pragma unroll
            for (int i = 0; i < LSC; ++i)
                lds_dma4(ssrc[i] + st, dst0 + ROWB + (wave + i * NW) * 256);
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

    const int nst = s_end - s_beg;
    for (int i = 0; i < S - 1 && i < nst; ++i)
        issue(s_beg + i, i);
    for (int i = 0; i < nst; ++i) {
        const int s = s_beg + i;
        wait_steps<L, S - 2>(nst - 1 - i);              // steps issued after step i stay in flight
        __syncthreads();
        if (i + S - 1 < nst)
            issue(s + S - 1, (i + S - 1) % S);
        const uint8_t *la = lds + (i % S) * STAGE;
        float sa[FM], sb[FN];
        if constexpr (BLK) {
            const float *sc = reinterpret_cast<const float *>(la + ROWB);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) sa[fm] = sc[wm * WTM + fm * 32 + fr];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                sb[fn] = sc[BM + ((n0 + wn * WTN + fn * 32) >> 7) - (n0 >> 7)];
        }
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
        // A fragments one 32-row block at a time, double-buffered: block fm+1
        // is read from LDS while block fm's MFMA pieces issue (interleaved
        // across the FN independent accumulators).  The scheduling barriers
        // keep the compiler from hoisting every read, which would not fit
        // the register file at 8 waves per workgroup.
        auto load_a = [&](v4i (&af)[4], int fm) {
            const int r = wm * WTM + fm * 32 + fr;
            const uint8_t *rowp = la + r * 128;
            const int sw = lds_swz(r);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                af[j] = *reinterpret_cast<const v4i *>(rowp + 16 * ((4 * fh + j) ^ sw));
        };
        auto block = [&](const v4i (&af)[4], int fm) {
            if constexpr (SCAL == SC_BLOCK) {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    A16 z;
#pragma unroll
                    for (int v = 0; v < 16; ++v) z[v] = 0;
                    A16 pz = SWAP ? mma32<FMT>(bf[fn], af, z) : mma32<FMT>(af, bf[fn], z);
                    const float scale = sa[fm] * sb[fn];
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[fm][fn][v] = __builtin_fmaf((float)pz[v], scale, (float)acc[fm][fn][v]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < Pieces<FMT>::n; ++j)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        acc[fm][fn] = SWAP ? mma32_piece<FMT>(bf[fn], af, j, acc[fm][fn])
                                           : mma32_piece<FMT>(af, bf[fn], j, acc[fm][fn]);
            }
        };
        if constexpr (SCAL == SC_BLOCK && NW >= 8) {
            // Block scaling with 8 waves (256 registers per lane): pipelined
            // one 32x32 block deep, the group product of block k+1 on the
            // matrix cores while the VALU promotes block k, with two product
            // tiles and one A-fragment set live (the A-block-deep pipeline
            // below would hold 2 x FN product tiles and spill); the other
            // wave of the SIMD covers the LDS read of the next A block.
            constexpr int NB = FM * FN;
            A16 pz[2];
            v4i af[4];
            const A16 zero = {};
            load_a(af, 0);
            pz[0] = SWAP ? mma32<FMT>(bf[0], af, zero) : mma32<FMT>(af, bf[0], zero);
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int fm = k / FN;
                const int fn = k % FN;
                if (k + 1 < NB) {
                    const int fm1 = (k + 1) / FN;
                    const int fn1 = (k + 1) % FN;
                    if (fn1 == 0)
                        load_a(af, fm1);
                    pz[(k + 1) & 1] = SWAP ? mma32<FMT>(bf[fn1], af, zero)
                                           : mma32<FMT>(af, bf[fn1], zero);
                }
                const float scale = sa[fm] * sb[fn];
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[fm][fn][v] = __builtin_fmaf((float)pz[k & 1][v], scale, (float)acc[fm][fn][v]);
            }
        } else if constexpr (SCAL == SC_BLOCK) {
            // Block scaling, software-pipelined across the 32-row A blocks:
            // the group products of block fm+1 go to the matrix cores while
            // the VALU promotes block fm's (acc += p * sA * sB), so the two
            // units overlap instead of waiting on each other.
            A16 pz[2][FN];
            v4i af[2][4];
            const A16 zero = {};
            load_a(af[0], 0);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                pz[0][fn] = SWAP ? mma32<FMT>(bf[fn], af[0], zero) : mma32<FMT>(af[0], bf[fn], zero);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int cur = fm & 1;
                if (fm + 1 < FM) {
                    load_a(af[cur ^ 1], fm + 1);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
                        pz[cur ^ 1][fn] = SWAP ? mma32<FMT>(bf[fn], af[cur ^ 1], zero)
                                               : mma32<FMT>(af[cur ^ 1], bf[fn], zero);
                }
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const float scale = sa[fm] * sb[fn];
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        acc[fm][fn][v] = __builtin_fmaf((float)pz[cur][fn][v], scale, (float)acc[fm][fn][v]);
                }
            }
        } else {
        v4i a0[4], a1[4];
        load_a(a0, 0);
#pragma unroll
        for (int fm = 0; fm < FM; fm += 2) {
            if (fm + 1 < FM)
                load_a(a1, fm + 1);
            __builtin_amdgcn_sched_barrier(0);
            block(a0, fm);
            __builtin_amdgcn_sched_barrier(0);
            if (fm + 1 < FM) {
                if (fm + 2 < FM)
                    load_a(a0, fm + 2);
                __builtin_amdgcn_sched_barrier(0);
                block(a1, fm + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        }
    }

    static_assert(BM * BN * 2 <= S * STAGE, "the output tile is staged in the ring");
    tile_finish<FMT, SCAL, SWAP, BM, BN, WM, WN>(p, acc, m0, n0, wm, wn, lane, lds);
}

template <int FMT, int SCAL, bool SWAP, int BM, int BN, int WM, int WN, int S>
hipError_t launch_tile(const KArgs &a, dim3 grid, hipStream_t s)
{
    const dim3 block(64 * WM * WN);
    if (a.M <= BM)
        hipLaunchKernelGGL((k_tile<FMT, SCAL, SWAP, BM, BN, WM, WN, S, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_tile<FMT, SCAL, SWAP, BM, BN, WM, WN, S, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

#define QLIN_TILE_INSTANCE(FMT, SCAL, BIT, SW, BM, BN, WM, WN, S)                             \
    {{QLIN_KERNEL_TILE, SW, BM, BN, 128, WM, WN, S, 1, 0}, BIT, FMT, SCAL,                    \
     &launch_tile<FMT, SCAL, (SW) != 0, BM, BN, WM, WN, S>}

// (BM, BN, WM, WN, S) for token/channel scaling; LDS = S * (BM + BN) * 128 B.
// 256 x 160 gives N = 5120 at M = 2048 exactly 256 tiles (one per CU; a
// 256 x 256 tile leaves 96 CUs idle there).
#define QLIN_TILE_SHAPES(X, FMT, SCAL, BIT, SW) \
    X(FMT, SCAL, BIT, SW, 64, 128, 1, 4, 4),    \
    X(FMT, SCAL, BIT, SW, 64, 128, 2, 4, 4),    \
    X(FMT, SCAL, BIT, SW, 64, 128, 2, 4, 6),    \
    X(FMT, SCAL, BIT, SW, 128, 128, 2, 2, 2),   \
    X(FMT, SCAL, BIT, SW, 128, 128, 2, 2, 4),   \
    X(FMT, SCAL, BIT, SW, 128, 128, 4, 2, 4),   \
    X(FMT, SCAL, BIT, SW, 128, 256, 2, 2, 3),   \
    X(FMT, SCAL, BIT, SW, 256, 128, 2, 2, 3),   \
    X(FMT, SCAL, BIT, SW, 256, 256, 2, 2, 2),   \
    X(FMT, SCAL, BIT, SW, 256, 256, 2, 4, 2),   \
    X(FMT, SCAL, BIT, SW, 256, 256, 4, 2, 2),   \
    X(FMT, SCAL, BIT, SW, 256, 128, 4, 2, 3),   \
    X(FMT, SCAL, BIT, SW, 128, 256, 2, 4, 3),   \
    X(FMT, SCAL, BIT, SW, 256, 160, 4, 1, 3)

// Block scaling (the stage also carries the step's scales, under 2 KB).
#define QLIN_TILE_SHAPES_BLOCK(X, FMT, SCAL, BIT, SW) \
    X(FMT, SCAL, BIT, SW, 64, 128, 1, 4, 2),          \
    X(FMT, SCAL, BIT, SW, 64, 128, 1, 4, 4),          \
    X(FMT, SCAL, BIT, SW, 64, 128, 2, 4, 4),          \
    X(FMT, SCAL, BIT, SW, 64, 128, 2, 4, 5),          \
    X(FMT, SCAL, BIT, SW, 128, 128, 2, 2, 2),         \
    X(FMT, SCAL, BIT, SW, 128, 128, 2, 2, 4),         \
    X(FMT, SCAL, BIT, SW, 128, 128, 4, 2, 2),         \
    X(FMT, SCAL, BIT, SW, 128, 128, 4, 2, 4),         \
    X(FMT, SCAL, BIT, SW, 128, 256, 2, 2, 2),         \
    X(FMT, SCAL, BIT, SW, 256, 128, 2, 2, 2),         \
    X(FMT, SCAL, BIT, SW, 256, 256, 2, 4, 2),         \
    X(FMT, SCAL, BIT, SW, 256, 256, 4, 2, 2),         \
    X(FMT, SCAL, BIT, SW, 256, 128, 4, 2, 2),         \
    X(FMT, SCAL, BIT, SW, 256, 128, 4, 2, 3),         \
    X(FMT, SCAL, BIT, SW, 128, 256, 2, 4, 2),         \
    X(FMT, SCAL, BIT, SW, 128, 256, 2, 4, 3)

}  // namespace qlin
