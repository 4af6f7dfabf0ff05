// The STREAM_TOK kernel family: decode (8-32 tokens), persistent
// workgroups with the token rows stationary in LDS.
//
// Why: a CU keeps only so many 128-byte line requests in flight (about 80
// measured, whichever path issues them: register loads or copies into LDS),
// so at decode a GEMM's time is its line requests per CU times the memory
// latency over that capacity.  A workgroup that copies its token rows again
// for every weight tile spends a share of those requests on bytes it already
// had: at 16-32 tokens and 48-128 weight rows per tile, 15-80% on top of the
// weight requests.  Here one workgroup runs per CU for the whole launch: it
// copies the token rows of its K range into LDS once, then streams all of
// its weight rows through a ring that holds weight rows only.
//
// Workgroup: NW waves; a tile is NW blocks of 16 weight rows, one block per
// wave (the wave reads its block's weight fragment and every token fragment
// of the chunk from LDS, so no partial sums cross waves).  The workgroup's
// rows are an even share of the 16-row blocks (grid.x workgroups per token
// tile and split), at most kTokTiles tiles, whose accumulators stay in
// registers until every copy has landed; the stores come last, so every
// wait inside the loop is an exact count of copies.  K ranges: split-K with
// the two-pass reduction when a split's token rows would not fit the LDS
// area kTokLds (TMS * K-range bytes).
//
// LDS: [TMS token rows][KS bytes of the split] then S stages of [16 * NW
// weight rows][CHK].  Both areas keep the 16-byte piece p of row r in slot
// p ^ (r & 15) within its 256-byte group, so a fragment read (16 lanes, 16
// consecutive rows, one piece) touches 16 distinct bank groups; the swizzle
// is applied on the global side of the copies.  The token rows are copied as
// 1 KB instructions over the flattened [TMS][KS] area (instructions past its
// end repeat the first one: the same bytes to the same place).
//
// Variants and split-K as in the "Kernel Implementation" section of
// "Building a High-Performance and Portable vLLM Linear Backend with Helion"
// (built in the Swap-AB orientation only: weights on the matrix-core rows,
// tokens on its columns, four consecutive outputs per lane); token/channel
// scaling (FP8_Dynamic, W8A8_INT8; section "Helion Linear Backend / Scope").
#pragma once

#include "qlin_stream_lds.h"

namespace qlin {

constexpr int kTokLds = 80 * 1024;   // token area of a workgroup (bytes)
constexpr int kTokTiles = 4;         // weight tiles per workgroup at most

template <int FMT, int TMS, int NW, int CHK, int S>
__global__ void __launch_bounds__(64 * NW)
k_stream_tok(KArgs p)
{
    typedef typename AccT<FMT>::v4 A4;
    typedef typename AccT<FMT>::scalar AS;
    constexpr int TB = (TMS + 15) / 16;
    constexpr int TR = 16 * NW;                 // weight rows of a tile
    constexpr int RPI = 1024 / CHK;             // rows per copy instruction
    constexpr int LPR = CHK / 16;               // lanes per row of an instruction
    constexpr int L = TR / RPI / NW;            // weight copies per wave per chunk
    constexpr int STAGE = TR * CHK;
    constexpr int KSMAX = kTokLds / TMS;
    constexpr int TL = (kTokLds / 1024 + NW - 1) / NW;   // token copies per wave
    constexpr int MT = kTokTiles;
    static_assert(CHK == 256 || CHK == 512 || CHK == 1024, "chunk");
    static_assert(TMS == 8 || TMS == 16 || TMS == 32, "tokens per tile");
    static_assert((TR / RPI) % NW == 0, "copies split evenly over the waves");
    static_assert(kTokLds + S * STAGE <= 160 * 1024, "LDS per workgroup");
    static_assert(S >= 2 && TL + S * L <= 63 && L * (S - 1) <= 63, "vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t lds[kTokLds + S * STAGE];
    uint8_t *const tok = lds;
    uint8_t *const ring = lds + kTokLds;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;

    const int m0 = blockIdx.y * TMS;
    if (m0 >= p.M)
        return;
    const int split = blockIdx.z;
    const int mend = min(p.M, m0 + TMS);

    // K range of this split (256-byte units), KS bytes.
    const int KP = p.K >> 8;
    const int pps = (KP + p.split_k - 1) / p.split_k;
    const int kbeg = min(KP, split * pps) * 256;
    const int KS = min(KP, split * pps + pps) * 256 - kbeg;
    // 16-row blocks b0 .. b1-1 of the workgroup, in tiles of NW blocks.
    const int nblk = (p.N + 15) >> 4;
    const int b0 = (int)((int64_t)nblk * blockIdx.x / gridDim.x);
    const int b1 = (int)((int64_t)nblk * (blockIdx.x + 1) / gridDim.x);
    const int ntile = (b1 - b0 + NW - 1) / NW;
    if (ntile == 0 || ntile > MT || KS > KSMAX)
        return;                 // no rows; or a shape the host rejects
    const int nch = (KS + CHK - 1) / CHK;
    const int nq = ntile * nch;                 // chunks of the workgroup, tile-major
    const int nend = min(p.N, 16 * b1);         // rows past nend belong to others

    A4 acc[MT][TB];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            acc[t][tb] = A4{0, 0, 0, 0};

    if (nq > 0) {
        // Token rows of the split, once: instruction j covers LDS bytes
        // [1024 j, 1024 j + 1024) of [TMS][KS]; token rows past M repeat the
        // last one (they feed only outputs that are never stored).
        const int ntok = TMS * KS / 1024;
#pragma unroll
        for (int i = 0; i < TL; ++i) {
            int j = wave + i * NW;
            if (j >= ntok)
                j = 0;
            const int o = j * 1024 + 16 * lane;
            const int t = o / KS;
            const int ks = o - t * KS;
            const int row = min(m0 + t, p.M - 1);
            lds_dma16(p.A + (int64_t)row * p.lda + kbeg + 16 * ((ks >> 4) ^ (t & 15)), tok + j * 1024);
        }

        // Weight copies of chunk q (tile q / nch, chunk q % nch) into stage
        // q % S; rows past nend read one valid cache line instead.
        const int slot = lane % LPR;
        auto issue = [&](int q) {
            const int T = q / nch;
            const int c = q - T * nch;
            uint8_t *st = ring + (q % S) * STAGE;
            const int64_t koff = kbeg + c * CHK;
            const int len = min(CHK, KS - c * CHK);     // >= 256: lanes 0..15 of a row always copy
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const int ins = wave + i * NW;
                const int j = ins * RPI + lane / LPR;                   // stage row
                const int n = 16 * b0 + T * TR + j;
                const uint8_t *src = n < nend
                                         ? p.B + (int64_t)n * p.ldb + koff + 16 * (slot ^ (j & 15))
                                         : p.B + (int64_t)(nend - 1) * p.ldb + koff;
                if (slot * 16 < len)
                    lds_dma16_nt(src, st + ins * 1024);
            }
        };
        for (int q = 0; q < S && q < nq; ++q)
            issue(q);

        // token row of each fragment lane (rows past TMS alias the last one)
        int trow[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            trow[tb] = min(tb * 16 + r16, TMS - 1);

#pragma unroll
        for (int T = 0; T < MT; ++T) {
            if (T >= ntile)
                break;
            const bool mine = b0 + T * NW + wave < b1;     // this wave's block exists
            for (int c = 0; c < nch; ++c) {
                const int q = T * nch + c;
                wait_chunks<L, S - 1>(nq - 1 - q);        // chunks issued after q stay in flight
                __syncthreads();
                if (mine) {
                    const uint8_t *st = ring + (q % S) * STAGE;
                    const int steps = min(CHK, KS - c * CHK) >> 7;
                    const int wr = 16 * wave + r16;
                    for (int s = 0; s < steps; ++s) {
                        v4i bf[2], af[TB][2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int piece = s * 8 + h * 4 + g;
                            bf[h] = *reinterpret_cast<const v4i *>(st + wr * CHK + 16 * (piece ^ (wr & 15)));
                            const int tp = (c * CHK >> 4) + piece;   // piece within the split's K
#pragma unroll
                            for (int tb = 0; tb < TB; ++tb)
                                af[tb][h] = *reinterpret_cast<const v4i *>(
                                    tok + trow[tb] * KS + 16 * (tp ^ (trow[tb] & 15)));
                        }
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb)
                            acc[T][tb] = mma16<FMT>(bf[0], bf[1], af[tb][0], af[tb][1], acc[T][tb]);
                    }
                }
                if (q + S < nq) {
                    __syncthreads();                      // every wave is done with stage q % S
                    issue(q + S);
                }
            }
        }
    }

    // Every copy has landed (the last wait counted none in flight): store.
    // Lane: rows n = 16 * block + 4 * g + v, token t = m0 + 16 * tb + r16.
    const bool scaled = p.acc_out == nullptr;
#pragma unroll
    for (int T = 0; T < MT; ++T) {
        if (T >= ntile)
            break;
        const int blk = b0 + T * NW + wave;
        if (blk >= b1)
            continue;
        const int n = 16 * blk + 4 * g;
        if (n >= nend)
            continue;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = m0 + tb * 16 + r16;
            if (t >= mend)
                continue;
            if (p.split_k > 1) {
                AS *d = part_ptr<FMT>(p, split, t, n);
                if (n + 3 < nend && (p.N & 3) == 0) {
                    *reinterpret_cast<A4 *>(d) = acc[T][tb];
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (n + v < nend)
                            d[v] = acc[T][tb][v];
                }
            } else if (!scaled) {
                if (n + 3 < nend) {
                    store_final4<FMT, SC_TC>(p, t, n, acc[T][tb]);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (n + v < nend)
                            store_final<FMT, SC_TC>(p, t, n + v, acc[T][tb][v]);
                }
            } else if (n + 3 < nend) {
                const v4f sb = v4f{p.sB[n], p.sB[n + 1], p.sB[n + 2], p.sB[n + 3]};
                store_final4_pre<FMT, SC_TC>(p, t, n, acc[T][tb], p.sA[t], sb);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (n + v < nend)
                        p.Y[(int64_t)t * p.ldy + n + v] =
                            bf16_bits(((float)acc[T][tb][v] * p.sA[t]) * p.sB[n + v]);
            }
        }
    }
}

template <int FMT, int TMS, int NW, int CHK, int S>
hipError_t launch_stream_tok(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_stream_tok<FMT, TMS, NW, CHK, S>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// tile_m = tokens held, tile_n = weight rows of a tile (16 per wave), tile_k =
// chunk bytes, waves_k = waves, stages = ring depth; Swap-AB only.
#define QLIN_STREAM_TOK_INSTANCE(FMT, BIT, TMS, NW, CHK, S)                            \
    {{QLIN_KERNEL_STREAM_TOK, QLIN_SWAP_AB, TMS, 16 * (NW), CHK, 1, NW, S, 1, 0}, BIT, FMT, \
     SC_TC, &launch_stream_tok<FMT, TMS, NW, CHK, S>}

#define QLIN_STREAM_TOK_SHAPES(X, FMT, BIT) \
    X(FMT, BIT, 8, 8, 256, 2),              \
    X(FMT, BIT, 8, 4, 512, 2),              \
    X(FMT, BIT, 16, 8, 256, 2),             \
    X(FMT, BIT, 16, 4, 512, 2),             \
    X(FMT, BIT, 32, 8, 256, 2),             \
    X(FMT, BIT, 32, 4, 512, 2)

}  // namespace qlin
