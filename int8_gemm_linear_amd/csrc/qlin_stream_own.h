// Wide-row form of the STREAM_LDS family (tile_k = 256): one workgroup per
// CU holds up to TR = 128 or 256 weight rows and every token row of its tile
// (16-32 tokens).
//
// Why: at 16-32 tokens each workgroup of the LDS ring copies its token rows
// once per K range, so the token bytes a CU copies per weight byte are
// TMS / TR.  With (K, N) = (5120, 51200) and spread placement a CU's share
// is 200 weight rows; holding them all in one workgroup copies the token
// rows once per CU instead of two or more times, and leaves no CU idle
// (a 128 x 256 matrix-core tile gives 200 workgroups for 256 CUs).
//
// Chunks are 256 bytes of K (two 128-byte steps), so a stage of 256 weight
// rows and 32 token rows is 72 KB and two stages fit the 160 KB LDS.  Each
// copy instruction brings 4 rows x 256 bytes (lane i: row i / 16, 16-byte
// slot i % 16); the XOR swizzle of the ring (slot s of row r holds piece
// s ^ (r & 15)) is applied on the global side as in the LDS ring.
//
// With two K steps per chunk, splitting steps over the waves (as the LDS
// ring does) would leave most waves idle and need a cross-wave combine of
// TR x TMS partial sums.  Here each wave owns whole 16-row blocks instead
// (block rb belongs to wave rb % NW) for every K step, reads the token
// fragments itself, and stores its own outputs: no partial sums cross waves.
//
// Swap-AB only (weights on the matrix-core rows, tokens on the N side, each
// lane storing four consecutive output columns), as in the "Kernel
// Implementation" section of "Building a High-Performance and Portable vLLM
// Linear Backend with Helion".  Split-K, Block_FP8 group promotion and the
// chunk-carried group scales follow the LDS ring (qlin_stream_lds.h); a
// workgroup's rows (at most TR, starting at a multiple of 8) touch at most
// NBW = (TR + 119) / 128 + 1 weight-block rows of sB.
#pragma once

#include "qlin_stream_lds.h"

namespace qlin {

template <int FMT, int SCAL, int TMS, int TR, int NW, int S>
__global__ void __launch_bounds__(64 * NW)
k_stream_own(KArgs p_)
{
    typedef typename AccT<FMT>::v4 A4;
    typedef typename AccT<FMT>::scalar AS;
    constexpr int CHK = 256;
    constexpr int RPI = 4;                           // rows per copy instruction
    constexpr int TB = (TMS + 15) / 16;              // 16-token blocks
    constexpr int RB = TR / 16;                      // 16-row weight blocks
    constexpr int RBW = (RB + NW - 1) / NW;          // weight blocks per wave
    constexpr int ROWS0 = TR + TMS;
    constexpr int INSTR = ((ROWS0 + RPI * NW - 1) / (RPI * NW)) * NW;   // padded
    constexpr int ROWB = INSTR * RPI * CHK;
    constexpr int L0 = INSTR / NW;                   // row copies per wave per chunk
    constexpr bool BLK = SCAL == SC_BLOCK;
    constexpr int GPC = CHK / 128;                   // K groups per chunk
    constexpr int NBW = (TR + 119) / 128 + 1;        // weight-block rows a workgroup touches
    constexpr int SDW = BLK ? TMS * GPC + NBW * GPC : 0;
    constexpr int LS = BLK ? (SDW + 64 * NW - 1) / (64 * NW) : 0;
    constexpr int STAGE = ROWB + LS * NW * 256;
    constexpr int L = L0 + LS;
    static_assert(TR % 16 == 0 && RB >= NW, "every wave owns a weight block");
    static_assert(TMS >= 1 && TMS <= 32, "tokens per tile");
    static_assert(S >= 2 && S <= 8 && L * (S - 1) <= 63, "ring");
    static_assert(S * STAGE <= 160 * 1024, "LDS per workgroup");
    static_assert(!BLK || FMT == FMT_E4M3, "block scaling is e4m3 only");

    __shared__ __attribute__((aligned(16))) uint8_t lds[S * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;

    KArgs p = p_;
    if (p.group_off && !enter_group<SCAL>(p))
        return;
    int n0, nend;
    if (p.nspread) {
        const int u0 = (int)((int64_t)p.nspread * blockIdx.x / gridDim.x);
        const int u1 = (int)((int64_t)p.nspread * (blockIdx.x + 1) / gridDim.x);
        n0 = 8 * u0;
        nend = min(p.N, 8 * u1);
    } else {
        n0 = blockIdx.x * TR;
        nend = min(p.N, n0 + TR);
    }
    const int m0 = blockIdx.y * TMS;
    const int split = split_index(p);
    if (m0 >= p.M)
        return;                 // a group with fewer rows than the grid covers

    // K range of this split in 256-byte units (K % 256 == 0 for this family).
    const int KP = p.K >> 8;
    const int pps = (KP + p.split_k - 1) / p.split_k;
    const int kbeg = min(KP, split * pps) * 256;
    const int kend = min(KP, split * pps + pps) * 256;
    const int nch = (kend - kbeg) / CHK;

    // Per-copy source rows; padding rows and rows past N or M read one cache
    // line (all lanes the same 16 bytes) so every wave issues L copies per
    // chunk and the waits stay exact counts.
    const uint8_t *src[L0];
    unsigned wmask = 0;
#pragma unroll
    for (int i = 0; i < L0; ++i) {
        const int ins = wave + i * NW;
        const int j = ins * RPI + (lane >> 4);                 // stage row
        const int slot = lane & 15;
        const bool isb = j < TR;
        const int row = isb ? n0 + j : m0 + j - TR;
        const bool valid = isb ? row < nend : (j < TR + TMS && row < p.M);
        const uint8_t *base = isb ? p.B + (int64_t)(valid ? row : 0) * p.ldb
                                  : p.A + (int64_t)(valid ? row : 0) * p.lda;
        src[i] = valid ? base + 16 * (slot ^ (j & 15)) : base;
        if (ins * RPI < TR)
            wmask |= 1u << i;                                  // a copy of weight rows
    }
    wmask = __builtin_amdgcn_readfirstlane(wmask);

    // Block scaling: this lane's scale dword for the split's first chunk
    // (chunk c adds c * GPC) and its group in the chunk, or -1 (it then
    // reads a fixed valid scale).  Area layout: [TMS][GPC] of sA, then
    // [NBW][GPC] of sB from weight-block row n0 / 128 on.
    const float *ssrc[LS > 0 ? LS : 1];
    int sgl[LS > 0 ? LS : 1];
    const float *ssafe = BLK ? p.sA + (int64_t)m0 * p.G : nullptr;
    if constexpr (BLK) {
        const int g0 = kbeg >> 7;
#pragma unroll
        for (int i = 0; i < LS; ++i) {
            const int idx = (wave + i * NW) * 64 + lane;
            ssrc[i] = ssafe;
            sgl[i] = -1;
            if (idx < TMS * GPC) {
                const int tok = idx / GPC, gl = idx % GPC;
                if (m0 + tok < p.M) {
                    ssrc[i] = p.sA + (int64_t)(m0 + tok) * p.G + g0 + gl;
                    sgl[i] = gl;
                }
            } else if (idx < SDW) {
                const int b = (idx - TMS * GPC) / GPC, gl = (idx - TMS * GPC) % GPC;
                const int nb = (n0 >> 7) + b;
                if (nb < (p.N >> 7)) {
                    ssrc[i] = p.sB + (int64_t)nb * p.G + g0 + gl;
                    sgl[i] = gl;
                }
            }
        }
    }

    auto issue = [&](int c) {
        const int k0 = kbeg + c * CHK;
        uint8_t *st = lds + (c % S) * STAGE;
#pragma unroll
        for (int i = 0; i < L0; ++i) {
            const int ins = wave + i * NW;
            if ((wmask >> i) & 1u)
                lds_dma16_nt(src[i] + k0, st + ins * 1024);
            else
                lds_dma16(src[i] + k0, st + ins * 1024);
        }
        if constexpr (BLK) {
#pragma unroll
            for (int i = 0; i < LS; ++i)
                lds_dma4(sgl[i] >= 0 ? ssrc[i] + c * GPC : ssafe, st + ROWB + (wave + i * NW) * 256);
        }
    };

    A4 acc[RBW][TB];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            acc[i][tb] = A4{0, 0, 0, 0};

    // Epilogue scales (token/channel), loaded before the first copy so the
    // chunk waits stay exact: sa1[tb] = sA[t], sb4[i] = sB[n .. n+3].
    const bool scaled = !BLK && p.acc_out == nullptr;
    float sa1[TB];
    v4f sb4[RBW];
    if (scaled) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = m0 + tb * 16 + r16;
            sa1[tb] = t < p.M ? p.sA[t] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int n = n0 + (wave + i * NW) * 16 + 4 * g + v;
                sb4[i][v] = n < p.N ? p.sB[n] : 0.f;
            }
    }

    for (int c = 0; c < S && c < nch; ++c)
        issue(c);

    // Token row of the stage a fragment lane reads (rows past TMS alias the
    // first token row: their outputs are never stored).
    int arow[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
        arow[tb] = TR + (tb * 16 + r16 < TMS ? tb * 16 + r16 : 0);
    int sa_at[TB], sb_at[RBW];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
        sa_at[tb] = (tb * 16 + r16 < TMS ? tb * 16 + r16 : 0) * GPC;
#pragma unroll
    for (int i = 0; i < RBW; ++i)
        sb_at[i] = TMS * GPC + (((n0 + (wave + i * NW) * 16 + 4 * g) >> 7) - (n0 >> 7)) * GPC;

    for (int c = 0; c < nch; ++c) {
        wait_chunks<L, S - 1>(nch - 1 - c);           // chunks issued after c stay in flight
        __syncthreads();
        const uint8_t *st = lds + (c % S) * STAGE;
#pragma unroll
        for (int s = 0; s < CHK / 128; ++s) {
            v4i af[TB][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int piece = s * 8 + h * 4 + g;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    af[tb][h] = *reinterpret_cast<const v4i *>(st + arow[tb] * CHK +
                                                                16 * (piece ^ (arow[tb] & 15)));
            }
            float fa[TB];
            if constexpr (BLK) {
                const float *sc = reinterpret_cast<const float *>(st + ROWB);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    fa[tb] = sc[sa_at[tb] + s];
            }
#pragma unroll
            for (int i = 0; i < RBW; ++i) {
                const int rb = wave + i * NW;
                if (RB % NW != 0 && rb >= RB)
                    continue;                          // wave-uniform
                const int wr = rb * 16 + r16;
                v4i bf[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int piece = s * 8 + h * 4 + g;
                    bf[h] = *reinterpret_cast<const v4i *>(st + wr * CHK + 16 * (piece ^ r16));
                }
                if constexpr (BLK) {
                    // one K group: product on the matrix cores, then promoted
                    const float *sc = reinterpret_cast<const float *>(st + ROWB);
                    const float fb = sc[sb_at[i] + s];
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        const A4 pr = mma16<FMT>(bf[0], bf[1], af[tb][0], af[tb][1], A4{0, 0, 0, 0});
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[i][tb][v] += pr[v] * (fa[tb] * fb);
                    }
                } else {
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
                        acc[i][tb] = mma16<FMT>(bf[0], bf[1], af[tb][0], af[tb][1], acc[i][tb]);
                }
            }
        }
        if (c + S < nch) {
            __syncthreads();                     // every wave is done with stage c % S
            issue(c + S);
        }
    }

    // Lane outputs: n = n0 + 16*rb + 4*g + v (rb = wave + i*NW), t = m0 + 16*tb + r16.
    const int mend = min(p.M, m0 + TMS);
    auto emit = [&](const A4 (&val)[RBW][TB]) {
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
            const int rb = wave + i * NW;
            if (RB % NW != 0 && rb >= RB)
                continue;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int t = m0 + tb * 16 + r16;
                const int n = n0 + rb * 16 + 4 * g;
                if (t >= mend || n >= nend)
                    continue;
                if (!scaled) {
                    if (n + 3 < nend) {
                        store_final4<FMT, SCAL>(p, t, n, val[i][tb]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (n + v < nend)
                                store_final<FMT, SCAL>(p, t, n + v, val[i][tb][v]);
                    }
                } else if (n + 3 < nend) {
                    store_final4_pre<FMT, SC_TC>(p, t, n, val[i][tb], sa1[tb], sb4[i]);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (n + v < nend)
                            p.Y[(int64_t)t * p.ldy + n + v] =
                                bf16_bits(((float)val[i][tb][v] * sa1[tb]) * sb4[i][v]);
                }
            }
        }
    };

    if (p.split_k == 1) {
        emit(acc);
        return;
    }

    // Split-K: every wave writes the partials of its own outputs.
    const bool la = p.reduce == QLIN_REDUCE_LAST_ARRIVER;
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int rb = wave + i * NW;
        if (RB % NW != 0 && rb >= RB)
            continue;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = m0 + tb * 16 + r16;
                const int n = n0 + rb * 16 + 4 * g + v;
                if (t < mend && n < nend) {
                    AS *d = part_ptr<FMT>(p, split, t, n);
                    if (la)
                        st_dev(d, (AS)acc[i][tb][v]);
                    else
                        *d = acc[i][tb][v];
                }
            }
    }
    if (!la)
        return;
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    // the flag lives in the ring, which every wave has left (the barrier
    // inside arrive_last follows each wave's last fragment read)
    if (!arrive_last(p.counters + tile, p.split_k, reinterpret_cast<int *>(lds)))
        return;
    A4 sum[RBW][TB];
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
        const int rb = wave + i * NW;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            sum[i][tb] = A4{0, 0, 0, 0};
            if (RB % NW != 0 && rb >= RB)
                continue;
            for (int s = 0; s < p.split_k; ++s)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = m0 + tb * 16 + r16;
                    const int n = n0 + rb * 16 + 4 * g + v;
                    if (t < mend && n < nend)
                        sum[i][tb][v] += ld_dev(part_ptr<FMT>(p, s, t, n));
                }
        }
    }
    emit(sum);
    rearm(p.counters + tile);
}

template <int FMT, int SCAL, int TMS, int TR, int NW, int S>
hipError_t launch_stream_own(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_stream_own<FMT, SCAL, TMS, TR, NW, S>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// Registered as LDS-ring instances (kernel kind STREAM_LDS, Swap-AB) with
// tile_k = 256, the chunk size that identifies this form; the registry adds
// the spread-placement twin (waves_n = 2) as for every LDS-ring instance.
#define QLIN_STREAM_OWN_INSTANCE(FMT, BIT, SCALV, TMS, TR, NW, S)                     \
    {{QLIN_KERNEL_STREAM_LDS, 1, TMS, TR, 256, 1, NW, S, 1, 0}, BIT, FMT, SCALV, \
     &launch_stream_own<FMT, SCALV, TMS, TR, NW, S>}

#define QLIN_STREAM_OWN_SHAPES(FMT, BIT, SCALV)                \
    QLIN_STREAM_OWN_INSTANCE(FMT, BIT, SCALV, 16, 256, 8, 2),  \
    QLIN_STREAM_OWN_INSTANCE(FMT, BIT, SCALV, 32, 256, 8, 2),  \
    QLIN_STREAM_OWN_INSTANCE(FMT, BIT, SCALV, 16, 128, 8, 3),  \
    QLIN_STREAM_OWN_INSTANCE(FMT, BIT, SCALV, 32, 128, 8, 3)

}  // namespace qlin
