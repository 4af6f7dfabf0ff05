// The STREAM_LDS kernel family: small token counts (decode), weight tiles
// copied HBM -> LDS in 1 KB row segments.
//
// Why: on MI355X a weight stream read as 1 KB contiguous row segments per
// load instruction runs markedly faster than the matrix-core operand layout
// read straight into registers (16 rows x 64 bytes per instruction), and
// global_load_lds keeps many segments in flight without holding registers.
// The LDS round trip costs nothing that matters here: LDS bandwidth is far
// above a CU's share of HBM bandwidth.
//
// Workgroup: NW waves own TR = 8, 16, 32, 48, 64, 96, 112 or 128 weight rows (the matrix core sees
// blocks of 16; with 8 rows, fragment rows 8..15 repeat rows 0..7 and their
// outputs are dropped, which doubles the workgroup count for small N without
// a split-K reduction) and TMS tokens (1..32; the
// matrix core sees them as TB = ceil(TMS/16) blocks of 16, the rows past TMS
// hold stale data that only feeds outputs never stored) of one K split.  The
// split's K range is cut into chunks of CHK bytes; a chunk stage in LDS holds
// [TR weight rows][CHK], [TMS token rows][CHK] and padding rows.  Each load
// instruction copies 1 KB (CHK = 1024: one row segment; CHK = 512: two rows,
// 512 bytes each) with global_load_lds_dwordx4, so every byte moves HBM/L2 ->
// LDS in contiguous runs; padding instructions read one cache line so every
// wave issues the same count L per chunk.  All S stages are filled up front
// (for decode K this is usually the whole split: one round trip), and stage
// c % S is refilled with chunk c + S after chunk c is consumed.  All global
// loads inside the loop are these copies, so the wait for chunk c is an
// exact s_waitcnt vmcnt(L * chunks issued after c).  Weight rows are copied
// with the non-temporal policy (streamed once), token rows with the default
// one (every workgroup re-reads them from L2).
//
// LDS swizzle: within a row, 16-byte slot s holds the chunk's 16-byte piece
// s ^ (row & 15).  A matrix-core fragment read (16 lanes, 16 consecutive
// rows, the same piece) then touches 16 distinct slot residues, i.e. 16
// distinct bank groups.  The swizzle is applied on the global side (lane i
// fetches piece i ^ (row & 15)), which keeps every instruction inside its
// 1 KB segment, and stays inside a partial chunk because chunk lengths are
// multiples of 256 bytes (K % 256 == 0 for this family).
//
// The waves split each chunk's 128-byte K steps; their partial sums are
// combined in LDS in fixed wave order, then the epilogue (scales, bf16,
// Swap-AB orientation, Split-K partials / last arriver) is the stream
// kernel's.  Variants and split-K as in the "Kernel Implementation" section
// of "Building a High-Performance and Portable vLLM Linear Backend with
// Helion".
//
// Block_FP8 (1x128 activation groups, 128x128 weight blocks, same page,
// section "Helion Linear Backend / Scope"): a 128-byte K step is exactly one
// K group, because chunks start on 256-byte boundaries.  Each step's product
// goes to the matrix cores with a zero accumulator and is then added to the
// running sum times sA[t, g] * sB[n / 128, g].  The chunk's group scales
// travel with the chunk: every wave issues LS more copies per chunk
// (global_load_lds_dword, 4 bytes per lane) that bring sA[m0 .. m0+TMS-1]
// [chunk's groups] and sB[two weight-block rows][chunk's groups] into an
// area after the stage's rows, so the chunk waits stay exact counts.
#pragma once

#include "qlin_device.h"

namespace qlin {

template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    if constexpr (N == 0)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(L * min(n, NMAX)) for a run-time n >= 0: wait until at
// most n chunks' copies (L per chunk) are still in flight.
template <int L, int NMAX>
__device__ inline void wait_chunks(int n)
{
    if constexpr (NMAX > 0) {
        if (n >= NMAX) {
            wait_vm<L * NMAX>();
            return;
        }
        wait_chunks<L, NMAX - 1>(n);
    } else {
        wait_vm<0>();
    }
}

template <int FMT, int SCAL, bool SWAP, int TMS, int TRW, int NW, int S, int CHK>
__global__ void __launch_bounds__(64 * NW)
k_stream_lds(KArgs p_)
{
    typedef typename AccT<FMT>::v4 A4;
    typedef typename AccT<FMT>::scalar AS;
    constexpr int TB = (TMS + 15) / 16;
    constexpr int TR = TRW;                          // weight rows of the workgroup
    constexpr int RB = TR >= 16 ? TR / 16 : 1;       // 16-row matrix-core blocks
    constexpr int RMASK = TR >= 16 ? 15 : TR - 1;    // fragment row within the stage
    static_assert(TR == 8 || TR == 16 || TR == 32 || TR == 48 || TR == 64 || TR == 96 || TR == 112 ||
                      TR == 128,
                  "weight rows");
    constexpr int RPI = 1024 / CHK;                  // rows per load instruction
    constexpr int ROWS0 = TR + TMS;
    constexpr int INSTR = ((ROWS0 + RPI * NW - 1) / (RPI * NW)) * NW;   // padded
    constexpr int ROWS = INSTR * RPI;
    constexpr int ROWB = ROWS * CHK;                 // the stage's rows
    constexpr int L0 = INSTR / NW;                   // row copies per wave per chunk
    // Block scaling: group scales of the chunk after the rows, as dwords
    // [TMS][GPC] of sA then [2][GPC] of sB; LS dword copies per wave.
    constexpr bool BLK = SCAL == SC_BLOCK;
    constexpr int GPC = CHK / 128;                   // K groups per chunk
    constexpr int SDW = BLK ? TMS * GPC + 2 * GPC : 0;
    constexpr int LS = BLK ? (SDW + 64 * NW - 1) / (64 * NW) : 0;
    constexpr int STAGE = ROWB + LS * NW * 256;
    constexpr int L = L0 + LS;                       // copies per wave per chunk
    static_assert(CHK == 512 || CHK == 1024, "chunk");
    static_assert(TMS >= 1 && TMS <= 32, "tokens per tile");
    static_assert(S >= 1 && S <= 8 && L * (S - 1) <= 63, "ring");
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
    // Weight rows of the workgroup: TR rows per workgroup, or (spread
    // placement) 8-row units shared evenly over grid.x, at most TR rows each,
    // so a grid sized to the CU count gives every CU the same number of rows.
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

    // K range of this split, in 256-byte units.
    const int KP = p.K >> 8;
    const int pps = (KP + p.split_k - 1) / p.split_k;
    const int kbeg = min(KP, split * pps) * 256;
    const int kend = min(KP, split * pps + pps) * 256;
    const int nch = (kend - kbeg + CHK - 1) / CHK;

    // Per-instruction source rows.  Padding rows, and rows past the
    // workgroup's weight rows or past M (they feed only outputs that are
    // never stored), still issue their instruction
    // -- keeping the per-wave load count exact for the vmcnt waits -- but all
    // lanes read the same 16 bytes: one cache line instead of a 1 KB segment.
    const uint8_t *src[L0];
    // Bit i: copy i of this wave brings weight rows (all of its rows are
    // weight rows or none are: TR is a multiple of 8).  Derived from the
    // wave index through readfirstlane, so the choice of copy instruction
    // below is a scalar branch and every wave issues exactly one copy per i.
    unsigned wmask = 0;
#pragma unroll
    for (int i = 0; i < L0; ++i) {
        const int ins = wave + i * NW;
        const int j = ins * RPI + (RPI == 2 ? (lane >> 5) : 0);       // stage row
        const int slot = RPI == 2 ? (lane & 31) : lane;
        const bool isb = j < TR;
        const int row = isb ? n0 + j : m0 + j - TR;
        const bool valid = isb ? row < nend : (j < TR + TMS && row < p.M);
        const uint8_t *base = isb ? p.B + (int64_t)(valid ? row : 0) * p.ldb
                                  : p.A + (int64_t)(valid ? row : 0) * p.lda;
        src[i] = valid ? base + 16 * (slot ^ (j & 15)) : base;
        if (ins * RPI < TR)
            wmask |= 1u << i;
    }
    wmask = __builtin_amdgcn_readfirstlane(wmask);

    // Block scaling: per scale copy, the source of this lane's dword for the
    // split's first chunk (chunk c adds c * GPC), its group within the chunk,
    // or -1 for a lane with nothing to fetch (it reads a fixed, valid scale).
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
        const int len = min(CHK, kend - k0);
        uint8_t *st = lds + (c % S) * STAGE;
        const int slot = RPI == 2 ? (lane & 31) : lane;
#pragma unroll
        for (int i = 0; i < L0; ++i) {
            const int ins = wave + i * NW;
            // weight rows: non-temporal (read once per launch); token rows
            // keep the default policy (every workgroup re-reads them from L2)
            if (slot * 16 < len) {
                if ((wmask >> i) & 1u)
                    lds_dma16_nt(src[i] + k0, st + ins * 1024);
                else
                    lds_dma16(src[i] + k0, st + ins * 1024);
            }
        }
        if constexpr (BLK) {
            const int glen = len >> 7;                 // groups in this chunk
#pragma unroll
            for (int i = 0; i < LS; ++i) {
                const bool ok = sgl[i] >= 0 && sgl[i] < glen;
                lds_dma4(ok ? ssrc[i] + c * GPC : ssafe, st + ROWB + (wave + i * NW) * 256);
            }
        }
    };

    A4 acc[RB][TB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            acc[rb][tb] = A4{0, 0, 0, 0};

    // Epilogue scales of this lane's outputs, loaded before the first copy:
    // they complete ahead of every chunk (loads return in issue order), so
    // the chunk waits stay exact and their latency hides under the stream.
    //   SWAP: sa1[tb] = sA[t], sb4[rb] = sB[n..n+3]
    //   standard: sa4[tb] = sA[t..t+3], sb1[rb] = sB[n]
    float sa1[TB], sb1[RB];
    v4f sa4[TB], sb4[RB];
    const bool scaled = !BLK && p.acc_out == nullptr;   // Block_FP8 sums arrive scaled
    if (scaled) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            if (SWAP) {
                const int t = m0 + tb * 16 + r16;
                sa1[tb] = t < p.M ? p.sA[t] : 0.f;
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = m0 + tb * 16 + 4 * g + v;
                    sa4[tb][v] = t < p.M ? p.sA[t] : 0.f;
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (SWAP) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int n = n0 + rb * 16 + 4 * g + v;
                    sb4[rb][v] = n < p.N ? p.sB[n] : 0.f;
                }
            } else {
                const int n = n0 + rb * 16 + r16;
                sb1[rb] = n < p.N ? p.sB[n] : 0.f;
            }
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
    // Block scaling: where this lane's token scales and each 16-row block's
    // weight scales sit in the stage's scale area (dword index of group 0).
    int sa_at[TB][SWAP ? 1 : 4], sb_at[RB];   // sb_at: this lane's weight row(s) of block rb
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int v = 0; v < (SWAP ? 1 : 4); ++v) {
            const int tok = SWAP ? tb * 16 + r16 : tb * 16 + 4 * g + v;
            sa_at[tb][v] = (tok < TMS ? tok : 0) * GPC;
        }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        sb_at[rb] = TMS * GPC + (((n0 + rb * 16 + (SWAP ? 4 * g : r16)) >> 7) - (n0 >> 7)) * GPC;

    for (int c = 0; c < nch; ++c) {
        wait_chunks<L, S - 1>(nch - 1 - c);           // chunks issued after c stay in flight
        __syncthreads();
        const uint8_t *st = lds + (c % S) * STAGE;
        const int steps = min(CHK, kend - (kbeg + c * CHK)) >> 7;
        for (int s = wave; s < steps; s += NW) {
            v4i bf[RB][2], af[TB][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int piece = s * 8 + h * 4 + g;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int wr = rb * 16 + (r16 & RMASK);
                    bf[rb][h] = *reinterpret_cast<const v4i *>(st + wr * CHK +
                                                                16 * (piece ^ (wr & 15)));
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    af[tb][h] = *reinterpret_cast<const v4i *>(st + arow[tb] * CHK +
                                                                16 * (piece ^ (arow[tb] & 15)));
            }
            if constexpr (BLK) {
                // one K group: product on the matrix cores, then promoted
                const float *sc = reinterpret_cast<const float *>(st + ROWB);
                float fb[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    fb[rb] = sc[sb_at[rb] + s];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    v4f fa;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        fa[v] = sc[sa_at[tb][SWAP ? 0 : v] + s];
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const A4 z = A4{0, 0, 0, 0};
                        const A4 pr = SWAP ? mma16<FMT>(bf[rb][0], bf[rb][1], af[tb][0], af[tb][1], z)
                                           : mma16<FMT>(af[tb][0], af[tb][1], bf[rb][0], bf[rb][1], z);
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[rb][tb][v] += pr[v] * (fa[v] * fb[rb]);
                    }
                }
            } else {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
                        acc[rb][tb] = SWAP ? mma16<FMT>(bf[rb][0], bf[rb][1], af[tb][0], af[tb][1], acc[rb][tb])
                                           : mma16<FMT>(af[tb][0], af[tb][1], bf[rb][0], bf[rb][1], acc[rb][tb]);
            }
        }
        if (c + S < nch) {
            __syncthreads();                     // every wave is done with stage c % S
            issue(c + S);
        }
    }

    // Combine the waves' partial sums in fixed order (wave 0 first); the ring
    // is free once every wave has passed this barrier.  Without split-K the
    // combine is spread over the waves (below): wave w sums and stores the
    // accumulator elements e with e % NW == w, so no wave reads all the
    // others' partials in sequence.  Same order of additions either way.
    __syncthreads();
    constexpr int E = RB * TB * 4;                   // accumulator elements per lane
    constexpr bool SPREAD = NW > 1 && NW * E * 64 * 4 <= S * STAGE;
    const bool spread = SPREAD && p.split_k == 1;
    if (NW > 1 && !spread) {
        AS *red = reinterpret_cast<AS *>(lds);      // [NW-1][RB*TB*4][64]
        static_assert((NW - 1) * RB * TB * 4 * 64 * 4 <= S * STAGE, "reduction space");
        if (wave > 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        red[((wave - 1) * RB * TB * 4 + (rb * TB + tb) * 4 + v) * 64 + lane] = acc[rb][tb][v];
        }
        __syncthreads();
        if (wave == 0) {
            for (int w = 1; w < NW; ++w)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[rb][tb][v] += red[((w - 1) * RB * TB * 4 + (rb * TB + tb) * 4 + v) * 64 + lane];
        }
    }

    //   SWAP:     n = n0 + 16*rb + 4*g + v,  t = m0 + 16*tb + r16
    //   standard: n = n0 + 16*rb + r16,      t = m0 + 16*tb + 4*g + v
    const int mend = min(p.M, m0 + TMS);           // tokens of this tile
    auto emit = [&](const A4 (&val)[RB][TB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                if (SWAP) {
                    const int t = m0 + tb * 16 + r16;
                    const int n = n0 + rb * 16 + 4 * g;
                    if (t >= mend || n >= nend)
                        continue;
                    if (!scaled) {
                        if (n + 3 < nend) {
                            store_final4<FMT, SCAL>(p, t, n, val[rb][tb]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 4; ++v)
                                if (n + v < nend)
                                    store_final<FMT, SCAL>(p, t, n + v, val[rb][tb][v]);
                        }
                    } else if (n + 3 < nend) {
                        store_final4_pre<FMT, SC_TC>(p, t, n, val[rb][tb], sa1[tb], sb4[rb]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (n + v < nend)
                                p.Y[(int64_t)t * p.ldy + n + v] =
                                    bf16_bits(((float)val[rb][tb][v] * sa1[tb]) * sb4[rb][v]);
                    }
                } else {
                    const int n = n0 + rb * 16 + r16;
                    if (n >= nend)
                        continue;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = m0 + tb * 16 + 4 * g + v;
                        if (t >= mend)
                            continue;
                        if (!scaled)
                            store_final<FMT, SCAL>(p, t, n, val[rb][tb][v]);
                        else
                            p.Y[(int64_t)t * p.ldy + n] =
                                bf16_bits(((float)val[rb][tb][v] * sa4[tb][v]) * sb1[rb]);
                    }
                }
            }
    };

    if (spread) {
        AS *red = reinterpret_cast<AS *>(lds);      // [NW][E][64]
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[(wave * E + (rb * TB + tb) * 4 + v) * 64 + lane] = acc[rb][tb][v];
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int e = (rb * TB + tb) * 4 + v;
                    if (e % NW != wave)
                        continue;
                    AS sum = red[e * 64 + lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w)
                        sum += red[(w * E + e) * 64 + lane];
                    const int t = SWAP ? m0 + tb * 16 + r16 : m0 + tb * 16 + 4 * g + v;
                    const int n = SWAP ? n0 + rb * 16 + 4 * g + v : n0 + rb * 16 + r16;
                    if (t >= mend || n >= nend)
                        continue;
                    if (!scaled)
                        store_final<FMT, SCAL>(p, t, n, sum);
                    else
                        p.Y[(int64_t)t * p.ldy + n] =
                            bf16_bits(((float)sum * (SWAP ? sa1[tb] : sa4[tb][v])) *
                                      (SWAP ? sb4[rb][v] : sb1[rb]));
                }
        return;
    }
    if (p.split_k == 1) {
        if (wave == 0)
            emit(acc);
        return;
    }

    const bool la = p.reduce == QLIN_REDUCE_LAST_ARRIVER;
    if (wave == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = SWAP ? m0 + tb * 16 + r16 : m0 + tb * 16 + 4 * g + v;
                    const int n = SWAP ? n0 + rb * 16 + 4 * g + v : n0 + rb * 16 + r16;
                    if (t < mend && n < nend) {
                        AS *d = part_ptr<FMT>(p, split, t, n);
                        if (la)
                            st_dev(d, (AS)acc[rb][tb][v]);
                        else
                            *d = acc[rb][tb][v];
                    }
                }
    }
    if (!la)
        return;
    const int tile = blockIdx.y * gridDim.x + blockIdx.x;
    // the flag lives in the ring: wave 0's last read of it (the combine)
    // precedes the barrier inside arrive_last
    if (!arrive_last(p.counters + tile, p.split_k, reinterpret_cast<int *>(lds)))
        return;
    if (wave == 0) {
        A4 sum[RB][TB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                sum[rb][tb] = A4{0, 0, 0, 0};
                for (int s = 0; s < p.split_k; ++s)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int t = SWAP ? m0 + tb * 16 + r16 : m0 + tb * 16 + 4 * g + v;
                        const int n = SWAP ? n0 + rb * 16 + 4 * g + v : n0 + rb * 16 + r16;
                        if (t < mend && n < nend)
                            sum[rb][tb][v] += ld_dev(part_ptr<FMT>(p, s, t, n));
                    }
            }
        emit(sum);
    }
    rearm(p.counters + tile);
}

template <int FMT, int SCAL, bool SWAP, int TMS, int TRW, int NW, int S, int CHK>
hipError_t launch_stream_lds(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_stream_lds<FMT, SCAL, SWAP, TMS, TRW, NW, S, CHK>), grid, dim3(64 * NW), 0,
                       s, a);
    return hipGetLastError();
}

#define QLIN_STREAM_LDS_INSTANCE(FMT, BIT, SW, TMS, TRW, NW, S, CHK)                 \
    {{QLIN_KERNEL_STREAM_LDS, SW, TMS, TRW, CHK, 1, NW, S, 1, 0}, BIT, FMT, SC_TC, \
     &launch_stream_lds<FMT, SC_TC, (SW) != 0, TMS, TRW, NW, S, CHK>}

#define QLIN_STREAM_LDS_INSTANCE_BLOCK(FMT, BIT, SW, TMS, TRW, NW, S, CHK)                \
    {{QLIN_KERNEL_STREAM_LDS, SW, TMS, TRW, CHK, 1, NW, S, 1, 0}, BIT, FMT, SC_BLOCK, \
     &launch_stream_lds<FMT, SC_BLOCK, (SW) != 0, TMS, TRW, NW, S, CHK>}

// (weight rows, NW, S, CHK) per token count TMS; LDS per workgroup is about
// S * (rows + TMS) * CHK bytes.  8-row tiles double the workgroup count for
// small N (the matrix core still sees 16 rows; rows 8..15 repeat 0..7 and
// their outputs are not stored).
#define QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, TMS) \
    X(FMT, BIT, SW, TMS, 16, 4, 2, 1024),           \
    X(FMT, BIT, SW, TMS, 16, 8, 2, 1024),           \
    X(FMT, BIT, SW, TMS, 16, 4, 4, 512),            \
    X(FMT, BIT, SW, TMS, 16, 8, 3, 1024),           \
    X(FMT, BIT, SW, TMS, 8, 8, 2, 1024),            \
    X(FMT, BIT, SW, TMS, 8, 4, 2, 1024)

#define QLIN_STREAM_LDS_SHAPES(X, FMT, BIT, SW)    \
    QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, 1),      \
    QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, 2),      \
    QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, 4),      \
    QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, 8),      \
    X(FMT, BIT, SW, 2, 32, 8, 3, 1024),            \
    X(FMT, BIT, SW, 4, 32, 8, 3, 1024),            \
    X(FMT, BIT, SW, 8, 32, 8, 2, 1024),            \
    X(FMT, BIT, SW, 8, 32, 8, 3, 1024),            \
    QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, 16),     \
    QLIN_STREAM_LDS_RING(X, FMT, BIT, SW, 32),     \
    X(FMT, BIT, SW, 16, 32, 4, 2, 1024),           \
    X(FMT, BIT, SW, 32, 32, 8, 2, 1024),           \
    X(FMT, BIT, SW, 32, 32, 4, 2, 512),            \
    X(FMT, BIT, SW, 32, 32, 8, 4, 512),            \
    X(FMT, BIT, SW, 32, 64, 8, 3, 512),            \
    X(FMT, BIT, SW, 16, 48, 8, 3, 512),            \
    X(FMT, BIT, SW, 32, 48, 8, 3, 512)

// Wide tiles for 16-32 tokens: every workgroup copies its token rows once per
// K range, so rows per workgroup set the token bytes per weight byte
// (TMS / TR); split-K then keeps the grid wide.
#define QLIN_STREAM_LDS_WIDE(X, FMT, BIT, SW)      \
    X(FMT, BIT, SW, 16, 96, 8, 2, 512),            \
    X(FMT, BIT, SW, 32, 96, 8, 2, 512),            \
    X(FMT, BIT, SW, 32, 112, 8, 2, 512),           \
    X(FMT, BIT, SW, 16, 128, 8, 2, 512)

}  // namespace qlin
