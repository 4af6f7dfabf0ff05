// The GEMV kernel family: 1-8 tokens (token/channel scaling) or 1-2 tokens
// (Block_FP8), on the vector ALUs instead of the matrix cores.
//
// Why: at one to eight tokens a decode GEMM does 2-16 flops per weight byte,
// so the matrix cores idle whatever the kernel does, and what remains is the
// latency chain of one launch: the weight stream, then the combine of the
// partial sums and the store.  Here a wave owns whole weight rows and reads
// each row as 1 KB contiguous segments straight into registers (lane l
// holds bytes 16 l .. 16 l + 15 of every 1 KB of the row), multiplies them
// with the same bytes of the token rows on the VALU (v_dot4_i32_i8 for int8;
// e4m3 pairs converted to fp32 and fused multiply-adds for e4m3) and sums
// the 64 lanes with cross-lane shuffles.  No LDS staging, no matrix-core
// operand layout and no cross-wave combine: the wave that read a row writes
// its outputs.
//
// Workgroup: NW waves, RPW weight rows per wave, TMS tokens; the K range is
// walked in batches of JB KB per row, the next batch loaded before the
// current one is used (two register sets); with a batch as long as the row
// (JB = 2, 4, 6 for K = 2048, 4096, 6144) every load of the row is in flight
// at once.  INT8 sums are exact int32, so
// every output equals the other kernels' bit for bit; e4m3 sums are fp32 in
// this kernel's own order (the format's tolerance covers any order).
// Split-K is not offered: a wave covers a row's whole K.
//
// With SA (shared token rows) the workgroup copies each batch of the token
// rows into LDS once (two buffers, one barrier per batch) and every wave
// reads them from there: without it each wave re-reads TMS token rows from
// L2 per weight row, which at 4-8 tokens costs more than the weights.
#pragma once

#include "qlin_device.h"
#include "qlin_dpp.h"

namespace qlin {

template <int FMT>
struct GemvAcc;
template <>
struct GemvAcc<FMT_INT8> {
    typedef int32_t T;
};
template <>
struct GemvAcc<FMT_E4M3> {
    typedef float T;
};

// acc += <w, a> over 16 int8 bytes.
__device__ inline int32_t dot16_i8(v4i w, v4i a, int32_t acc)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_sdot4(w[i], a[i], acc, false);
    return acc;
}

// acc[t][r] += <w[r], a[t]> over one 16-byte piece of RPW weight rows and
// TMS token rows: int8 as dot4 instructions; e4m3 converts every operand
// piece to fp32 once (not once per product pair) and then multiply-adds.
template <int FMT, int TMS, int RPW>
__device__ inline void dot_piece(const v4i (&w)[RPW], const v4i (&a)[TMS],
                                 typename GemvAcc<FMT>::T (&acc)[TMS][RPW])
{
    if constexpr (FMT == FMT_INT8) {
#pragma unroll
        for (int t = 0; t < TMS; ++t)
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                acc[t][r] = dot16_i8(w[r], a[t], acc[t][r]);
    } else {
        float wf[RPW][16];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[r][i], false);
                const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[r][i], true);
                wf[r][4 * i] = lo[0];
                wf[r][4 * i + 1] = lo[1];
                wf[r][4 * i + 2] = hi[0];
                wf[r][4 * i + 3] = hi[1];
            }
#pragma unroll
        for (int t = 0; t < TMS; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(a[t][i], false);
                const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(a[t][i], true);
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    acc[t][r] = __builtin_fmaf(wf[r][4 * i], lo[0], acc[t][r]);
                    acc[t][r] = __builtin_fmaf(wf[r][4 * i + 1], lo[1], acc[t][r]);
                    acc[t][r] = __builtin_fmaf(wf[r][4 * i + 2], hi[0], acc[t][r]);
                    acc[t][r] = __builtin_fmaf(wf[r][4 * i + 3], hi[1], acc[t][r]);
                }
            }
    }
}

// A 16-byte load from global memory, typed as such: through a generic
// pointer the compiler emits a flat load, which counts against the LDS
// counter too and makes every later wait a full drain.
__device__ inline v4i ld_global16(const uint8_t *p)
{
    return *(const __attribute__((address_space(1))) v4i *)(p);
}

template <int FMT, int TMS, int RPW, int NW, int JB, bool SA, int SCAL>
__global__ void __launch_bounds__(64 * NW)
k_gemv(KArgs p_)
{
    typedef typename GemvAcc<FMT>::T T;
    constexpr bool BLK = SCAL == SC_BLOCK;           // Block_FP8: scales per 128-wide K group
    static_assert(!BLK || (FMT == FMT_E4M3 && !SA), "block scaling: e4m3, token rows per wave");
    static_assert(TMS >= 1 && TMS <= 8 && RPW >= 1 && RPW <= 2 && JB >= 1 && JB <= 8, "shape");
    static_assert(TMS * RPW <= 64, "one output per lane");
    constexpr int BK = 1024 * JB;                    // K bytes per batch
    constexpr int PB = BK / 16;                      // 16-byte pieces per token row and batch
    constexpr int AQ = SA ? TMS * PB / (64 * NW) : 1;  // token pieces each thread copies
    static_assert(!SA || (TMS * PB) % (64 * NW) == 0, "token copies split evenly");

    KArgs p = p_;
    if (p.group_off && !enter_group<SCAL>(p))
        return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m0 = blockIdx.y * TMS;
    if (m0 >= p.M)
        return;                 // a group with fewer rows than the grid covers
    const int nw0 = (blockIdx.x * NW + wave) * RPW;  // first weight row of the wave

    // Row pointers, clamped: rows past N or M feed only outputs never stored.
    const uint8_t *brow[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
        brow[r] = p.B + (int64_t)min(nw0 + r, p.N - 1) * p.ldb;
    const uint8_t *arow[TMS];
#pragma unroll
    for (int t = 0; t < TMS; ++t)
        arow[t] = p.A + (int64_t)min(m0 + t, p.M - 1) * p.lda;

    // Loads are never predicated (a predicated load makes the compiler wait
    // for every load in flight before the next use): a piece past the row's
    // end reads the row's last piece and its token bytes are zeroed before
    // use; a batch past the last one (issued only to keep the code straight)
    // has every lane read the row's first 16 bytes, one cache line per wave.
    // This lane's output (lane t * RPW + r stores (m0 + t, nw0 + r)) and its
    // two scales, loaded now: read at the end they would add a memory round
    // trip after the stream whenever the scale vectors are not in cache.
    // Unpredicated, so in raw-accumulator mode (no scales) they read B.
    const int t_out = min(lane / RPW, TMS - 1);
    const int r_out = lane % RPW;
    const bool scaled = p.acc_out == nullptr && !BLK;
    const float *sap = scaled ? p.sA : reinterpret_cast<const float *>(p.B);
    const float *sbp = scaled ? p.sB : reinterpret_cast<const float *>(p.B);
    const float sa_out = sap[scaled ? min(m0 + t_out, p.M - 1) : 0];
    const float sb_out = sbp[scaled ? min(nw0 + r_out, p.N - 1) : 0];

    const int K = p.K;
    const int nb = (K + BK - 1) / BK;
    auto koff = [&](int b, int piece) { return b < nb ? min(b * BK + 16 * piece, K - 16) : 0; };

    // Token rows shared through LDS: [buffer][token][piece].
    __shared__ __attribute__((aligned(16))) v4i lds_a[SA ? 2 : 1][SA ? TMS : 1][SA ? PB : 1];
    v4i ar[AQ];                                      // this thread's token pieces in flight
    auto load_a_shared = [&](int b) {
        if constexpr (SA) {
#pragma unroll
            for (int q = 0; q < AQ; ++q) {
                const int i = threadIdx.x + q * 64 * NW;
                ar[q] = ld_global16(arow[i / PB] + koff(b, i % PB));
            }
        }
    };
    auto store_a_shared = [&](int b, int buf) {
        if constexpr (SA) {
#pragma unroll
            for (int q = 0; q < AQ; ++q) {
                const int i = threadIdx.x + q * 64 * NW;
                const bool ok = b * BK + 16 * (i % PB) < K;      // K % 16 == 0
                lds_a[buf][i / PB][i % PB] = ok ? ar[q] : zero4i();
            }
        }
    };

    v4i w0[RPW][JB], a0[TMS][JB], w1[RPW][JB], a1[TMS][JB];
    // Block_FP8: the scales of each piece's 128-wide K group (weight block
    // row n / 128, token row), loaded with the piece, one set per batch.
    float gw0[BLK ? RPW : 1][BLK ? JB : 1], gx0[BLK ? TMS : 1][BLK ? JB : 1];
    float gw1[BLK ? RPW : 1][BLK ? JB : 1], gx1[BLK ? TMS : 1][BLK ? JB : 1];
    auto load_group_scales = [&](int b, float (&gw)[BLK ? RPW : 1][BLK ? JB : 1],
                                 float (&gx)[BLK ? TMS : 1][BLK ? JB : 1]) {
        if constexpr (BLK) {
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const int grp = koff(b, j * 64 + lane) >> 7;
#pragma unroll
                for (int r = 0; r < RPW; ++r)
                    gw[r][j] = p.sB[(int64_t)(min(nw0 + r, p.N - 1) >> 7) * p.G + grp];
#pragma unroll
                for (int t = 0; t < TMS; ++t)
                    gx[t][j] = p.sA[(int64_t)min(m0 + t, p.M - 1) * p.G + grp];
            }
        }
    };
    auto load = [&](int b, v4i (&w)[RPW][JB], v4i (&a)[TMS][JB]) {
        load_a_shared(b);                            // before the weights: waited for first
        if constexpr (SA)
            __builtin_amdgcn_sched_barrier(0);       // and kept there by the scheduler
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int k = koff(b, j * 64 + lane);
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                w[r][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(brow[r] + k));
            if constexpr (!SA) {
#pragma unroll
                for (int t = 0; t < TMS; ++t)
                    a[t][j] = ld_global16(arow[t] + k);
            }
        }
    };
    T acc[TMS][RPW];
#pragma unroll
    for (int t = 0; t < TMS; ++t)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
            acc[t][r] = 0;
    auto use = [&](int b, int buf, const v4i (&w)[RPW][JB], const v4i (&a)[TMS][JB],
                   const float (&gw)[BLK ? RPW : 1][BLK ? JB : 1],
                   const float (&gx)[BLK ? TMS : 1][BLK ? JB : 1]) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            v4i wj[RPW], aj[TMS];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                wj[r] = w[r][j];
            if constexpr (SA) {
#pragma unroll
                for (int t = 0; t < TMS; ++t)
                    aj[t] = lds_a[buf][t][j * 64 + lane];
            } else {
                const bool ok = b * BK + j * 1024 + 16 * lane < K;
#pragma unroll
                for (int t = 0; t < TMS; ++t)
                    aj[t] = ok ? a[t][j] : zero4i();
            }
            if constexpr (BLK) {
                // acc += (group piece product) * sA * sB, the promotion of
                // the block kernels applied per 16-value piece
                T d[TMS][RPW];
#pragma unroll
                for (int t = 0; t < TMS; ++t)
#pragma unroll
                    for (int r = 0; r < RPW; ++r)
                        d[t][r] = 0;
                dot_piece<FMT, TMS, RPW>(wj, aj, d);
#pragma unroll
                for (int t = 0; t < TMS; ++t)
#pragma unroll
                    for (int r = 0; r < RPW; ++r)
                        acc[t][r] = __builtin_fmaf(d[t][r], gx[t][j] * gw[r][j], acc[t][r]);
            } else {
                dot_piece<FMT, TMS, RPW>(wj, aj, acc);
            }
        }
    };

    // Two register sets (and with SA two LDS buffers), alternating by batch
    // parity: batch b + 1 is in flight while batch b is used.  With SA a
    // batch's token pieces go to LDS after the previous batch is used, then
    // one barrier publishes them (and retires the buffer read before).
    if (nb == 1) {
        load_group_scales(0, gw0, gx0);
        load(0, w0, a0);
        store_a_shared(0, 0);
        if (SA)
            __syncthreads();
        use(0, 0, w0, a0, gw0, gx0);
    } else {
        load_group_scales(0, gw0, gx0);
        load(0, w0, a0);
        store_a_shared(0, 0);
        if (SA)
            __syncthreads();
        for (int b = 0; b < nb; b += 2) {
            load_group_scales(b + 1, gw1, gx1);
            load(b + 1, w1, a1);
            use(b, 0, w0, a0, gw0, gx0);
            if (SA) {
                if (b + 1 < nb)
                    store_a_shared(b + 1, 1);
                __syncthreads();
            }
            if (b + 1 >= nb)
                break;
            load_group_scales(b + 2, gw0, gx0);
            load(b + 2, w0, a0);
            use(b + 1, 1, w1, a1, gw1, gx1);
            if (SA) {
                if (b + 2 < nb)
                    store_a_shared(b + 2, 0);
                __syncthreads();
            }
        }
    }

#pragma unroll
    for (int t = 0; t < TMS; ++t)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
            acc[t][r] = wave_sum(acc[t][r]);

    if (lane >= TMS * RPW || m0 + t_out >= p.M || nw0 + r_out >= p.N)
        return;
    T v = acc[0][0];
#pragma unroll
    for (int tt = 0; tt < TMS; ++tt)
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
            if (tt == t_out && rr == r_out)
                v = acc[tt][rr];
    const int64_t t = m0 + t_out, n = nw0 + r_out;
    if (scaled)
        p.Y[t * p.ldy + n] = bf16_bits(((float)v * sa_out) * sb_out);   // as store_final
    else
        store_final<FMT, SCAL>(p, (int)t, (int)n, v);
}

template <int FMT, int TMS, int RPW, int NW, int JB, bool SA, int SCAL>
hipError_t launch_gemv(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_gemv<FMT, TMS, RPW, NW, JB, SA, SCAL>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// Registry key: tile_m = tokens, tile_n = weight rows per workgroup
// (NW x RPW), tile_k = K bytes per batch, waves_k = NW, stages = 2 (two
// register sets, token rows read by every wave) or 4 (token rows shared
// through two LDS buffers as well); split_k = 1 only.
#define QLIN_GEMV_INSTANCE(FMT, BIT, TMS, RPW, NW, JB, SA)                                      \
    {{QLIN_KERNEL_GEMV, 0, TMS, (NW) * (RPW), 1024 * (JB), 1, NW, (SA) ? 4 : 2, 1, 0}, BIT, FMT, \
     SC_TC, &launch_gemv<FMT, TMS, RPW, NW, JB, SA, SC_TC>}
#define QLIN_GEMV_BLOCK_INSTANCE(TMS, RPW, NW, JB)                                              \
    {{QLIN_KERNEL_GEMV, 0, TMS, (NW) * (RPW), 1024 * (JB), 1, NW, 2, 1, 0}, FB_BLOCK, FMT_E4M3,   \
     SC_BLOCK, &launch_gemv<FMT_E4M3, TMS, RPW, NW, JB, false, SC_BLOCK>}

// Block_FP8 (token rows read by every wave).
#define QLIN_GEMV_BLOCK_SHAPES(X) \
    X(1, 1, 4, 2),                \
    X(1, 1, 8, 2),                \
    X(1, 2, 4, 2),                \
    X(1, 1, 4, 4),                \
    X(2, 1, 4, 2),                \
    X(2, 2, 4, 2)

#define QLIN_GEMV_SHAPES(X, FMT, BIT)  \
    X(FMT, BIT, 1, 1, 4, 2, false),    \
    X(FMT, BIT, 1, 2, 4, 2, false),    \
    X(FMT, BIT, 1, 1, 8, 2, false),    \
    X(FMT, BIT, 1, 1, 4, 1, false),    \
    X(FMT, BIT, 2, 1, 4, 2, false),    \
    X(FMT, BIT, 2, 2, 4, 2, false),    \
    X(FMT, BIT, 4, 1, 4, 2, false),    \
    X(FMT, BIT, 4, 2, 4, 1, false),    \
    X(FMT, BIT, 1, 1, 4, 4, false),    \
    X(FMT, BIT, 1, 1, 4, 6, false),    \
    X(FMT, BIT, 1, 1, 8, 6, false),    \
    X(FMT, BIT, 2, 1, 4, 4, false),    \
    X(FMT, BIT, 2, 1, 4, 6, false),    \
    X(FMT, BIT, 2, 1, 4, 6, true),     \
    X(FMT, BIT, 4, 1, 4, 6, true),     \
    X(FMT, BIT, 2, 1, 4, 2, true),     \
    X(FMT, BIT, 4, 1, 4, 2, true),     \
    X(FMT, BIT, 4, 2, 4, 2, true),     \
    X(FMT, BIT, 8, 1, 4, 2, true),     \
    X(FMT, BIT, 8, 2, 4, 2, true),     \
    X(FMT, BIT, 8, 1, 8, 2, true)

}  // namespace qlin
