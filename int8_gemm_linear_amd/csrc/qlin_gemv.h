// The GEMV kernel family: 1-4 tokens with token/channel scaling, on the
// vector ALUs instead of the matrix cores.
//
// Why: at one to four tokens a decode GEMM does 2-8 flops per weight byte,
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
// current one is used (two register sets).  INT8 sums are exact int32, so
// every output equals the other kernels' bit for bit; e4m3 sums are fp32 in
// this kernel's own order (the format's tolerance covers any order).
// Split-K is not offered: a wave covers a row's whole K.
#pragma once

#include "qlin_device.h"

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

// acc += <w, a> over 16 bytes (16 int8 or 16 e4m3 values).
template <int FMT>
__device__ inline typename GemvAcc<FMT>::T dot16(v4i w, v4i a, typename GemvAcc<FMT>::T acc);

template <>
__device__ inline int32_t dot16<FMT_INT8>(v4i w, v4i a, int32_t acc)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_sdot4(w[i], a[i], acc, false);
    return acc;
}

template <>
__device__ inline float dot16<FMT_E4M3>(v4i w, v4i a, float acc)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v2f w0 = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
        const v2f w1 = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
        const v2f a0 = __builtin_amdgcn_cvt_pk_f32_fp8(a[i], false);
        const v2f a1 = __builtin_amdgcn_cvt_pk_f32_fp8(a[i], true);
        acc = __builtin_fmaf(w0[0], a0[0], acc);
        acc = __builtin_fmaf(w0[1], a0[1], acc);
        acc = __builtin_fmaf(w1[0], a1[0], acc);
        acc = __builtin_fmaf(w1[1], a1[1], acc);
    }
    return acc;
}

// Sum over the 64 lanes of a wave (every lane gets the total).  Integer sums
// are exact in any order; fp32 sums use the same butterfly in every call.
template <typename T>
__device__ inline T wave_sum(T v)
{
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
        v += __shfl_xor(v, s, 64);
    return v;
}

template <int FMT, int TMS, int RPW, int NW, int JB>
__global__ void __launch_bounds__(64 * NW)
k_gemv(KArgs p_)
{
    typedef typename GemvAcc<FMT>::T T;
    static_assert(TMS >= 1 && TMS <= 4 && RPW >= 1 && RPW <= 2 && JB >= 1 && JB <= 4, "shape");
    static_assert(TMS * RPW <= 64, "one output per lane");
    constexpr int BK = 1024 * JB;                    // K bytes per batch

    KArgs p = p_;
    if (p.group_off && !enter_group<SC_TC>(p))
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
    // end reads the row's last piece and its token bytes are zeroed at use;
    // a batch past the last one (issued only to keep the code straight) has
    // every lane read the row's first 16 bytes, one cache line per wave.
    const int K = p.K;
    const int nb = (K + BK - 1) / BK;
    v4i w0[RPW][JB], a0[TMS][JB], w1[RPW][JB], a1[TMS][JB];
    auto load = [&](int b, v4i (&w)[RPW][JB], v4i (&a)[TMS][JB]) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int k = b < nb ? min(b * BK + j * 1024 + 16 * lane, K - 16) : 0;
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                w[r][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(brow[r] + k));
#pragma unroll
            for (int t = 0; t < TMS; ++t)
                a[t][j] = *reinterpret_cast<const v4i *>(arow[t] + k);
        }
    };
    T acc[TMS][RPW];
#pragma unroll
    for (int t = 0; t < TMS; ++t)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
            acc[t][r] = 0;
    auto use = [&](int b, const v4i (&w)[RPW][JB], const v4i (&a)[TMS][JB]) {
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const bool ok = b * BK + j * 1024 + 16 * lane < K;   // K % 16 == 0
#pragma unroll
            for (int t = 0; t < TMS; ++t) {
                const v4i at = ok ? a[t][j] : zero4i();
#pragma unroll
                for (int r = 0; r < RPW; ++r)
                    acc[t][r] = dot16<FMT>(w[r][j], at, acc[t][r]);
            }
        }
    };

    // Two register sets, alternating by batch parity: batch b + 1 is in
    // flight while batch b is used.
    if (nb == 1) {
        load(0, w0, a0);
        use(0, w0, a0);
    } else {
        load(0, w0, a0);
        for (int b = 0; b < nb; b += 2) {
            load(b + 1, w1, a1);
            use(b, w0, a0);
            if (b + 1 >= nb)
                break;
            load(b + 2, w0, a0);
            use(b + 1, w1, a1);
        }
    }

#pragma unroll
    for (int t = 0; t < TMS; ++t)
#pragma unroll
        for (int r = 0; r < RPW; ++r)
            acc[t][r] = wave_sum(acc[t][r]);

    // Lane t * RPW + r stores output (m0 + t, nw0 + r).
    const int t = lane / RPW;
    const int r = lane % RPW;
    if (lane >= TMS * RPW || m0 + t >= p.M || nw0 + r >= p.N)
        return;
    T v = acc[0][0];
#pragma unroll
    for (int tt = 0; tt < TMS; ++tt)
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr)
            if (tt == t && rr == r)
                v = acc[tt][rr];
    store_final<FMT, SC_TC>(p, m0 + t, nw0 + r, v);
}

template <int FMT, int TMS, int RPW, int NW, int JB>
hipError_t launch_gemv(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_gemv<FMT, TMS, RPW, NW, JB>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// Registry key: tile_m = tokens, tile_n = weight rows per workgroup
// (NW x RPW), tile_k = K bytes per batch, waves_k = NW, stages = 2 (two
// register sets); split_k = 1 only.
#define QLIN_GEMV_INSTANCE(FMT, BIT, TMS, RPW, NW, JB)                                    \
    {{QLIN_KERNEL_GEMV, 0, TMS, (NW) * (RPW), 1024 * (JB), 1, NW, 2, 1, 0}, BIT, FMT, SC_TC, \
     &launch_gemv<FMT, TMS, RPW, NW, JB>}

#define QLIN_GEMV_SHAPES(X, FMT, BIT) \
    X(FMT, BIT, 1, 1, 4, 2),          \
    X(FMT, BIT, 1, 2, 4, 2),          \
    X(FMT, BIT, 1, 1, 8, 2),          \
    X(FMT, BIT, 1, 1, 4, 1),          \
    X(FMT, BIT, 2, 1, 4, 2),          \
    X(FMT, BIT, 2, 2, 4, 2),          \
    X(FMT, BIT, 4, 1, 4, 2),          \
    X(FMT, BIT, 4, 2, 4, 1)

}  // namespace qlin
