// The half-step TILE kernel: prefill token counts with token/channel scaling,
// one wave per SIMD and large per-wave tiles.
//
// Why a second tile kernel.  At 128 bytes of K per LDS stage a 256x256 tile
// takes 64 KB per stage, so only two stages fit the 160 KB of LDS and a
// copy has one step of compute to land; and with eight waves per workgroup
// each wave owns only a 128x64 sub-tile, so every step reads 192 KB out of
// LDS for 2048 matrix-core cycles per SIMD, about the LDS bandwidth.  Here a
// stage holds 64 bytes of K (one 32x32x64 e4m3 or two 32x32x32 int8
// instructions per 32x32 block), so four stages of a 256x256 tile fit in
// 128 KB and a copy is issued three half-steps before it is read; and four
// waves each own a 128x128 sub-tile (256 accumulator registers), which cuts
// the LDS reads per matrix-core cycle by a third.
//
// Software pipeline, per half-step i with the fragments of step i already
// in registers:
//   wait for the copies of step i+1 (exact vmcnt: the copies of later steps
//   stay in flight) and for this wave's own LDS reads, barrier;
//   issue the copies of step i+S into the stage step i was read from;
//   run the matrix-core instructions of step i, interleaved one for one
//   with the LDS reads of step i+1's fragments into the other register set.
// So the LDS read latency hides behind the matrix cores, and the barrier of
// a half-step is the only point where the waves meet.
//
// LDS stage: [BM rows of A][BN rows of B], 64 bytes per row.  The four
// 16-byte chunks of stage row r are stored at slot c ^ swz64(r).  The
// swizzle was chosen by measurement: for this read pattern (lane l reads
// row l % 32, chunk pair l / 32) it sustains ~240 bytes per clock per CU of
// ds_read_b128, where the unswizzled layout gets a quarter of that and
// swizzles keyed on r >> 1 half.  global_load_lds writes lane
// i's 16 bytes to slot (i % 4) of row (i / 4) of its 1 KB, so the swizzle
// is applied on the global side: lane i fetches chunk (i % 4) ^ swz64(row).
//
// Matrix-core operands: for a 32x32 block lane l feeds row (l % 32) and
// holds chunks 2*(l/32) and 2*(l/32)+1 of the half-step.  e4m3 uses both in
// one v_mfma_f32_32x32x64_f8f6f4; int8 issues two v_mfma_i32_32x32x32_i8,
// piece j using chunk j of each lane pair.  A and B use the same lane -> K
// mapping, so every K of the half-step is summed exactly once.
#pragma once

#include "qlin_tile.h"

namespace qlin {

__device__ inline int swz64(int r) { return ((r >> 2) ^ (r >> 3)) & 3; }

// s_waitcnt vmcnt(L * n) lgkmcnt(0) for a run-time n in [0, NMAX].
template <int L, int NMAX>
__device__ inline void wait_copies(int n)
{
    static_assert(L * NMAX <= 63, "vmcnt range");
    if constexpr (NMAX > 0) {
        if (n >= NMAX) {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(L * NMAX) : "memory");
            return;
        }
        wait_copies<L, NMAX - 1>(n);
    } else {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
}

// Scheduling groups: matrix-core instruction k followed by LDS reads
// [k*NREAD/NMMA, (k+1)*NREAD/NMMA).
template <int NMMA, int NREAD, int K = 0>
__device__ inline void sched_interleave()
{
    if constexpr (K < NMMA) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int nr = ((K + 1) * NREAD) / NMMA - (K * NREAD) / NMMA;
        if constexpr (nr > 0)
            __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        sched_interleave<NMMA, NREAD, K + 1>();
    }
}

// Matrix-core pieces of one half-step on a 32x32 block.
template <int FMT> struct HalfPieces;
template <> struct HalfPieces<FMT_INT8> { static constexpr int n = 2; };
template <> struct HalfPieces<FMT_E4M3> { static constexpr int n = 1; };

template <int FMT>
__device__ inline typename AccT<FMT>::v16 mma_half(const v4i (&x)[2], const v4i (&y)[2], int j,
                                                   typename AccT<FMT>::v16 c);
template <>
__device__ inline v16i mma_half<FMT_INT8>(const v4i (&x)[2], const v4i (&y)[2], int j, v16i c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(x[j], y[j], c, 0, 0, 0);
}
template <>
__device__ inline v16f mma_half<FMT_E4M3>(const v4i (&x)[2], const v4i (&y)[2], int, v16f c)
{
    v8i a = __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7);
    v8i b = __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int FMT, bool SWAP, int BM, int BN, int WM, int WN, int S>
__global__ void __launch_bounds__(64 * WM * WN)
k_tile_h(KArgs p_)
{
    typedef typename AccT<FMT>::v16 A16;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM;
    constexpr int WTN = BN / WN;
    constexpr int FM = WTM / 32;
    constexpr int FN = WTN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int STAGE = ROWS * 64;
    constexpr int GROUPS = ROWS / 16;          // 1 KB copies per stage
    constexpr int GPW = GROUPS / NW;           // copies per wave per stage
    constexpr int L = GPW;
    constexpr int NP = HalfPieces<FMT>::n;
    constexpr int NREAD = 2 * (FM + FN);       // ds_read_b128 per wave per half-step
    constexpr int NMMA = FM * FN * NP;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile shape");
    static_assert(BM % 32 == 0 && GROUPS % NW == 0, "copies must split evenly over the waves");
    static_assert(S >= 3 && S <= 8, "stages");
    static_assert(S * STAGE <= 160 * 1024, "LDS");
    static_assert(L * (S - 1) <= 63, "vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t lds[S * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int fr = lane & 31;
    const int fh = lane >> 5;

    KArgs p = p_;
    if (p.group_off && !(enter_group<SC_TC>(p) && tile_in_group<BM, BN>(p)))
        return;

    int m0, n0;
    tile_origin<BM, BN>(p, m0, n0);

    // K range of this split, in 64-byte half-steps.
    const int KS = p.K >> 7;
    const int split = split_index(p);
    const int s_beg = min(KS, split * p.steps_per_split);
    const int s_end = min(KS, s_beg + p.steps_per_split);
    const int h_beg = 2 * s_beg;
    const int nh = 2 * (s_end - s_beg);

    // Per-lane global source of each copy of a stage: copy g covers stage
    // rows 16g .. 16g+15, lane i row 16g + i/4.
    const uint8_t *src[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int row = (wave + i * NW) * 16 + (lane >> 2);
        const uint8_t *base;
        if (row < BM) {
            const int t = min(m0 + row, p.M - 1);          // rows past M feed only masked outputs
            base = p.A + (int64_t)t * p.lda;
        } else {
            const int n = min(n0 + row - BM, p.N - 1);
            base = p.B + (int64_t)n * p.ldb;
        }
        src[i] = base + (int64_t)h_beg * 64 + 16 * ((lane & 3) ^ swz64(row));
    }
    auto issue = [&](int h, int stage) {
        uint8_t *dst0 = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < GPW; ++i)
            lds_dma16(src[i] + (int64_t)h * 64, dst0 + (wave + i * NW) * 1024);
    };

    // Fragment addresses inside a stage: row r = base row + fr, chunks
    // 2*fh and 2*fh + 1 (base rows are multiples of 32 and swz64(r + 32) =
    // swz64(r), so the swizzle depends on fr only).
    const int sw = swz64(fr);
    const int off0 = fr * 64 + 16 * ((2 * fh) ^ sw);
    const int off1 = fr * 64 + 16 * ((2 * fh + 1) ^ sw);
    const int a_row0 = wm * WTM;
    const int b_row0 = BM + wn * WTN;

    v4i fa[2][FM][2], fb[2][FN][2];
    A16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[fm][fn][v] = 0;

    auto read_frag = [&](v4i (&f)[2], const uint8_t *st, int row0) {
        f[0] = *reinterpret_cast<const v4i *>(st + row0 * 64 + off0);
        f[1] = *reinterpret_cast<const v4i *>(st + row0 * 64 + off1);
    };

    // One half-step: the matrix-core work of the fragments in set P,
    // interleaved with the LDS reads of the next half-step (stage `nst`) into
    // set P^1.  On the last half-step the reads are repeated from a valid
    // stage and never used, which keeps a single code path.
    auto half = [&](auto PC, const uint8_t *nst) {
        constexpr int P = decltype(PC)::value;
#pragma unroll
        for (int k = 0; k < NMMA; ++k) {
            const int j = k / (FM * FN);
            const int fm = (k / FN) % FM;
            const int fn = k % FN;
            acc[fm][fn] = SWAP ? mma_half<FMT>(fb[P][fn], fa[P][fm], j, acc[fm][fn])
                               : mma_half<FMT>(fa[P][fm], fb[P][fn], j, acc[fm][fn]);
#pragma unroll
            for (int r = (k * NREAD) / NMMA; r < ((k + 1) * NREAD) / NMMA; ++r) {
                const int blk = r >> 1;
                const int q = r & 1;
                const int row0 = blk < FM ? a_row0 + 32 * blk : b_row0 + 32 * (blk - FM);
                v4i *dstf = blk < FM ? &fa[P ^ 1][blk][q] : &fb[P ^ 1][blk - FM][q];
                *dstf = *reinterpret_cast<const v4i *>(nst + row0 * 64 + (q ? off1 : off0));
            }
        }
        // keep that interleave through scheduling: one matrix-core
        // instruction, then the reads assigned to it
        sched_interleave<NMMA, NREAD>();
    };

    if (nh > 0) {
        const int pre = min(S, nh);
        for (int h = 0; h < pre; ++h)
            issue(h, h);
        wait_copies<L, S - 1>(pre - 1);
        __syncthreads();
        {
            const uint8_t *st = lds;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) read_frag(fa[0][fm], st, a_row0 + 32 * fm);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) read_frag(fb[0][fn], st, b_row0 + 32 * fn);
        }
        int cur = 0;                           // stage of half-step i
        auto step = [&](auto PC, int i) {
            const bool more = i + 1 < nh;
            const int nxt = more ? (cur + 1 == S ? 0 : cur + 1) : cur;
            if (more) {
                wait_copies<L, S - 2>(min(S - 2, nh - 2 - i));
                __syncthreads();
                if (i + S < nh)
                    issue(i + S, cur);
            }
            half(PC, lds + nxt * STAGE);
            cur = nxt;
        };
        for (int i = 0; i < nh; i += 2) {
            step(std::integral_constant<int, 0>{}, i);
            if (i + 1 < nh)
                step(std::integral_constant<int, 1>{}, i + 1);
        }
    }

    static_assert(BM * BN * 2 <= S * STAGE, "the output tile is staged in the ring");
    tile_finish<FMT, SC_TC, SWAP, BM, BN, WM, WN>(p, acc, m0, n0, wm, wn, lane, lds);
}

template <int FMT, bool SWAP, int BM, int BN, int WM, int WN, int S>
hipError_t launch_tile_h(const KArgs &a, dim3 grid, hipStream_t s)
{
    hipLaunchKernelGGL((k_tile_h<FMT, SWAP, BM, BN, WM, WN, S>), grid, dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

// Registry entry: a TILE config with tile_k = 64 selects this kernel.
#define QLIN_TILE_H_INSTANCE(FMT, BIT, SW, BM, BN, WM, WN, S)                      \
    {{QLIN_KERNEL_TILE, SW, BM, BN, 64, WM, WN, S, 1, 0}, BIT, FMT, SC_TC,          \
     &launch_tile_h<FMT, (SW) != 0, BM, BN, WM, WN, S>}

// (BM, BN, WM, WN, S); LDS = S * (BM + BN) * 64 B.
// (The 8-wave 256x256 forms, with two fragment sets and 128 accumulators per
// wave, do not fit 256 registers and spill; they are not built.)
#define QLIN_TILE_H_SHAPES(X, FMT, BIT, SW) \
    X(FMT, BIT, SW, 256, 128, 4, 2, 6),     \
    X(FMT, BIT, SW, 256, 256, 2, 2, 4),     \
    X(FMT, BIT, SW, 256, 128, 2, 2, 6),     \
    X(FMT, BIT, SW, 128, 256, 2, 2, 6),     \
    X(FMT, BIT, SW, 128, 128, 2, 2, 8),     \
    X(FMT, BIT, SW, 128, 128, 2, 2, 4)

}  // namespace qlin
