// Row engine of the activation producers: one workgroup of W waves per token
// row produces the row's bf16 activation (a copy of the input, an RMS norm,
// or SiLU-and-mul) and quantizes it (per token, or per 1x128 group).
//
// These kernels are HBM-bound: per value 2 bytes in (4 for SiLU-and-mul,
// +4 for a residual read and written back) and 1 byte out.  What keeps them
// at the bandwidth is latency hiding, so a row is as few waves as fit it in
// registers (W = 1 for rows up to 4096 values, 2 up to 8192, ... 8 up to
// 32768) when there are rows enough to fill the machine, more (up to 8)
// when there are not (quantizer and RMS norm; SiLU-and-mul rows keep the
// fewest, see silu_waves): every lane issues all its 16-byte loads (kReg
// pieces) before it uses any, a single-wave row reduces with shuffles
// alone, and small workgroups let many rows be in flight per CU.  Lane t of the row owns the
// pieces t, t + 64W, ...; pieces beyond the register window (rows longer
// than 32768) are produced again from the L2-resident input in the
// quantizer's second pass.  Per-group scaling needs no row reduction: the
// 16 lanes of one 128-value group are consecutive (64W is a multiple of 16).
// SiLU-and-mul with a per-token scale at decode sizes spreads each row over
// several workgroups instead (k_silu_spread).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qlin_dpp.h"
#include "qlin_quant.h"

namespace qlin {
namespace rows {

using namespace quant;

enum { OP_QUANT = 0, OP_RMS = 1, OP_SILU = 2 };
enum { Q_TOKEN_E4M3 = 0, Q_TOKEN_INT8 = 1, Q_GROUP_E4M3 = 2 };
constexpr int kReg = 8;          // 16-byte pieces per lane held in registers
constexpr int kMaxW = 8;

struct RowArgs {
    const uint16_t *X;           // [M][ldx] bf16 (SiLU: gate | up, 2K values)
    int64_t ldx;
    uint16_t *R;                 // residual [M][ldr] (RMS norm, may be null)
    int64_t ldr;
    const uint16_t *Wt;          // RMS weight [K]
    float eps;
    uint8_t *Q;                  // codes [M][ldq]
    int64_t ldq;
    float *S;                    // scales [M] or [M][K/128]
    int K;
};

// double -> bf16 bits, nearest-even, one rounding: truncation to fp32 with
// the inexact bit kept in the last place (round to odd; 24 >= 8 + 2 bits),
// then nearest-even to bf16.
__device__ inline uint32_t bf16_of_double(double d)
{
    const float f = __double2float_rz(d);
    uint32_t u = __float_as_uint(f);
    if ((double)f != d)
        u |= 1u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline double dlo(uint32_t w) { return (double)bf16_lo(w); }
__device__ inline double dhi(uint32_t w) { return (double)bf16_hi(w); }
__device__ inline uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// h = bf16(x + r) for 8 values.  The fp32 sum of two bf16 values is exact
// unless their exponents differ by more than 16, and then the sum lies
// within 2^-16 of the larger value, far from any bf16 rounding boundary
// around it: rounding the fp32 sum to bf16 (nearest even) gives the bf16
// rounding of the exact sum.
__device__ inline uint32_t bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline u32x4 add_round8(u32x4 x, u32x4 r)
{
    u32x4 h;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        h[j] = pack2(bf16_rne(bf16_lo(x[j]) + bf16_lo(r[j])), bf16_rne(bf16_hi(x[j]) + bf16_hi(r[j])));
    return h;
}

__device__ inline double sumsq8(u32x4 h, double acc)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc = fma(dlo(h[j]), dlo(h[j]), acc);
        acc = fma(dhi(h[j]), dhi(h[j]), acc);
    }
    return acc;
}

// y = bf16((h * w) * inv) for 8 values (h * w is exact in double).
__device__ inline u32x4 norm8(u32x4 h, u32x4 w, double inv)
{
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        y[j] = pack2(bf16_of_double((dlo(h[j]) * dlo(w[j])) * inv),
                     bf16_of_double((dhi(h[j]) * dhi(w[j])) * inv));
    return y;
}

// bf16(g / (1 + e^-g) * u), the real value rounded once, for 8 values.
// Fast path in fp32 for |g| <= 64: p = -g log2(e) carried as p_hi + p_lo
// (p_lo from an fma: the argument is exact to ~2^-48), e^-g = 2^p_hi *
// (1 + p_lo ln 2) with the hardware exp2 (~1 ulp), then 1 + t, the hardware
// reciprocal (~1 ulp) and two products.  Measured on the MI355X against the
// double evaluation over every bf16 gate in [-64, 64] times 256 bf16 ups
// (6.75 million pairs): y32 is within 3.4 fp32 ulp of the real value.  When
// every intermediate is a normal fp32 number and y32's low 16 bits are more
// than 24 ulp (7x that) from the bf16 tie pattern 0x8000, no bf16 rounding
// boundary lies between y32 and the real value, so rounding y32 gives the
// same bf16.  The other values (about 0.07%, and |g| > 64 where e^-g leaves
// fp32) are computed in double (library exp, correctly rounded division)
// and rounded once.
// Out of line: rare, and inlined it would raise the register count of every
// SiLU kernel (and multiply the code size).
__device__ __attribute__((noinline)) uint32_t silu_exact(float g, float u)
{
    const double gd = g;
    return bf16_of_double((gd / (1.0 + exp(-gd))) * (double)u);
}

// The fast path of one value: its bf16 bits from y32 in `b`; false when
// they must come from silu_exact instead.
__device__ inline bool silu_fast1(float g, float u, uint32_t &b)
{
    constexpr float L_HI = 1.44269502162933349609375f;          // log2(e) rounded to fp32
    constexpr float L_LO = 1.925962989e-8f;                     // log2(e) - L_HI
    constexpr float LN2 = 0.693147180559945309f;
    const float ng = -g;
    const float p_hi = ng * L_HI;
    const float p_lo = fmaf(ng, L_HI, -p_hi) + ng * L_LO;
    const float t = __builtin_amdgcn_exp2f(p_hi) * fmaf(p_lo, LN2, 1.0f);
    const float sv = g * __builtin_amdgcn_rcpf(1.0f + t);
    const float y = sv * u;
    const float as = fabsf(sv), ay = fabsf(y);
    const uint32_t bits = __float_as_uint(y);
    b = (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
    return fabsf(g) <= 64.0f && as >= 0x1p-100f && ay >= 0x1p-100f && ay <= 0x1p+100f &&
           ((bits & 0xFFFFu) - 0x7FE8u) >= 48u;
}

__device__ inline u32x4 silu8(u32x4 gw, u32x4 uw)
{
    float g[8], u[8];
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        g[2 * j] = bf16_lo(gw[j]);
        g[2 * j + 1] = bf16_hi(gw[j]);
        u[2 * j] = bf16_lo(uw[j]);
        u[2 * j + 1] = bf16_hi(uw[j]);
    }
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        need |= silu_fast1(g[j], u[j], b[j]) ? 0u : 1u << j;
    if (need) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (need & (1u << j))
                b[j] = silu_exact(g[j], u[j]);
    }
    u32x4 y;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        y[j] = pack2(b[2 * j], b[2 * j + 1]);
    return y;
}

// Sum / maximum over the row's W waves (every lane gets the result).
template <int W>
__device__ inline double row_sum(double v)
{
    v = wave_sum(v);
    if constexpr (W > 1) {
        __shared__ double red[kMaxW];
        if ((threadIdx.x & 63) == 0)
            red[threadIdx.x >> 6] = v;
        __syncthreads();
        v = red[0];
#pragma unroll
        for (int w = 1; w < W; ++w)
            v += red[w];
    }
    return v;
}

template <int W>
__device__ inline float row_max(float v)
{
    v = wave_max(v);
    if constexpr (W > 1) {
        __shared__ float red[kMaxW];
        if ((threadIdx.x & 63) == 0)
            red[threadIdx.x >> 6] = v;
        __syncthreads();
        v = red[0];
#pragma unroll
        for (int w = 1; w < W; ++w)
            v = fmaxf(v, red[w]);
    }
    return v;
}

// Quantizes the row: pieces of the register window in `y`, the rest
// produced again by redo(p).
template <int QM, int W, class Redo>
__device__ inline void quantize_row(const u32x4 (&y)[kReg], int P, uint8_t *qrow, float *srow,
                                    Redo redo)
{
    constexpr int NT = 64 * W;
    uint2 *q = reinterpret_cast<uint2 *>(qrow);
    const int t = threadIdx.x;
    if constexpr (QM == Q_GROUP_E4M3) {
        // P is a multiple of 16: the 16 lanes of a group are all active or
        // all idle, so the 16-wide butterfly stays inside the group
        auto emit = [&](const u32x4 &v, int p) {
            const float m = row16_max(amax8(v));
            const float s = span_scale<false>(m);
            q[p] = quant8<false>(v, s);
            if ((t & 15) == 0)
                srow[p >> 4] = s;
        };
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            if (p < P)
                emit(y[i], p);
        }
        for (int p = t + kReg * NT; p < P; p += NT)
            emit(redo(p), p);
    } else {
        constexpr bool INT8 = QM == Q_TOKEN_INT8;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kReg; ++i)
            m = fmaxf(m, amax8(y[i]));
        for (int p = t + kReg * NT; p < P; p += NT)
            m = fmaxf(m, amax8(redo(p)));
        const float s = span_scale<INT8>(row_max<W>(m));
        if (t == 0)
            srow[0] = s;
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            if (p < P)
                q[p] = quant8<INT8>(y[i], s);
        }
        for (int p = t + kReg * NT; p < P; p += NT)
            q[p] = quant8<INT8>(redo(p), s);
    }
}

// SKIP (SiLU-and-mul only): register slots past the row's end are not
// evaluated (they hold zeros, which would take the exact double path).
template <int OP, int QM, int W, bool RES, bool SKIP = false>
__global__ void __launch_bounds__(64 * W)
k_rows(RowArgs a)
{
    constexpr int NT = 64 * W;
    const int row = blockIdx.x;
    const int t = threadIdx.x;
    const int P = a.K >> 3;
    const u32x4 *x = reinterpret_cast<const u32x4 *>(a.X + (int64_t)row * a.ldx);
    uint8_t *qrow = a.Q + (int64_t)row * a.ldq;
    float *srow = a.S + (QM == Q_GROUP_E4M3 ? (int64_t)row * (a.K >> 7) : (int64_t)row);
    const u32x4 zero = {0, 0, 0, 0};
    u32x4 y[kReg];

    if constexpr (OP == OP_QUANT) {
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            y[i] = p < P ? __builtin_nontemporal_load(x + p) : zero;
        }
        quantize_row<QM, W>(y, P, qrow, srow, [&](int p) { return x[p]; });
    } else if constexpr (OP == OP_SILU) {
        const u32x4 *u = x + P;                     // up half of the row
        u32x4 gu[kReg];
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            y[i] = p < P ? __builtin_nontemporal_load(x + p) : zero;
            gu[i] = p < P ? __builtin_nontemporal_load(u + p) : zero;
        }
#pragma unroll
        for (int i = 0; i < kReg; ++i)
            if (!SKIP || t + i * NT < P)
                y[i] = silu8(y[i], gu[i]);
        quantize_row<QM, W>(y, P, qrow, srow, [&](int p) { return silu8(x[p], u[p]); });
    } else {
        u32x4 *r = RES ? reinterpret_cast<u32x4 *>(a.R + (int64_t)row * a.ldr) : nullptr;
        const u32x4 *w = reinterpret_cast<const u32x4 *>(a.Wt);
        u32x4 rr[kReg];
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            y[i] = p < P ? __builtin_nontemporal_load(x + p) : zero;
            if (RES)
                rr[i] = p < P ? r[p] : zero;
        }
        // h (the residual row replaced by it) and the sum of its squares
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            if (RES && p < P) {
                y[i] = add_round8(y[i], rr[i]);
                r[p] = y[i];
            }
            acc = sumsq8(y[i], acc);
        }
        for (int p = t + kReg * NT; p < P; p += NT) {
            u32x4 h = x[p];
            if (RES) {
                h = add_round8(h, r[p]);
                r[p] = h;
            }
            acc = sumsq8(h, acc);
        }
        const double inv = 1.0 / sqrt(row_sum<W>(acc) / (double)a.K + (double)a.eps);
#pragma unroll
        for (int i = 0; i < kReg; ++i) {
            const int p = t + i * NT;
            if (p < P)
                y[i] = norm8(y[i], w[p], inv);
        }
        // beyond the register window h is re-read (the residual row holds it)
        quantize_row<QM, W>(y, P, qrow, srow,
                            [&](int p) { return norm8(RES ? r[p] : x[p], w[p], inv); });
    }
}

// Upper bound of |bf16 SiLU-and-mul| of one value: silu(g) < g for g > 0 and
// |silu(g)| < 0.2785 for g <= 0, so |silu(g) u| <= max(g, 0.279) |u|.  The
// fp32 product is exact for g > 0.279 (two bf16 factors) and at most half an
// ulp low otherwise (still above 0.2785 |u|); a NaN product, or one under
// 2^-100 (where underflow could make it low), counts as unbounded.
__device__ inline float silu_bound(float g, float u)
{
    const float b = fmaxf(g, 0.279f) * fabsf(u);
    return b >= 0x1p-100f ? b : INFINITY;
}

// SiLU-and-mul with a per-token scale at decode sizes: a row spread over
// several workgroups, none of which needs another's result.  At a few tokens
// one workgroup per row leaves most CUs idle and every lane with a long
// serial chain of SiLU and quantizer work.  Here workgroup (row, sl) of W
// waves owns the row's pieces sl * 64W + lane, evaluated exactly (silu8) and
// quantized; the row's scale needs the maximum |value| of the whole row,
// which every workgroup of the row finds on its own: the maximum m of its
// own values, then an upper bound of every other value of the row
// (silu_bound, a multiply per value), and the exact value of only those
// whose bound is not below m -- any other value is below m, so its bf16
// rounding is at most m (m is a bf16 value).  Candidates are taken one value
// per lane per pass, so a pass costs one SiLU evaluation however the
// candidates fall; they are a few per row for real activations (the bound is
// within a factor 1 + e^-g of the value for g > 0).  Every workgroup of a
// row thus computes the same maximum and scale, exactly those of the
// one-workgroup kernel.  The row is read whole by each of its workgroups
// (from L2 after the first): a few KB per row at these sizes.
template <int QM, int W, int PR>
__global__ void __launch_bounds__(64 * W)
k_silu_spread(RowArgs a)
{
    constexpr int NT = 64 * W;
    constexpr bool INT8 = QM == Q_TOKEN_INT8;
    static_assert(QM != Q_GROUP_E4M3, "per-token scaling");
    static_assert(PR <= 16, "candidate masks");
    const int row = blockIdx.x;
    const int sl = blockIdx.y;
    const int t = threadIdx.x;
    const int P = a.K >> 3;
    const u32x4 *x = reinterpret_cast<const u32x4 *>(a.X + (int64_t)row * a.ldx);
    const u32x4 *up = x + P;
    const u32x4 zero = {0, 0, 0, 0};
    u32x4 g[PR], v[PR];
#pragma unroll
    for (int i = 0; i < PR; ++i) {
        const int p = t + i * NT;
        g[i] = p < P ? x[p] : zero;
        v[i] = p < P ? up[p] : zero;
    }
    const bool own = sl * NT + t < P;
    u32x4 yo = zero;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < PR; ++i)
        if (i == sl && own) {
            yo = silu8(g[i], v[i]);
            m = amax8(yo);
        }
    const float mown = row_max<W>(m);
    uint64_t cand[2] = {0, 0};           // bit 8 * (i % 8) + j of word i / 8
#pragma unroll
    for (int i = 0; i < PR; ++i) {
        if (i == sl || t + i * NT >= P)
            continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float gg = (j & 1) ? bf16_hi(g[i][j >> 1]) : bf16_lo(g[i][j >> 1]);
            const float uu = (j & 1) ? bf16_hi(v[i][j >> 1]) : bf16_lo(v[i][j >> 1]);
            if (!(silu_bound(gg, uu) < mown))
                cand[i >> 3] |= 1ull << (8 * (i & 7) + j);
        }
    }
    while (__any((cand[0] | cand[1]) != 0)) {
        if (cand[0] | cand[1]) {
            const int w = cand[0] ? 0 : 1;
            const int k = __builtin_ctzll(cand[w]);
            cand[w] &= cand[w] - 1;
            const int i = 8 * w + (k >> 3), j = k & 7;
            u32x4 gi = g[0], vi = v[0];
#pragma unroll
            for (int q = 1; q < PR; ++q)
                if (q == i) {
                    gi = g[q];
                    vi = v[q];
                }
            const uint32_t gw = gi[j >> 1], uw = vi[j >> 1];
            const float gg = (j & 1) ? bf16_hi(gw) : bf16_lo(gw);
            const float uu = (j & 1) ? bf16_hi(uw) : bf16_lo(uw);
            uint32_t b;
            if (!silu_fast1(gg, uu, b))
                b = silu_exact(gg, uu);
            m = fmaxf(m, fabsf(__uint_as_float(b << 16)));
        }
    }
    if constexpr (W > 1)
        __syncthreads();                 // row_max's slots are written again
    const float s = span_scale<INT8>(row_max<W>(m));
    if (sl == 0 && t == 0)
        a.S[row] = s;
    if (own)
        reinterpret_cast<uint2 *>(a.Q + (int64_t)row * a.ldq)[sl * NT + t] = quant8<INT8>(yo, s);
}

// Workgroups of k_silu_spread are 8 waves (every lane holding kReg pieces of
// the row, so rows up to 32768 values).  Measured at 32 tokens (SiLU-and-mul
// then per-token e4m3, K = 6144 / 12288): 2 waves per workgroup 7.07 / 7.89
// us, 4 waves 6.85 / 7.96, 8 waves 6.75 / 7.29, one wave with 16 pieces per
// lane 9.66 us at K = 6144; the one-workgroup-per-row kernel 7.3 / 11.1.
constexpr int kSpreadW = 8;

// Waves per row: the fewest that hold the row's pieces in registers, and
// more while the grid has fewer than 2048 waves: with few rows (decode) the
// per-lane work of a one-wave row is a long serial chain, so the row is
// spread over up to 8 waves instead.
inline int waves_for(int64_t M, int64_t K)
{
    const int64_t P = K >> 3;
    int w = 1;
    while (w < kMaxW && (int64_t)64 * w * kReg < P)
        w *= 2;
    while (w < kMaxW && M * w < 2048 && (int64_t)64 * w < P)
        w *= 2;
    return w;
}

// Waves per SiLU-and-mul row.  With rows enough to fill the machine, the
// fewest that hold the row's pieces in registers, at most 4 (the kernels
// need ~125 registers, so an 8-wave workgroup would leave room for only one
// per CU; longer rows recompute the pieces past the register window:
// measured faster, 113 vs 134 us at 2048 x 25600); every lane then runs all
// kReg slots.  With few rows (fewer than 2048 waves in the grid: decode)
// the row is spread over up to 8 waves to shorten each lane's serial chain,
// and the slots past the row's end are skipped (`skip`): evaluated, their
// zeros would take the exact double path, which made wider rows slower.
inline int silu_waves(int64_t M, int64_t K, bool *skip)
{
    const int64_t P = K >> 3;
    int w = 1;
    while (w < 4 && (int64_t)64 * w * kReg < P)
        w *= 2;
    const int fewest = w;
    while (w < kMaxW && M * w < 2048 && (int64_t)64 * w < P)
        w *= 2;
    *skip = w > fewest;
    return w;
}

template <int OP, int QM, bool RES>
hipError_t launch_rows(const RowArgs &a, int64_t M, hipStream_t s)
{
    const dim3 grid((unsigned)M);
    bool skip = false;
    const int w = OP == OP_SILU ? silu_waves(M, a.K, &skip) : waves_for(M, a.K);
    if constexpr (OP == OP_SILU && QM != Q_GROUP_E4M3) {
        // decode sizes with a per-token scale: the row spread over workgroups
        const int64_t P = a.K >> 3;
        if (skip && P <= (int64_t)64 * kSpreadW * kReg) {
            const dim3 g2((unsigned)M, (unsigned)((P + 64 * kSpreadW - 1) / (64 * kSpreadW)));
            hipLaunchKernelGGL((k_silu_spread<QM, kSpreadW, kReg>), g2, dim3(64 * kSpreadW), 0, s, a);
            return hipGetLastError();
        }
    }
    if constexpr (OP == OP_SILU) {
        if (skip) {
            switch (w) {
            case 2: hipLaunchKernelGGL((k_rows<OP, QM, 2, RES, true>), grid, dim3(128), 0, s, a); break;
            case 4: hipLaunchKernelGGL((k_rows<OP, QM, 4, RES, true>), grid, dim3(256), 0, s, a); break;
            default: hipLaunchKernelGGL((k_rows<OP, QM, 8, RES, true>), grid, dim3(512), 0, s, a); break;
            }
            return hipGetLastError();
        }
    }
    switch (w) {
    case 1: hipLaunchKernelGGL((k_rows<OP, QM, 1, RES>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_rows<OP, QM, 2, RES>), grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_rows<OP, QM, 4, RES>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_rows<OP, QM, 8, RES>), grid, dim3(512), 0, s, a); break;
    }
    return hipGetLastError();
}

// Launch with the scaling mode chosen at run time.
template <int OP, bool RES>
hipError_t launch_rows_qm(int qm, const RowArgs &a, int64_t M, hipStream_t s)
{
    if (qm == Q_TOKEN_INT8)
        return launch_rows<OP, Q_TOKEN_INT8, RES>(a, M, s);
    if (qm == Q_TOKEN_E4M3)
        return launch_rows<OP, Q_TOKEN_E4M3, RES>(a, M, s);
    return launch_rows<OP, Q_GROUP_E4M3, RES>(a, M, s);
}

}  // namespace rows
}  // namespace qlin
