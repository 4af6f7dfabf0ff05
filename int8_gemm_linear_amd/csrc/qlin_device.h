// Device-side building blocks for the gfx950 kernels: matrix-core wrappers,
// the 128-byte K step, bf16 rounding, and the scale-and-store epilogue.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_internal.h"

namespace qlin {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Accumulator element: exact int32 for int8 operands, fp32 for e4m3.
template <int FMT> struct AccT;
template <> struct AccT<FMT_INT8> { typedef int32_t scalar; typedef v4i v4; typedef v16i v16; };
template <> struct AccT<FMT_E4M3> { typedef float scalar; typedef v4f v4; typedef v16f v16; };

__device__ inline v4i zero4i() { return v4i{0, 0, 0, 0}; }

// One 128-byte K step of a 16x16 output block on the matrix cores.
//
// Operand layout (verified on gfx950 for both instructions): lane l feeds
// row (l % 16) of its operand and holds 32 bytes of the step's K, as two
// 16-byte pieces x0 and x1 (which bytes is up to the caller).  The A-side
// and B-side operands use the same lane -> K mapping, so the K sum is
// complete whatever slot order the hardware uses inside a lane.
//   int8: two v_mfma_i32_16x16x64_i8 (x0 pair, then x1 pair), exact int32.
//   e4m3: one v_mfma_f32_16x16x128_f8f6f4 (format 0 = OCP e4m3, no block
//         scaling), fp32 accumulate.
// Result layout: lane l holds column (l % 16), rows 4*(l/16) + 0..3.
template <int FMT>
__device__ inline typename AccT<FMT>::v4 mma16(v4i a0, v4i a1, v4i b0, v4i b1,
                                               typename AccT<FMT>::v4 c);

template <>
__device__ inline v4i mma16<FMT_INT8>(v4i a0, v4i a1, v4i b0, v4i b1, v4i c)
{
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, c, 0, 0, 0);
    return c;
}

template <>
__device__ inline v4f mma16<FMT_E4M3>(v4i a0, v4i a1, v4i b0, v4i b1, v4f c)
{
    v8i a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    v8i b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    // cbsz/blgp = 0: both operands e4m3; scale operands 0 select the
    // unscaled encoding (no microscaling).
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 32x32 blocks: lane l feeds row (l % 32) and holds 64 bytes of the 128-byte
// K step, bytes [64*(l/32), 64*(l/32)+64), as x[0..3] (16 bytes each).
//   int8: four v_mfma_i32_32x32x32_i8 (one per 16-byte piece).
//   e4m3: two v_mfma_f32_32x32x64_f8f6f4 (pieces 0-1, then 2-3).
// Result layout: lane l holds column (l % 32), rows 8*(v/4) + 4*(l/32) + v%4.
template <int FMT>
__device__ inline typename AccT<FMT>::v16 mma32(const v4i *a, const v4i *b,
                                                typename AccT<FMT>::v16 c);

template <>
__device__ inline v16i mma32<FMT_INT8>(const v4i *a, const v4i *b, v16i c)
{
#pragma unroll
    for (int j = 0; j < 4; ++j)
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[j], c, 0, 0, 0);
    return c;
}

template <>
__device__ inline v16f mma32<FMT_E4M3>(const v4i *a, const v4i *b, v16f c)
{
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        v8i x = __builtin_shufflevector(a[2 * j], a[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        v8i y = __builtin_shufflevector(b[2 * j], b[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
    }
    return c;
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950;
// NaN stays NaN, overflow goes to infinity, fp32 subnormals are kept).
__device__ inline uint16_t bf16_bits(float f)
{
    __hip_bfloat16 h = __float2bfloat16(f);
    return *reinterpret_cast<uint16_t *>(&h);
}

// Copy 16 bytes per lane HBM/L2 -> LDS (global_load_lds_dwordx4): lane i's
// bytes land at lds + 16*i (the LDS base is wave-uniform, passed in M0).
// Written as inline assembly on purpose: for the builtin the compiler must
// assume the in-flight copy may alias any later LDS read and inserts
// vmcnt(0) before every ds_read, which would also wait for the copies of
// later pipeline stages.  Callers therefore wait for their own copies with
// explicit, exactly counted s_waitcnt vmcnt(n) before reading the stage.
// No register output: the copy writes only LDS.
__device__ inline void lds_dma16(const void *g, const void *lds)
{
    const unsigned off = (unsigned)(size_t)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(off))
                 : "memory", "m0");
}

// As lds_dma16, with the non-temporal cache policy: for weight bytes that
// are read once per launch (streamed past L2 rather than kept there).  A
// plain read of a 262 MB weight matrix through LDS runs about 7% faster
// this way on MI355X.
__device__ inline void lds_dma16_nt(const void *g, const void *lds)
{
    const unsigned off = (unsigned)(size_t)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(off))
                 : "memory", "m0");
}

// Copy 4 bytes per lane HBM/L2 -> LDS (global_load_lds_dword): lane i's
// bytes land at lds + 4*i.  Same contract as lds_dma16 (inline assembly, no
// register output, the caller counts its own copies in vmcnt).
__device__ inline void lds_dma4(const void *g, const void *lds)
{
    const unsigned off = (unsigned)(size_t)lds;
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(off))
                 : "memory", "m0");
}

__device__ inline v4i ld_nt(const uint8_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

__device__ inline v4i ld16(const uint8_t *p)
{
    return *reinterpret_cast<const v4i *>(p);
}

// ---------------------------------------------------------------------------
// Epilogue.  `v` is the full-K dot product for (t, n): an int32 (int8), an
// fp32 sum (e4m3, token/channel), or the already group-scaled fp32 sum
// (Block_FP8).  Token/channel scaling multiplies by sA[t] then sB[n] in fp32;
// the result is rounded once to bf16.
// ---------------------------------------------------------------------------
template <int FMT, int SCAL>
__device__ inline float finish_value(const KArgs &p, int t, int n,
                                     typename AccT<FMT>::scalar v)
{
    if (SCAL == SC_BLOCK)
        return (float)v;
    return ((float)v * p.sA[t]) * p.sB[n];
}

// Store one final value.  Raw mode (acc_out != NULL) writes the int32 sum.
template <int FMT, int SCAL>
__device__ inline void store_final(const KArgs &p, int t, int n, typename AccT<FMT>::scalar v)
{
    if (FMT == FMT_INT8 && p.acc_out) {
        p.acc_out[(int64_t)t * p.ldacc + n] = (int32_t)v;
        return;
    }
    p.Y[(int64_t)t * p.ldy + n] = bf16_bits(finish_value<FMT, SCAL>(p, t, n, v));
}

// Four final token/channel outputs for columns n..n+3 of row t (all in
// range) with the scales already in registers: sa = sA[t], sb = sB[n..n+3].
template <int FMT, int SCAL>
__device__ inline void store_final4_pre(const KArgs &p, int t, int n,
                                        typename AccT<FMT>::v4 v, float sa, v4f sb)
{
    uint16_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = bf16_bits(((float)v[j] * sa) * sb[j]);
    uint16_t *d = p.Y + (int64_t)t * p.ldy + n;
    if ((p.ldy & 3) == 0) {
        uint2 w;
        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<uint2 *>(d) = w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = h[j];
    }
}

// Store four final values for columns n..n+3 of row t (all in range).
template <int FMT, int SCAL>
__device__ inline void store_final4(const KArgs &p, int t, int n,
                                    typename AccT<FMT>::v4 v)
{
    if (FMT == FMT_INT8 && p.acc_out) {
        int32_t *d = p.acc_out + (int64_t)t * p.ldacc + n;
        if ((p.ldacc & 3) == 0) {
            *reinterpret_cast<v4i *>(d) = v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) d[j] = (int32_t)v[j];
        }
        return;
    }
    uint16_t h[4];
    if (SCAL == SC_BLOCK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = bf16_bits((float)v[j]);
    } else {
        const float sa = p.sA[t];
        const float *sb = p.sB + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = bf16_bits(((float)v[j] * sa) * sb[j]);
    }
    uint16_t *d = p.Y + (int64_t)t * p.ldy + n;
    if ((p.ldy & 3) == 0) {
        uint2 w;
        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        *reinterpret_cast<uint2 *>(d) = w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = h[j];
    }
}

// ---------------------------------------------------------------------------
// Split-K exchange between workgroups on different XCDs.  The L2 of each XCD
// is not coherent with the others, and an agent-scope fence (__threadfence)
// compiles to a write-back plus invalidate of the whole L2, which costs tens
// of microseconds when every workgroup issues it.  Instead the partials are
// written and read with agent-scope atomic stores/loads (device-coherent
// accesses that do not leave stale or dirty lines in a non-coherent L2), and
// the writer waits for its own stores to be acknowledged before the counter
// increment.  The last arriver observes the final counter value through an
// agent-scope atomic, then reads every partial with agent-scope loads.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline void st_dev(T *p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ inline T ld_dev(T *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the workgroup calls this after writing its partials with
// st_dev.  Returns true (in all threads) for the workgroup whose increment
// brought the tile's counter to split_k.  `flag` is one int of LDS for the
// broadcast; the caller may pass memory of a pipeline ring it no longer reads
// (the barrier below orders it after every wave's last use).
__device__ inline bool arrive_last(int32_t *counter, int split_k, int *flag)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // own partial stores acknowledged
    __syncthreads();
    if (threadIdx.x == 0)
        *flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                split_k - 1;
    __syncthreads();
    return *flag != 0;
}

__device__ inline bool arrive_last(int32_t *counter, int split_k)
{
    __shared__ int s_last;
    return arrive_last(counter, split_k, &s_last);
}

// The last arriver re-arms the counter for the next call (stream order makes
// it visible to the next launch).
__device__ inline void rearm(int32_t *counter)
{
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Partials: [split][M][N], 4-byte elements, row stride N.
template <int FMT>
__device__ inline typename AccT<FMT>::scalar *part_ptr(const KArgs &p, int split, int t, int n)
{
    typedef typename AccT<FMT>::scalar S;
    return reinterpret_cast<S *>(p.part) + ((int64_t)split * p.M + t) * p.N + n;
}

// Grouped GEMM: narrows the arguments to the workgroup's group (grid.z).
// p.M holds the bound on rows per group; the group's own row count caps it.
// Returns false when the group is empty.  Called first thing in a kernel,
// before any barrier, so a workgroup with nothing to do simply returns.
template <int SCAL>
__device__ inline bool enter_group(KArgs &p)
{
    const int g = blockIdx.z;
    const int m_beg = p.group_off[g];
    p.M = min(p.group_off[g + 1] - m_beg, p.M);
    if (p.M <= 0)
        return false;
    p.A += (int64_t)m_beg * p.lda;
    p.sA += SCAL == SC_BLOCK ? (int64_t)m_beg * p.G : (int64_t)m_beg;
    p.Y += (int64_t)m_beg * p.ldy;
    p.B += (int64_t)g * p.b_gstride;
    p.sB += (int64_t)g * p.sb_gstride;
    return true;
}

// Split index of the workgroup: grid.z, unless grid.z is the group.
__device__ inline int split_index(const KArgs &p) { return p.group_off ? 0 : (int)blockIdx.z; }

}  // namespace qlin
