// Activation quantization: bf16 activations -> 8-bit codes + fp32 scales,
// the producer of the GEMM's A operand.
//
// "HelionがvLLMに統合 ..." (24-ai.news), section "vLLMに統合されたカーネル"
// (kernels integrated into vLLM), items 1 and 5, names dynamic per-token FP8
// quantization and per-token-group FP8 quantization; the pages give no
// formula.  The rule used (the dynamic-scaling rule of the GEMM inputs): a
// token row (or a 1x128 group of it) gets s = amax / 448 (e4m3) or
// amax / 127 (int8), one correctly rounded fp32 division, s = 1 when amax is
// 0; each code is x / s (fp32, correctly rounded), clamped to +-448 and
// rounded to the nearest e4m3 value with ties to the even code (int8:
// nearest integer, ties to even, clamped to +-127).
//
// Both kernels are HBM-bound (2 bytes read, 1 byte written per element).
//   per token: one workgroup of 512 threads per row; each lane loads 16-byte
//     pieces (8 bf16) of the row, keeps up to kTokReg of them in registers for
//     the second pass (longer rows re-read the rest, which is L2-resident),
//     the row maximum is reduced across the workgroup, and every lane
//     writes 8 codes (8 bytes) per piece.
//   per group: 16 lanes own one 128-element group (16 bytes each); the
//     group maximum is a 16-lane butterfly; each lane writes 8 codes; a
//     256-thread workgroup covers 16 groups per sweep, grid-stride over all
//     groups of the matrix.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlinear.h"

namespace qlin {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Nearest e4m3 code to v, |v| <= 448, ties to the even code; keeps the sign
// bit of v (so -0 -> 0x80).  Below 2^-6 the e4m3 grid is the subnormal
// spacing 2^-9 (a * 512 is exact, rintf rounds half to even; 8 * 2^-9 is the
// smallest normal, code 0x08, so the code is that integer).  Above, the fp32
// fraction is rounded to 3 bits (half to even), carrying into the exponent.
__device__ inline uint32_t e4m3_code(float v)
{
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a < 0.015625f)
        return sign | (uint32_t)rintf(a * 512.0f);
    const uint32_t ab = b & 0x7FFFFFFFu;
    int e = (int)(ab >> 23) - 127;
    uint32_t m = (ab >> 20) & 7u;
    const uint32_t rest = ab & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u)))
        ++m;
    if (m == 8u) {
        m = 0;
        ++e;
    }
    return sign | ((uint32_t)(e + 7) << 3) | m;
}

template <bool INT8>
__device__ inline uint32_t quant1(float x, float s)
{
    float v = __fdiv_rn(x, s);
    if (INT8) {
        float r = fminf(fmaxf(rintf(v), -127.0f), 127.0f);
        return (uint32_t)(int32_t)r & 0xFFu;
    }
    v = fminf(fmaxf(v, -448.0f), 448.0f);
    return e4m3_code(v);
}

// Eight bf16 (one 16-byte piece) -> eight codes packed in two words.
template <bool INT8>
__device__ inline uint2 quant8(u32x4 w, float s)
{
    uint2 o;
    o.x = quant1<INT8>(bf16_lo(w.x), s) | (quant1<INT8>(bf16_hi(w.x), s) << 8) |
          (quant1<INT8>(bf16_lo(w.y), s) << 16) | (quant1<INT8>(bf16_hi(w.y), s) << 24);
    o.y = quant1<INT8>(bf16_lo(w.z), s) | (quant1<INT8>(bf16_hi(w.z), s) << 8) |
          (quant1<INT8>(bf16_lo(w.w), s) << 16) | (quant1<INT8>(bf16_hi(w.w), s) << 24);
    return o;
}

__device__ inline float amax8(u32x4 w)
{
    float m = fmaxf(fabsf(bf16_lo(w.x)), fabsf(bf16_hi(w.x)));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(w.y)), fabsf(bf16_hi(w.y))));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(w.z)), fabsf(bf16_hi(w.z))));
    m = fmaxf(m, fmaxf(fabsf(bf16_lo(w.w)), fabsf(bf16_hi(w.w))));
    return m;
}

constexpr int kTokThreads = 512;
constexpr int kTokReg = 8;          // pieces per lane kept in registers: rows up to 32768

template <bool INT8>
__global__ void __launch_bounds__(kTokThreads)
k_quant_token(const uint16_t *__restrict__ X, int64_t ldx, uint8_t *__restrict__ Q, int64_t ldq,
              float *__restrict__ S, int K)
{
    __shared__ float red[kTokThreads / 64];
    const int row = blockIdx.x;
    const u32x4 *x = reinterpret_cast<const u32x4 *>(X + (int64_t)row * ldx);
    uint2 *q = reinterpret_cast<uint2 *>(Q + (int64_t)row * ldq);
    const int P = K >> 3;                                  // 16-byte pieces in the row
    u32x4 keep[kTokReg];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kTokReg; ++i) {
        const int p = threadIdx.x + i * kTokThreads;
        keep[i] = p < P ? __builtin_nontemporal_load(x + p) : u32x4{0, 0, 0, 0};
        m = fmaxf(m, amax8(keep[i]));
    }
    for (int p = threadIdx.x + kTokReg * kTokThreads; p < P; p += kTokThreads)
        m = fmaxf(m, amax8(x[p]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < kTokThreads / 64; ++w)
        m = fmaxf(m, red[w]);
    const float s = m == 0.0f ? 1.0f : __fdiv_rn(m, INT8 ? 127.0f : 448.0f);
    if (threadIdx.x == 0)
        S[row] = s;
#pragma unroll
    for (int i = 0; i < kTokReg; ++i) {
        const int p = threadIdx.x + i * kTokThreads;
        if (p < P)
            q[p] = quant8<INT8>(keep[i], s);
    }
    for (int p = threadIdx.x + kTokReg * kTokThreads; p < P; p += kTokThreads)
        q[p] = quant8<INT8>(x[p], s);
}

constexpr int kGrpThreads = 256;

__global__ void __launch_bounds__(kGrpThreads)
k_quant_group128(const uint16_t *__restrict__ X, int64_t ldx, uint8_t *__restrict__ Q, int64_t ldq,
                 float *__restrict__ S, int M, int G)
{
    const int sub = threadIdx.x & 15;                       // lane within the group
    const int64_t total = (int64_t)M * G;
    for (int64_t grp = (int64_t)blockIdx.x * (kGrpThreads / 16) + (threadIdx.x >> 4); grp < total;
         grp += (int64_t)gridDim.x * (kGrpThreads / 16)) {
        const int64_t row = grp / G;
        const int g = (int)(grp - row * G);
        const u32x4 w = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(X + row * ldx + (int64_t)g * 128) + sub);
        float m = amax8(w);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o, 16));
        const float s = m == 0.0f ? 1.0f : __fdiv_rn(m, 448.0f);
        reinterpret_cast<uint2 *>(Q + row * ldq + (int64_t)g * 128)[sub] = quant8<false>(w, s);
        if (sub == 0)
            S[grp] = s;
    }
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxRows = (int64_t)1 << 24;
constexpr int64_t kMaxK = (int64_t)1 << 20;

qlin_status check_common(int64_t M, int64_t K, const void *X, int64_t ldx, const void *Q,
                         int64_t ldq, const float *scale)
{
    if (M < 0 || M > kMaxRows || K <= 0 || K > kMaxK || K % 16 != 0)
        return QLIN_ERR_BAD_SHAPE;
    if (M == 0)
        return QLIN_OK;
    if (!X || !Q || !scale)
        return QLIN_ERR_NULL_POINTER;
    if (ldx < K || ldq < K || ldx % 8 != 0 || ldq % 16 != 0 || ldx > kMaxK * 16 || ldq > kMaxK * 16)
        return QLIN_ERR_BAD_STRIDE;
    if (!aligned(X, 16) || !aligned(Q, 16) || !aligned(scale, 4))
        return QLIN_ERR_MISALIGNED;
    return QLIN_OK;
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" {

qlin_status qlin_quant_per_token(qlin_dtype dt, int64_t M, int64_t K, const uint16_t *X,
                                 int64_t ldx, void *Q, int64_t ldq, float *scale, void *stream)
{
    if (dt != QLIN_E4M3 && dt != QLIN_INT8)
        return QLIN_ERR_BAD_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    qlin_status st = check_common(M, K, X, ldx, Q, ldq, scale);
    if (st != QLIN_OK || M == 0)
        return st;
    if (dt == QLIN_INT8)
        hipLaunchKernelGGL(k_quant_token<true>, dim3((unsigned)M), dim3(kTokThreads), 0, s, X,
                           ldx, static_cast<uint8_t *>(Q), ldq, scale, (int)K);
    else
        hipLaunchKernelGGL(k_quant_token<false>, dim3((unsigned)M), dim3(kTokThreads), 0, s, X,
                           ldx, static_cast<uint8_t *>(Q), ldq, scale, (int)K);
    return hipGetLastError() == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
}

qlin_status qlin_quant_per_group128(int64_t M, int64_t K, const uint16_t *X, int64_t ldx, void *Q,
                                    int64_t ldq, float *scale, void *stream)
{
    qlin_status st = check_common(M, K, X, ldx, Q, ldq, scale);
    if (st != QLIN_OK)
        return st;
    if (K % 128 != 0)
        return QLIN_ERR_BAD_SHAPE;
    if (M == 0)
        return QLIN_OK;
    const int64_t groups = M * (K / 128);
    const int64_t per_wg = kGrpThreads / 16;
    const int64_t blocks = (groups + per_wg - 1) / per_wg;
    const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
    hipLaunchKernelGGL(k_quant_group128, dim3(grid), dim3(kGrpThreads), 0,
                       static_cast<hipStream_t>(stream), X, ldx,
                       static_cast<uint8_t *>(Q), ldq, scale, (int)M, (int)(K / 128));
    return hipGetLastError() == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
}

}  // extern "C"
