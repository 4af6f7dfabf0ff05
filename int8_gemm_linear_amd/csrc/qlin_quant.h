// Device helpers of the dynamic activation quantizer, shared by the
// standalone quantization kernels and the fused producers: the scale rule
// and the code rounding are one piece of code, so a fused producer returns
// exactly what the quantizer returns on the producer's bf16 output.
//
// Rule (the dynamic-scaling rule of the GEMM inputs): a token row, or a 1x128
// group of it, gets s = amax / 448 (e4m3) or amax / 127 (int8), one correctly
// rounded fp32 division, s = 1 when amax is 0; each code is x / s (fp32,
// correctly rounded) clamped to +-448 and rounded to the nearest e4m3 value
// with ties to the even code (int8: nearest integer, ties to even, clamped
// to +-127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {
namespace quant {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Nearest e4m3 code to v, |v| <= 448, ties to the even code; keeps the sign
// bit of v (so -0 -> 0x80).  Branch-free.  Below 2^-6 the e4m3 grid is the
// subnormal spacing 2^-9 (a * 512 is exact and rintf rounds half to even;
// 8 * 2^-9 is the smallest normal, code 0x08, so the code is that integer).
// Above, the fp32 pattern is rounded to 3 fraction bits, half to even
// (adding 0x7FFFF plus the kept last bit carries into the exponent when the
// fraction overflows), and exponent and fraction re-biased from 127 to 7.
__device__ inline uint32_t e4m3_code(float v)
{
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t ab = b & 0x7FFFFFFFu;
    const float a = __uint_as_float(ab);
    const uint32_t sub = (uint32_t)rintf(a * 512.0f);
    const uint32_t nrm = ((ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20) - (120u << 3);
    return sign | (a < 0.015625f ? sub : nrm);
}

// Code of x at scale s: the nearest code to the correctly rounded fp32
// quotient x / s, taken as v = x * (1/s) where that provably gives the same
// code (r = 1/s correctly rounded, so v is within 2 ulp of the quotient):
//   e4m3: v in the normal range [2^-6, 448] and its fraction bits farther
//     than 16 ulp from the tie pattern 0x80000 of the 3-bit grid; the code
//     is then the hardware's nearest-even conversion (v_cvt_pk_fp8_f32,
//     OCP e4m3 on gfx950) of v clamped to +-448;
//   int8: v farther than 2^-13 from a half-integer.
// Any other value (a near-tie, the e4m3 subnormal range, a subnormal scale
// with no finite fp32 reciprocal) is recomputed from the exact quotient
// __fdiv_rn(x, s) with the software rounding above.  Either way the code
// equals that of the exact quotient; the recomputed values are rare.
__device__ inline uint32_t e4m3_exact(float x, float s)
{
    return e4m3_code(fminf(fmaxf(__fdiv_rn(x, s), -448.0f), 448.0f));
}

__device__ inline uint32_t int8_of(float v)
{
    return (uint32_t)(int32_t)fminf(fmaxf(rintf(v), -127.0f), 127.0f) & 0xFFu;
}

// Eight bf16 (one 16-byte piece) -> eight codes packed in two words.
template <bool INT8>
__device__ inline uint2 quant8(u32x4 w, float s)
{
    const float r = __fdiv_rn(1.0f, s);
    const bool rok = s >= 0x1p-126f;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(w[j]);
        x[2 * j + 1] = bf16_hi(w[j]);
    }
    uint32_t need = 0;          // values to recompute from the exact quotient
    uint2 o;
    if (INT8) {
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = x[j] * r;
            const float a = fabsf(v);
            const bool ok = rok && (fabsf(a - floorf(a) - 0.5f) > 0x1p-13f || a > 128.0f);
            need |= ok ? 0u : 1u << j;
            c[j] = int8_of(v);
        }
        if (need) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (need & (1u << j))
                    c[j] = int8_of(__fdiv_rn(x[j], s));
        }
        o.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        o.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    } else {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j] = __builtin_amdgcn_fmed3f(x[j] * r, 448.0f, -448.0f);
            const float a = fabsf(v[j]);
            const bool ok = rok && a >= 0.015625f &&
                            ((__float_as_uint(a) & 0xFFFFFu) - 0x7FFF0u) >= 32u;
            need |= ok ? 0u : 1u << j;
        }
        o.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        o.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], (int)o.x, true);
        o.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
        o.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], (int)o.y, true);
        if (need) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (need & (1u << j)) {
                    const uint32_t sh = 8 * (j & 3);
                    const uint32_t c = e4m3_exact(x[j], s) << sh;
                    if (j < 4)
                        o.x = (o.x & ~(0xFFu << sh)) | c;
                    else
                        o.y = (o.y & ~(0xFFu << sh)) | c;
                }
        }
    }
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

// Scale of a span whose maximum |x| is m.
template <bool INT8>
__device__ inline float span_scale(float m)
{
    return m == 0.0f ? 1.0f : __fdiv_rn(m, INT8 ? 127.0f : 448.0f);
}

}  // namespace quant
}  // namespace qlin
