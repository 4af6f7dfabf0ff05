// Fused producers of the GEMM's A operand: RMS norm (with an optional
// residual add) or SiLU-and-mul, followed by the dynamic quantizer, in one
// pass over the activation.
//
// "HelionがvLLMに統合 ..." (24-ai.news), section "vLLMに統合されたカーネル"
// (kernels integrated into vLLM), items 2, 3, 6 and 7 name
// rms_norm_dynamic_per_token_quant, silu_and_mul_dynamic_per_token_quant,
// rms_norm_per_block_quant and silu_and_mul_per_block_quant, and the section
// on per-kernel performance reports their speed-ups over the unfused
// kernels; the pages give no formula.  Reading: a fused kernel returns
// exactly what the unfused pair returns, i.e. the quantizer (per token, or
// per 1x128 group) applied to the producer's bf16 output, where that bf16
// value is the real-number result rounded once to nearest-even:
//   RMS norm over a row of K:  h = x, or h = bf16(x + r) with a residual r
//     (and r is replaced by h);  y_k = bf16(h_k * w_k / sqrt(mean(h^2) + eps));
//   SiLU-and-mul over a row of 2K (gate | up):  y_k = bf16(g_k / (1 + e^-g_k) * u_k).
// The producer is evaluated in double: squares and products of bf16 values
// are exact there, the square root and the division are correctly rounded,
// exp is the device library's double exp; only the order of the sum of
// squares (a workgroup tree here) differs from a sequential sum, by far less
// than a bf16 rounding interval.  Double -> bf16 rounds once: truncation to
// fp32 with the inexact bit kept in the last place (round to odd, 24 >= 8 + 2
// bits), then nearest-even to bf16.
//
// The kernels are the row engine's (one workgroup of 1-8 waves per token
// row, every load of a lane issued before its first use); SiLU takes an
// fp32 fast path whose bf16 rounding is provably the same and falls back to
// double near a rounding boundary.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qlin_rows.h"
#include "qlinear.h"

namespace qlin {
namespace {

using namespace rows;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int64_t kMaxRows = (int64_t)1 << 24;
constexpr int64_t kMaxK = (int64_t)1 << 20;

// Shared argument checks: K output values per row, X rows of xcols values.
qlin_status check_args(int64_t M, int64_t K, int group, const void *X, int64_t ldx, int64_t xcols,
                       const void *Q, int64_t ldq, const float *scale)
{
    if (M < 0 || M > kMaxRows || K <= 0 || K > kMaxK || K % 16 != 0 || (group && K % 128 != 0))
        return QLIN_ERR_BAD_SHAPE;
    if (M == 0)
        return QLIN_OK;
    if (!X || !Q || !scale)
        return QLIN_ERR_NULL_POINTER;
    if (ldx < xcols || ldq < K || ldx % 8 != 0 || ldq % 16 != 0 || ldx > kMaxK * 16 ||
        ldq > kMaxK * 16)
        return QLIN_ERR_BAD_STRIDE;
    if (!aligned(X, 16) || !aligned(Q, 16) || !aligned(scale, 4))
        return QLIN_ERR_MISALIGNED;
    return QLIN_OK;
}

qlin_status rms_norm_quant(int qm, int64_t M, int64_t K, const uint16_t *X, int64_t ldx,
                           uint16_t *residual, int64_t ldr, const uint16_t *weight, float eps,
                           void *Q, int64_t ldq, float *scale, void *stream)
{
    qlin_status st = check_args(M, K, qm == Q_GROUP_E4M3, X, ldx, K, Q, ldq, scale);
    if (st != QLIN_OK || M == 0)
        return st;
    if (!weight)
        return QLIN_ERR_NULL_POINTER;
    if (!aligned(weight, 16) || (residual && !aligned(residual, 16)))
        return QLIN_ERR_MISALIGNED;
    if (residual && (ldr < K || ldr % 8 != 0 || ldr > kMaxK * 16))
        return QLIN_ERR_BAD_STRIDE;
    if (!(eps > 0.0f) || isinf(eps))
        return QLIN_ERR_BAD_ARGUMENT;   // eps = 0 leaves an all-zero row undefined (0 / 0)
    const RowArgs a{X, ldx, residual, ldr, weight, eps, static_cast<uint8_t *>(Q), ldq, scale, (int)K};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = residual ? launch_rows_qm<OP_RMS, true>(qm, a, M, s)
                                  : launch_rows_qm<OP_RMS, false>(qm, a, M, s);
    return e == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
}

qlin_status silu_and_mul_quant(int qm, int64_t M, int64_t K, const uint16_t *X, int64_t ldx,
                               void *Q, int64_t ldq, float *scale, void *stream)
{
    if (K > kMaxK / 2)
        return QLIN_ERR_BAD_SHAPE;
    qlin_status st = check_args(M, K, qm == Q_GROUP_E4M3, X, ldx, 2 * K, Q, ldq, scale);
    if (st != QLIN_OK || M == 0)
        return st;
    const RowArgs a{X, ldx, nullptr, 0, nullptr, 0.0f, static_cast<uint8_t *>(Q), ldq, scale, (int)K};
    const hipError_t e = launch_rows_qm<OP_SILU, false>(qm, a, M, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" {

qlin_status qlin_rms_norm_dynamic_per_token_quant(qlin_dtype dt, int64_t M, int64_t K,
                                                  const uint16_t *X, int64_t ldx,
                                                  uint16_t *residual, int64_t ldr,
                                                  const uint16_t *weight, float eps, void *Q,
                                                  int64_t ldq, float *scale, void *stream)
{
    if (dt != QLIN_E4M3 && dt != QLIN_INT8)
        return QLIN_ERR_BAD_ARGUMENT;
    return rms_norm_quant(dt == QLIN_INT8 ? rows::Q_TOKEN_INT8 : rows::Q_TOKEN_E4M3, M, K, X, ldx, residual,
                          ldr, weight, eps, Q, ldq, scale, stream);
}

qlin_status qlin_rms_norm_per_block_quant(int64_t M, int64_t K, const uint16_t *X, int64_t ldx,
                                          uint16_t *residual, int64_t ldr,
                                          const uint16_t *weight, float eps, void *Q,
                                          int64_t ldq, float *scale, void *stream)
{
    return rms_norm_quant(rows::Q_GROUP_E4M3, M, K, X, ldx, residual, ldr, weight, eps, Q, ldq, scale,
                          stream);
}

qlin_status qlin_silu_and_mul_dynamic_per_token_quant(qlin_dtype dt, int64_t M, int64_t K,
                                                      const uint16_t *X, int64_t ldx, void *Q,
                                                      int64_t ldq, float *scale, void *stream)
{
    if (dt != QLIN_E4M3 && dt != QLIN_INT8)
        return QLIN_ERR_BAD_ARGUMENT;
    return silu_and_mul_quant(dt == QLIN_INT8 ? rows::Q_TOKEN_INT8 : rows::Q_TOKEN_E4M3, M, K, X, ldx, Q, ldq,
                              scale, stream);
}

qlin_status qlin_silu_and_mul_per_block_quant(int64_t M, int64_t K, const uint16_t *X,
                                              int64_t ldx, void *Q, int64_t ldq, float *scale,
                                              void *stream)
{
    return silu_and_mul_quant(rows::Q_GROUP_E4M3, M, K, X, ldx, Q, ldq, scale, stream);
}

}  // extern "C"
