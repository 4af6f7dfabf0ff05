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
// The kernels are the row engine's (qlin_rows.h) with the identity producer:
// one workgroup of 1-8 waves per token row, every 16-byte load of a lane in
// flight before its first use, the row (or 1x128 group) maximum reduced by
// shuffles (and LDS across the row's waves), 8 codes written per piece.
// HBM-bound: 2 bytes read and 1 byte written per value.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin_rows.h"
#include "qlinear.h"

namespace qlin {
namespace {

using namespace rows;

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
    qlin_status st = check_common(M, K, X, ldx, Q, ldq, scale);
    if (st != QLIN_OK || M == 0)
        return st;
    const RowArgs a{X, ldx, nullptr, 0, nullptr, 0.0f, static_cast<uint8_t *>(Q), ldq, scale, (int)K};
    const hipError_t e = launch_rows_qm<OP_QUANT, false>(dt == QLIN_INT8 ? Q_TOKEN_INT8 : Q_TOKEN_E4M3,
                                                          a, M, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
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
    const RowArgs a{X, ldx, nullptr, 0, nullptr, 0.0f, static_cast<uint8_t *>(Q), ldq, scale, (int)K};
    const hipError_t e = launch_rows_qm<OP_QUANT, false>(Q_GROUP_E4M3, a, M,
                                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? QLIN_OK : QLIN_ERR_HIP;
}

}  // extern "C"
