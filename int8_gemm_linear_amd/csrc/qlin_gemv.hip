// GEMV kernel instances (e4m3 and int8 with token/channel scaling, Block_FP8); see qlin_gemv.h.
#include "qlin_gemv.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_GEMV_SHAPES(QLIN_GEMV_INSTANCE, FMT_E4M3, FB_FP8),
                                      QLIN_GEMV_SHAPES(QLIN_GEMV_INSTANCE, FMT_INT8, FB_INT8),
                                      QLIN_GEMV_BLOCK_SHAPES(QLIN_GEMV_BLOCK_INSTANCE)};

const Instance *gemv_instances(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
