// STREAM_LDS kernel instances for one format (fp8); see qlin_stream_lds.h.
#include "qlin_stream_lds.h"

namespace qlin {

static const Instance kInstances[] = {
    QLIN_STREAM_LDS_SHAPES(QLIN_STREAM_LDS_INSTANCE, FMT_E4M3, FB_FP8, 0),
    QLIN_STREAM_LDS_SHAPES(QLIN_STREAM_LDS_INSTANCE, FMT_E4M3, FB_FP8, 1),
    QLIN_STREAM_LDS_WIDE(QLIN_STREAM_LDS_INSTANCE, FMT_E4M3, FB_FP8, 0),
    QLIN_STREAM_LDS_WIDE(QLIN_STREAM_LDS_INSTANCE, FMT_E4M3, FB_FP8, 1)};

const Instance *stream_lds_instances_fp8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
