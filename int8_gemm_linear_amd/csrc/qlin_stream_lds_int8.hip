// STREAM_LDS kernel instances for one format (int8); see qlin_stream_lds.h.
#include "qlin_stream_lds.h"

namespace qlin {

static const Instance kInstances[] = {
    QLIN_STREAM_LDS_SHAPES(QLIN_STREAM_LDS_INSTANCE, FMT_INT8, FB_INT8, 0),
    QLIN_STREAM_LDS_SHAPES(QLIN_STREAM_LDS_INSTANCE, FMT_INT8, FB_INT8, 1)};

const Instance *stream_lds_instances_int8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
