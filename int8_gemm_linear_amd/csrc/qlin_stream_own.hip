// Wide-row LDS-ring instances (all three formats); see qlin_stream_own.h.
#include "qlin_stream_own.h"

namespace qlin {

static const Instance kInstances[] = {
    QLIN_STREAM_OWN_SHAPES(FMT_E4M3, FB_FP8, SC_TC),
    QLIN_STREAM_OWN_SHAPES(FMT_INT8, FB_INT8, SC_TC),
    QLIN_STREAM_OWN_SHAPES(FMT_E4M3, FB_BLOCK, SC_BLOCK)};

const Instance *stream_own_instances(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
