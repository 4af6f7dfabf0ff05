// STREAM kernel instances for one format (int8); see qlin_stream.h.
#include "qlin_stream.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_STREAM_ALL(FMT_INT8, SC_TC, FB_INT8)};

const Instance *stream_instances_int8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
