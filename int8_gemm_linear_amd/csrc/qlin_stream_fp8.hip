// STREAM kernel instances for one format (fp8); see qlin_stream.h.
#include "qlin_stream.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_STREAM_ALL(FMT_E4M3, SC_TC, FB_FP8)};

const Instance *stream_instances_fp8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
