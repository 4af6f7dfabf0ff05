// STREAM kernel instances for one format (block); see qlin_stream.h.
#include "qlin_stream.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_STREAM_ALL(FMT_E4M3, SC_BLOCK, FB_BLOCK)};

const Instance *stream_instances_block(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
