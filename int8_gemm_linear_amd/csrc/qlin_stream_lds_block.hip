// STREAM_LDS kernel instances for Block_FP8 (e4m3, 1x128 / 128x128 scales);
// see qlin_stream_lds.h.
#include "qlin_stream_lds.h"

namespace qlin {

static const Instance kInstances[] = {
    QLIN_STREAM_LDS_SHAPES(QLIN_STREAM_LDS_INSTANCE_BLOCK, FMT_E4M3, FB_BLOCK, 0),
    QLIN_STREAM_LDS_SHAPES(QLIN_STREAM_LDS_INSTANCE_BLOCK, FMT_E4M3, FB_BLOCK, 1),
    QLIN_STREAM_LDS_WIDE(QLIN_STREAM_LDS_INSTANCE_BLOCK, FMT_E4M3, FB_BLOCK, 0),
    QLIN_STREAM_LDS_WIDE(QLIN_STREAM_LDS_INSTANCE_BLOCK, FMT_E4M3, FB_BLOCK, 1)};

const Instance *stream_lds_instances_block(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
