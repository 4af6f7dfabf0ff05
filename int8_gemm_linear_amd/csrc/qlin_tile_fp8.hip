// TILE kernel instances for one format (fp8); see qlin_tile.h.
#include "qlin_tile.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_TILE_SHAPES(QLIN_TILE_INSTANCE, FMT_E4M3, SC_TC, FB_FP8, 0), QLIN_TILE_SHAPES(QLIN_TILE_INSTANCE, FMT_E4M3, SC_TC, FB_FP8, 1)};

const Instance *tile_instances_fp8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
