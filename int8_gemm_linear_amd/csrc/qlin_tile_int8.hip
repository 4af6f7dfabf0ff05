// TILE kernel instances for one format (int8); see qlin_tile.h.
#include "qlin_tile.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_TILE_SHAPES(QLIN_TILE_INSTANCE, FMT_INT8, SC_TC, FB_INT8, 0), QLIN_TILE_SHAPES(QLIN_TILE_INSTANCE, FMT_INT8, SC_TC, FB_INT8, 1)};

const Instance *tile_instances_int8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
