// TILE kernel instances for one format (block); see qlin_tile.h.
#include "qlin_tile.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_TILE_SHAPES_BLOCK(QLIN_TILE_INSTANCE, FMT_E4M3, SC_BLOCK, FB_BLOCK, 1)};

const Instance *tile_instances_block(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
