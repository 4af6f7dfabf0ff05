// Half-step TILE kernel instances for W8A8_INT8; see qlin_tile_h.h.
#include "qlin_tile_h.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_TILE_H_SHAPES(QLIN_TILE_H_INSTANCE, FMT_INT8, FB_INT8, 0),
                                      QLIN_TILE_H_SHAPES(QLIN_TILE_H_INSTANCE, FMT_INT8, FB_INT8, 1)};

const Instance *tile_h_instances_int8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
