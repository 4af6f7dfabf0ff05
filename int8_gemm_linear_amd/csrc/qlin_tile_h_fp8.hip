// Half-step TILE kernel instances for FP8_Dynamic; see qlin_tile_h.h.
#include "qlin_tile_h.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_TILE_H_SHAPES(QLIN_TILE_H_INSTANCE, FMT_E4M3, FB_FP8, 0),
                                      QLIN_TILE_H_SHAPES(QLIN_TILE_H_INSTANCE, FMT_E4M3, FB_FP8, 1)};

const Instance *tile_h_instances_fp8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
