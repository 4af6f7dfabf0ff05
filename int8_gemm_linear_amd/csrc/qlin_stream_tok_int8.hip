// STREAM_TOK kernel instances for one format (int8); see qlin_stream_tok.h.
#include "qlin_stream_tok.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_STREAM_TOK_SHAPES(QLIN_STREAM_TOK_INSTANCE, FMT_INT8, FB_INT8)};

const Instance *stream_tok_instances_int8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
