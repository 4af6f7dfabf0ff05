// STREAM_TOK kernel instances for one format (fp8); see qlin_stream_tok.h.
#include "qlin_stream_tok.h"

namespace qlin {

static const Instance kInstances[] = {QLIN_STREAM_TOK_SHAPES(QLIN_STREAM_TOK_INSTANCE, FMT_E4M3, FB_FP8)};

const Instance *stream_tok_instances_fp8(int *count)
{
    *count = (int)(sizeof(kInstances) / sizeof(kInstances[0]));
    return kInstances;
}

}  // namespace qlin
