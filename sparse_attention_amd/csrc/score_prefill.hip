// Prefill lightning-indexer score (rows_per_seq query rows share one cache).
// Not yet implemented in this build: dsa_index_score reports
// DSA_ERR_UNSUPPORTED for rows_per_seq > 1.
#include "dsa_internal.h"

namespace dsa {

bool score_prefill_available() { return false; }

hipError_t launch_score_prefill(const void*, const float*, const void*, const int32_t*, int32_t, int32_t, int32_t,
                                int32_t, int32_t, float, bool, float*, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace dsa
